// Latent-cache (MLA) decode with 32 query heads per wave, for many heads.
//
// The 10100.com article on the retirement of vLLM's PagedAttention kernels
// (§2) describes the latent cache: every token stores one compressed row
// [c_kv (512), k_rope (64)], which in the absorbed decode step is the key of
// every query head (all 576 elements) and, through its first 512, the value.
// With many heads per latent row the step is a dense contraction per block,
// and the cost of a kernel that gives each wave 16 heads is operand traffic:
// every wave reads the whole tile again from LDS and rebuilds its transposed
// value operand. Here one workgroup holds all heads of a stream-K share, up to
// four waves of 32 heads each (v_mfma_f32_32x32x16_bf16, 32 tokens by 32 heads
// per product), and a tile is two 16-token cache blocks:
//   S[t][g] = sum_d row_t[d] q[g][d]: A = the tile (32 token rows; lane
//     (i + 32h) reads bytes 16h..16h+15 of chunk 2s of token i, one 16-byte LDS
//     read per step), B = q (this lane's head i, eight d per step, held in
//     registers), 36 steps of 16 d.
//   O[d][g] += sum_t c_kv_t[d] P[g][t]: A = c_kv transposed (32 d rows by 16
//     tokens), read with gfx950's transposing LDS read ds_read_b64_tr_b16, which
//     hands each lane four tokens of one d; B = P straight from the S result
//     registers: the result row order (token 8(v/4) + 4h + v%4 in register v of
//     lane half h) is also the reduction order of the value product when both
//     operands enumerate tokens that way.
// O[d][g] puts head g = lane % 32 in every register of a lane, so each lane's
// softmax state (running max, sum) is its head's; the two lane halves hold the
// two halves of the head's tokens and meet through v_permlane32_swap.
//
// Tiles go from HBM straight to LDS (buffer_load_dwordx4 ... lds, each wave a part
// of every tile) into two 36 KiB buffers used in turn: while one tile is
// computed the copy of the next is in flight, and one barrier per tile
// separates them. (A third buffer with two tiles in flight was slower: its
// three-step loop holds six copies of the tile arithmetic instead of four.)
// The buffers are distinct arrays named at compile time in the code that reads
// and the code that writes them, so the compiler orders reads of one only
// after copies into that one.
//
// Scheduling is the decode kernels' stream-K over (sequence, tile) units: every
// workgroup takes an equal share; a sequence cut by a share boundary writes
// partials that pa_mla_reduce_kernel combines.
//
// With 32-token cache blocks ([num_blocks, 72, 32, 8]) a tile is one block:
// chunk c of its tokens 16 h .. 16 h + 15 is 256 bytes at 512 c + 256 h, and
// goes to the LDS rows of tile half h as above (the copy addresses differ,
// the LDS layout does not).
//
// fp8 latent cache (the pages' scaled fp8 storage, §4, one scale for the row;
// [num_blocks, 36, 16, 16] codes): each wave copies its part of the next tile
// (18 KiB of codes) into an LDS staging buffer, and once the current tile is
// computed converts that same part, exactly, into the bf16 tile layout above
// in the other tile buffer. The barrier that opens the next step then makes
// the converted tile whole for every wave, and the arithmetic is the bf16
// path's; the scale multiplies the logits and the output.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pa_decode.h"
#include "pa_kernels.h"
#include "pa_sched.h"
#include "pa_wave.h"

namespace pa {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

constexpr int kLatent = PA_MLA_LATENT_DIM;                   // value width (c_kv)
constexpr int kWidth = PA_MLA_LATENT_DIM + PA_MLA_ROPE_DIM;  // row width
constexpr int kBS = 16;                                      // tokens per cache block
constexpr int kTileTok = 2 * kBS;                            // tokens per tile
constexpr int kSteps = kWidth / 16;                          // S steps of 16 d
constexpr int kDt = kLatent / 32;                            // 32-d output tiles
constexpr int kBlockBytes = kWidth * kBS * 2;                // 18 KiB
constexpr int kBlockVec = kBlockBytes / 16;
constexpr int kCopySlots = 2 * kBlockBytes / 1024;           // 1 KiB copy instructions per tile
constexpr int kFpBlockBytes = kWidth * kBS;                  // 9 KiB: a block of fp8 codes
constexpr int kFpBlockVec = kFpBlockBytes / 16;
constexpr int kFpSlots = 2 * kFpBlockBytes / 1024;           // 1 KiB copies per fp8 tile
// Fourth word of a raw buffer resource on this GPU family (byte offsets,
// 32-bit data format; out-of-range offsets read zero).
constexpr int kRsrcWord3 = 0x00020000;

// Operand reads issued one group ahead of the products: S steps per group
// (dividing 36) and value-product tiles per group (dividing 16).
#ifndef PA_MLA_WIDE_KG
#define PA_MLA_WIDE_KG 2
#endif
#ifndef PA_MLA_WIDE_KV
#define PA_MLA_WIDE_KV 2
#endif
static_assert(kSteps % PA_MLA_WIDE_KG == 0 && kDt % PA_MLA_WIDE_KV == 0, "groups must divide the steps");

__shared__ u32x4 mla_wide_tile0[2 * kBlockVec];
__shared__ u32x4 mla_wide_tile1[2 * kBlockVec];
// fp8 cache: two 18 KiB staging buffers for the codes of the next tile.
__shared__ u32x4 mla_wide_codes[2 * 2 * kFpBlockVec];
// Per-wave staging of one output tile (16 floats per lane), the only route by
// which the output accumulators reach ordinary registers. The accumulators
// (256 registers per lane: 16 tiles of 32 d x 32 heads) fill the
// accumulation register file; the register allocator keeps them there only
// if nothing but MFMAs defines them and nothing but MFMAs and stores reads
// them, so a rescale and the final normalisation pass each tile through LDS,
// and a rescaled tile re-enters through an MFMA that adds it to a zero
// product.
__shared__ f32x4 mla_wide_stage[4 * 4 * 64];

template <int B>
__device__ __forceinline__ u32x4* tile_buf() {
  static_assert(B == 0 || B == 1, "two tile buffers");
  return B == 0 ? mla_wide_tile0 : mla_wide_tile1;
}
template <int F>
__device__ __forceinline__ u32x4* code_buf() {
  static_assert(F == 0 || F == 1, "two staging buffers");
  return mla_wide_codes + F * (2 * kFpBlockVec);
}

// LDS layout of a cache block: chunk c (eight d of 16 tokens, 256 bytes) keeps
// its 16-byte token granules in a row of its own, token t in slot
// t ^ 4 (c % 4). A transposing read takes four tokens of four consecutive
// chunks in one 16-lane group, which without the swizzle would all fall in the
// same sixteen banks; with it each chunk's tokens sit in their own quarter of
// the row. The 16-byte score reads cover whole rows and stay conflict-free.
__device__ __forceinline__ int slot_of(int c, int t) { return t ^ (4 * (c & 3)); }
// The copy of a 1 KiB piece (chunks 4 p .. 4 p + 3 of a block) writes lane L's
// 16 bytes to slot L % 16 of chunk 4 p + L / 16, so lane L reads the token
// that slot holds: granule L ^ 4 (L / 16) of the piece.
__device__ __forceinline__ int src_granule(int lane) { return lane ^ ((lane >> 4) << 2); }

// Eight fp32 values to the bf16x8 operand (round to nearest even).
__device__ __forceinline__ bf16x8 pack8(const float (&p)[16], int v0) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(p[v0 + e]);
  return r;
}

// Start of a tile: at most N of this wave's copies into LDS are still in
// flight (the next tiles'), its LDS reads have completed, and every wave of the
// workgroup has reached this point; the empty asm statements keep the compiler
// from moving LDS accesses across it. A workgroup fence is not used: its
// release half waits for every copy in flight.
template <int N>
__device__ __forceinline__ void tile_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);   // vmcnt(N) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Element i of read-only per-call metadata (a block table, the sequence
// lengths) at an index that is the same in every lane, as a scalar load: the
// index is taken from the first lane, and the constant address space lets the
// compiler read through the scalar cache.
__device__ __forceinline__ int ld_uniform(const int32_t* p, int64_t i) {
  const uint64_t u = (uint64_t)i;
  const int64_t j = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(u >> 32)) << 32) |
                              (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u));
  return ((const __attribute__((address_space(4))) int32_t*)p)[j];
}

// Max / sum of this lane and lane l ^ 32 (v_permlane32_swap on two copies).
template <typename Op>
__device__ __forceinline__ float pair_reduce(float v, Op op) {
  const unsigned b = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <bool FP8>
struct WideWave {
  bf16x8 q[kSteps];   // B operand of S: head i, d = 16 s + 8 h + e
  f32x16 o[kDt];      // O[32 dt + 8(v/4) + 4h + v%4][head i]
  float m, lsum, c;
  float vs;           // fp8: the cache's scale (output multiplier)
  int lane, half, wave;
  bool active;        // this lane's head exists
  uint32_t k_off[2];  // byte offset of this lane's S operand in a tile buffer, even / odd steps (step 0 / 1 less 512 B)
  uint32_t v_off[2];  // byte offsets of this lane's transposing reads (d-tile 0, block 0; tokens 0-7, 8-15)

  __device__ __forceinline__ void init(const MlaArgs& a, int hg) {
    lane = threadIdx.x & 63;
    half = lane >> 5;
    wave = hg;
    const int i = lane & 31;
    active = hg * 32 + i < a.d.num_heads;
    vs = (FP8 && a.d.k_scale) ? *a.d.k_scale : 1.f;
    c = a.d.scale * kLog2e * (FP8 ? vs : 1.f);
    // S operand: token i (block i / 16), chunk 2 s + h, in its swizzled slot.
    const int t = i & 15;
    k_off[0] = (uint32_t)((i >> 4) * kBlockBytes + half * 256 + slot_of(half, t) * 16);
    k_off[1] = (uint32_t)((i >> 4) * kBlockBytes + half * 256 + slot_of(2 + half, t) * 16);
    // Transposing read: lane 4u + w of 16-lane group G reads the 8 bytes of
    // token 4 (G / 2) + u (+ 8 for the second half of the token order) at
    // d = 16 (G % 2) + 4 w (+ 32 dt); lane j of the group then receives that
    // token range's four values of d = 16 (G % 2) + j.
    const int G = lane >> 4, mm = lane & 15, u = mm >> 2, w = mm & 3;
    const int vc = 2 * (G & 1) + (w >> 1);
    v_off[0] = (uint32_t)(vc * 256 + slot_of(vc, 4 * (G >> 1) + u) * 16 + 8 * (w & 1));
    v_off[1] = (uint32_t)(vc * 256 + slot_of(vc, 8 + 4 * (G >> 1) + u) * 16 + 8 * (w & 1));
  }

  __device__ __forceinline__ void load_q(const MlaArgs& a, int seq, int hg) {
    const int h = hg * 32 + (active ? (lane & 31) : 0);
    const __bf16* qh = reinterpret_cast<const __bf16*>(a.d.query) + ((int64_t)seq * a.d.num_heads + h) * kWidth;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      u32x4 w = {0, 0, 0, 0};
      if (active) w = *reinterpret_cast<const u32x4*>(qh + 16 * s + 8 * half);
      q[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // An accumulation tile in ordinary registers, through this wave's LDS
  // staging area (the barrier keeps the compiler from forwarding the store).
  __device__ __forceinline__ f32x16 through_lds(const f32x16& x) const {
    f32x4* t = mla_wide_stage + wave * 256 + lane;
    t[0] = f32x4{x[0], x[1], x[2], x[3]};
    t[64] = f32x4{x[4], x[5], x[6], x[7]};
    t[128] = f32x4{x[8], x[9], x[10], x[11]};
    t[192] = f32x4{x[12], x[13], x[14], x[15]};
    asm volatile("" ::: "memory");
    const f32x4 a0 = t[0], a1 = t[64], a2 = t[128], a3 = t[192];
    asm volatile("" ::: "memory");
    return f32x16{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3],
                  a2[0], a2[1], a2[2], a2[3], a3[0], a3[1], a3[2], a3[3]};
  }
  // x as an accumulation tile: the MFMA adds it to a zero product.
  __device__ __forceinline__ static f32x16 to_acc(const f32x16& x) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf16x8{}, bf16x8{}, x, 0, 0, 0);
  }

  __device__ __forceinline__ void reset() {
    m = kNegInf;
    lsum = 0.f;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) o[dt] = to_acc(f32x16{});
  }

  // Multiplies every accumulation tile by alpha (rare: the running max rose).
  __device__ __forceinline__ void rescale(float alpha) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) o[dt] = to_acc(through_lds(o[dt]) * alpha);
  }

  // One tile from buffer B: nvalid (1..32) valid tokens. Tokens past nvalid
  // get logit -inf by select and their value elements are zeroed by select
  // (stale slots may hold NaN, and 0 * NaN would poison the products).
  //
  // Both products are software-pipelined by hand: the operand reads of group
  // g + 1 are issued before the products of group g, and a scheduling barrier
  // after each group keeps the compiler from hoisting further reads, whose
  // registers the queries and accumulators leave no room for.
  template <int B, bool PARTIAL>
  __device__ __forceinline__ void compute(int nvalid) {
    const char* base = reinterpret_cast<const char*>(tile_buf<B>());
    // Token 8(v/4) + 4h + v%4 of register v (16 b + 8(e/4) + 4h + e%4 of
    // element e of block b's value operand) is valid when its constant part is
    // below thr.
    const int thr = nvalid - 4 * half;
    const bool two = !PARTIAL || nvalid > kBS;   // the tile's second block holds tokens

    // S = K q^T, 36 steps in groups of kG.
    constexpr int kG = PA_MLA_WIDE_KG, kGroups = kSteps / kG;
    f32x16 s0 = {};
    bf16x8 ka[2][kG];
    auto read_k = [&](int g, bf16x8 (&k)[kG]) {
#pragma unroll
      for (int j = 0; j < kG; ++j)
        k[j] = *reinterpret_cast<const bf16x8*>(base + k_off[(kG * g + j) & 1] + 512 * (kG * g + j));
    };
    read_k(0, ka[0]);
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      if (g + 1 < kGroups) read_k(g + 1, ka[(g + 1) & 1]);
#pragma unroll
      for (int j = 0; j < kG; ++j)
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[g & 1][j], q[kG * g + j], s0, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }

    float z[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      z[v] = s0[v] * c;
      if constexpr (PARTIAL) {
        if (8 * (v >> 2) + (v & 3) >= thr) z[v] = kNegInf;
      }
    }
    float mx = z[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, z[v]);
    mx = pair_reduce(mx, [](float x, float y) { return fmaxf(x, y); });
    if (wave_any(mx > m + kRescaleSlack)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2(m - m_new);
      // A head whose max is still -inf has a zero sum and zero accumulators:
      // the first tile of a segment rescales nothing.
      const bool live = wave_any(m != kNegInf && mx > m + kRescaleSlack);
      m = m_new;
      lsum *= alpha;
      if (live) rescale(alpha);
    }
    float p[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) p[v] = fast_exp2(z[v] - m);
#pragma unroll
    for (int v = 0; v < 16; v += 4) lsum += (p[v] + p[v + 1]) + (p[v + 2] + p[v + 3]);
    const bf16x8 pb[2] = {pack8(p, 0), pack8(p, 8)};

    // O += c_kv^T P per block, 16 d-tiles in groups of kV.
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    constexpr int kV = PA_MLA_WIDE_KV, kVGroups = kDt / kV;
    s16x8 va[2][kV];
    auto read_v = [&](int b, int g, s16x8 (&v)[kV]) {
#pragma unroll
      for (int j = 0; j < kV; ++j) {
        const uint32_t off = (uint32_t)((kV * g + j) * 1024 + b * kBlockBytes);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + v_off[0] + off));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + v_off[1] + off));
        v[j] = s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    };
    auto value_products = [&](int b) {
      read_v(b, 0, va[0]);
#pragma unroll
      for (int g = 0; g < kVGroups; ++g) {
        if (g + 1 < kVGroups) read_v(b, g + 1, va[(g + 1) & 1]);
#pragma unroll
        for (int j = 0; j < kV; ++j) {
          s16x8 w = va[g & 1][j];
          if constexpr (PARTIAL) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (16 * b + 8 * (e >> 2) + (e & 3) >= thr) w[e] = 0;
          }
          const int dt = kV * g + j;
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pb[b], o[dt], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    value_products(0);
    if (two) value_products(1);
  }

  __device__ __forceinline__ void finish() { lsum = pair_reduce(lsum, [](float x, float y) { return x + y; }); }

  // o / lsum into rows [row_base + h row_stride] for the nh heads of this
  // wave (nh <= 32). Register v of tile dt is d = 32 dt + 8 (v / 4) + 4 h +
  // v % 4 of this lane's head; each tile passes through the wave's LDS
  // staging and comes back transposed, so that lane L holds d = 32 dt +
  // 4 (L % 8) .. + 3 of head 8 k + L / 8, and one store instruction writes 128
  // contiguous bytes (64 for bf16 rows) of each of eight rows instead of
  // 32-byte pieces of 32 rows. The accumulators go to LDS as they are (only
  // MFMAs and stores touch them); the scale is applied after the transpose.
  template <typename T>
  __device__ __forceinline__ void store_rows(T* row_base, int64_t row_stride, int nh) const {
    f32x4* t = mla_wide_stage + wave * 256;
    int c = lane & 7, r = lane >> 3;
    // Opaque to the optimiser, so that the addressing below is formed here
    // (a rare path) rather than hoisted into registers the loop needs.
    asm volatile("" : "+v"(c), "+v"(r));
    const int src = (c >> 1) * 64 + (c & 1) * 32 + r;   // slot of chunk c of head r
    const float f = (FP8 ? vs : 1.f) / lsum;
    float fk[4];   // 1 / lsum of head 8 k + r
#pragma unroll
    for (int k = 0; k < 4; ++k)
      fk[k] = __int_as_float(__builtin_amdgcn_ds_bpermute((8 * k + r) * 4, __float_as_int(f)));
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) {
      const f32x16& x = o[dt];
      t[lane] = f32x4{x[0], x[1], x[2], x[3]};
      t[64 + lane] = f32x4{x[4], x[5], x[6], x[7]};
      t[128 + lane] = f32x4{x[8], x[9], x[10], x[11]};
      t[192 + lane] = f32x4{x[12], x[13], x[14], x[15]};
      asm volatile("" ::: "memory");
      f32x4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = t[src + 8 * k];
      asm volatile("" ::: "memory");
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (8 * k + r < nh) store4(row_base + (int64_t)(8 * k + r) * row_stride + 32 * dt + 4 * c, v[k] * fk[k]);
    }
  }
};

// Staging cursor of a share: tile st of sequence sseq (L tokens) is the next
// to copy; its segment of the share ends before tile st1; sleft tiles of the
// share follow that segment. Sequence lengths and table entries are read
// through the scalar cache (uniform loads; waiting for them never waits for
// copies). Each buffer's tile has a descriptor: its sequence, and its token
// count (1..32) with the kLast / kFirstOfSeq / kLastOfSeq bits.
struct ShareCursor {
  static constexpr int kLast = 64, kFirstOfSeq = 128, kLastOfSeq = 256;
  const DecodeArgs& d;
  int S;
  unsigned top;
  int one;            // 1: 32-token cache blocks, a tile is one block
  int sseq, st, L, st1, sleft, sflags;
  bool sdone;
  int dseq[3], dinf[3];
  // The table entries of the cursor's tile, read one step ahead (fetch), so
  // that their latency passes under a step's work instead of holding up its
  // copies.
  unsigned np0, np1;

  __device__ __forceinline__ ShareCursor(const DecodeArgs& args, int seq, int tile, int units)
      : d(args), S(args.num_seqs), top((unsigned)(args.num_blocks - 1)), one(args.block_size == 32 ? 1 : 0) {
    sseq = seq;
    st = tile;
    L = clamp_len(ld_uniform(d.seq_lens, seq), d.max_seq_len);
    st1 = min(blocks_of<kTileTok>(L), tile + units);
    sleft = units - (st1 - tile);
    sflags = (tile == 0 ? kFirstOfSeq : 0) | (st1 == blocks_of<kTileTok>(L) ? kLastOfSeq : 0);
    sdone = false;
    np0 = np1 = 0;
  }

  __device__ __forceinline__ void fetch() {
    if (one) {
      np0 = np1 = (unsigned)ld_uniform(d.block_tables, (int64_t)sseq * d.max_blocks_per_seq + st);
      return;
    }
    const int64_t e = (int64_t)sseq * d.max_blocks_per_seq + 2 * st;
    np0 = (unsigned)ld_uniform(d.block_tables, e);
    np1 = (unsigned)ld_uniform(d.block_tables, e + (2 * st + 1 < blocks_of<kBS>(L) ? 1 : 0));
  }

  // Takes the cursor's tile for buffer B: records its descriptor, sets its
  // physical blocks (p1 = p0 when it has one block) and advances the cursor;
  // false when the share has no tile left.
  template <int B>
  __device__ __forceinline__ bool take(unsigned& p0, unsigned& p1) {
    if (sdone) return false;
    p0 = np0 < top ? np0 : top;
    p1 = np1 < top ? np1 : top;
    dseq[B] = sseq;
    dinf[B] = min(kTileTok, L - st * kTileTok);
    if (st + 1 < st1) {
      ++st;
    } else {
      dinf[B] |= kLast | sflags;
      int s = sseq;
      if (sleft > 0) {
        do {
          ++s;
        } while (s < S && clamp_len(ld_uniform(d.seq_lens, s), d.max_seq_len) == 0);
      }
      if (sleft > 0 && s < S) {   // s >= S only with inputs that disagree with the tile count
        sseq = s;
        L = clamp_len(ld_uniform(d.seq_lens, s), d.max_seq_len);
        st = 0;
        st1 = min(blocks_of<kTileTok>(L), sleft);
        sleft -= st1;
        sflags = kFirstOfSeq | (st1 == blocks_of<kTileTok>(L) ? kLastOfSeq : 0);
      } else {
        sdone = true;
      }
    }
    return true;
  }
};

// A workgroup's share: tiles [u0, u0 + units) in (sequence, tile) order, one
// pipeline across the sequences it spans. Wave WAVE of W copies slots
// [36 WAVE / W, 36 (WAVE + 1) / W) of every tile (slot s: 1 KiB s % 18 of the
// tile's block s / 18; a tile with one block copies that block twice, so that
// every tile costs each wave the same number of copy instructions).
//
// Two cursors walk the share: the staging cursor, one tile ahead, and the
// compute cursor. Step k (tile k of the share, in buffer k % 2) opens with a
// barrier behind which every wave's copies of tile k have landed and every
// wave is done with tile k - 1; it then starts the copy of tile k + 1 into
// tile k - 1's buffer and computes tile k.
template <int W, int WAVE>
__device__ __forceinline__ void wide_share(const MlaArgs& a, int share, int seq, int tile, int units) {
  constexpr int kS0 = kCopySlots * WAVE / W, kS1 = kCopySlots * (WAVE + 1) / W;
  const DecodeArgs& d = a.d;
  const int hg = WAVE;

  WideWave<false> wv;
  wv.init(a, hg);
  const int lane = wv.lane;
  const char* cache = reinterpret_cast<const char*>(d.key_cache);

  ShareCursor cur(d, seq, tile, units);
  cur.fetch();
  constexpr int kLast = ShareCursor::kLast, kFirstOfSeq = ShareCursor::kFirstOfSeq,
                kLastOfSeq = ShareCursor::kLastOfSeq;
  // Copy slot s of a tile: LDS tile half blk = s / 18, piece part = s % 18.
  // Lane L fills LDS slot L of the piece with granule g = src_granule(L):
  // chunk 4 part + g / 16 of token g % 16 of the half. In the cache that is
  // byte voff(s) of block p_blk (16-token blocks) or of the tile's one block
  // (32-token blocks: chunks 512 bytes apart, the half 256 bytes in).
  const int one = cur.one;
  const int blk_bytes = kBlockBytes << one;
  const int lane_off = (src_granule(lane) >> 4) * (256 << one) + (src_granule(lane) & 15) * 16;
  auto voff = [&](int s) {
    const int blk = s / (kCopySlots / 2), part = s % (kCopySlots / 2);
    return part * (1024 << one) + blk * 256 * one + lane_off;
  };
  auto slot_src = [&](int s, unsigned p0, unsigned p1) {
    return cache + (int64_t)(s / (kCopySlots / 2) ? p1 : p0) * blk_bytes + voff(s);
  };
  auto slot_dst = [&](auto bsel, int s) {
    constexpr int B = decltype(bsel)::value;
    return tile_buf<B>() + (s / (kCopySlots / 2)) * kBlockVec + (s % (kCopySlots / 2)) * 64;
  };
  // Copies the next tile into buffer B straight from HBM to LDS, with the
  // buffer form of the LDS copy (one resource per cache block, offsets within
  // its 18 KiB). The global form is a flat-encoded instruction that may touch
  // LDS, and while one is outstanding the compiler cannot count LDS reads
  // separately: every wait for an operand read would wait for all of them,
  // and the reads issued ahead of the products would buy nothing.
  auto stage = [&](auto bsel) -> bool {
    unsigned p0, p1;
    if (!cur.template take<decltype(bsel)::value>(p0, p1)) return false;
    const __amdgpu_buffer_rsrc_t r0 =
        __builtin_amdgcn_make_buffer_rsrc((void*)(cache + (int64_t)p0 * blk_bytes), 0, blk_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t r1 =
        __builtin_amdgcn_make_buffer_rsrc((void*)(cache + (int64_t)p1 * blk_bytes), 0, blk_bytes, kRsrcWord3);
#pragma unroll
    for (int s = kS0; s < kS1; ++s) {
      const int blk = s / (kCopySlots / 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(blk ? r1 : r0, (__attribute__((address_space(3))) void*)slot_dst(bsel, s),
                                               16, voff(s), 0, 0, 2 /* nt */);
    }
    return true;
  };
  // The same through registers, for the tile copied before the loop: the
  // compiler's bookkeeping of copies into LDS, merged at the loop head, would
  // otherwise make one of the loop's steps wait for every copy in flight.
  auto stage_through_registers = [&](auto bsel) -> bool {
    unsigned p0, p1;
    if (!cur.template take<decltype(bsel)::value>(p0, p1)) return false;
#pragma unroll
    for (int s = kS0; s < kS1; ++s)
      slot_dst(bsel, s)[lane] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(slot_src(s, p0, p1)));
    return true;
  };

  // The first tile and the queries are waited for before the loop: the loop
  // is then entered with nothing outstanding, as it is left at a segment end,
  // and the compiler's count of outstanding loads stays exact inside it.
  stage_through_registers(std::integral_constant<int, 0>{});
  cur.fetch();
  wv.load_q(a, seq, hg);
  wv.reset();
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // Computes the tile in buffer B; false once the share is done.
  auto step = [&](auto bsel) -> bool {
    constexpr int B = decltype(bsel)::value;
    // Nothing but this wave's copies of the current tile is outstanding here.
    tile_barrier<0>();
    const bool has_next = stage(std::integral_constant<int, 1 - B>{});
    const int inf = cur.dinf[B];
    const int nvalid = inf & 63;
    if (nvalid < kTileTok)
      wv.template compute<B, true>(nvalid);
    else
      wv.template compute<B, false>(kTileTok);
    // The cursor always points at a tile of the share (the last one once it
    // is done); its entries are read here, after the tile's LDS reads, so that
    // no scalar load is outstanding while they are waited for.
    cur.fetch();
    if (!(inf & kLast)) return true;
    // The segment ends with this tile: the next segment's queries are loaded
    // while this one's rows are written.
    wv.finish();
    const float m_end = wv.m, l_end = wv.lsum;
    if (has_next) wv.load_q(a, cur.dseq[1 - B], hg);
    const int cseq = cur.dseq[B];
    const int nh = min(32, d.num_heads - hg * 32);
    if ((inf & kFirstOfSeq) && (inf & kLastOfSeq)) {
      wv.store_rows(reinterpret_cast<__bf16*>(d.out) + ((int64_t)cseq * d.num_heads + hg * 32) * kLatent, kLatent, nh);
    } else {
      const int64_t row = (int64_t)(cseq + share) * a.hpad + hg * 32;   // slot (seq + share)
      wv.store_rows(reinterpret_cast<__bf16*>(d.seg_out) + row * kLatent, kLatent, nh);
      float* mbase = d.seg_max;
      float* sbase = d.seg_sum;
      asm volatile("" : "+s"(mbase), "+s"(sbase));   // kept in scalar registers
      float* const mrow = mbase + row;
      float* const srow = sbase + row;
      if (wv.active && wv.half == 0) {
        mrow[lane & 31] = m_end;
        srow[lane & 31] = l_end;
      }
    }
    if (hg == 0 && lane == 0) {
      if (inf & kFirstOfSeq) d.seg_meta[2 * cseq] = share;
      if (inf & kLastOfSeq) d.seg_meta[2 * cseq + 1] = share;
    }
    // Wait for the stores and the query loads here (with the copies in
    // flight; a segment end is rare): left outstanding across the loop, they
    // would keep the compiler from counting which loads have completed, and
    // every later wait would become a wait for all of them.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (!has_next) return false;
    wv.reset();
    return true;
  };
  while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
  }
  // Nothing may be left in flight into LDS when the workgroup ends.
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Converts this lane's 16-byte granules of e4m3 codes, slots S0 .. S0 + N - 1
// of a tile of codes (slot s: granule `lane` of 1 KiB s % 9 of block s / 9,
// i.e. 16 d of token lane % 16, chunk c16 = 4 (s % 9) + lane / 16), into the
// bf16 layout of tile buffer T: chunks c = 2 c16 + h (h = 0, 1) of that token
// in their swizzled slots, byte 2048 (s % 9) + 512 (lane / 16) + 256 h +
// 16 slot_of(c, token) of the block, where c % 4 = (2 (lane / 16) + h) % 4.
// Exact: every e4m3 value is a bf16 value. The two lane-dependent offsets are
// formed here, so that they are not held in registers across the loop.
template <int T, int S0, int N>
__device__ __forceinline__ void convert_granules(const u32x4 (&raw)[N], int lane) {
  int t = lane & 15, q = lane >> 4;
  asm volatile("" : "+v"(t), "+v"(q));
  const uint32_t a0 = (uint32_t)(q * 512 + (t ^ (4 * ((2 * q) & 3))) * 16);
  const uint32_t a1 = (uint32_t)(q * 512 + 256 + (t ^ (4 * ((2 * q + 1) & 3))) * 16);
  char* const tb = reinterpret_cast<char*>(tile_buf<T>());
#pragma unroll
  for (int i = 0; i < N; ++i) {
    constexpr int kHalf = kFpSlots / 2;
    const int off = ((S0 + i) / kHalf) * kBlockBytes + ((S0 + i) % kHalf) * 2048;
    const u32x4 w0 = {fp8x2_to_bf16x2<false>(raw[i][0]), fp8x2_to_bf16x2<true>(raw[i][0]),
                      fp8x2_to_bf16x2<false>(raw[i][1]), fp8x2_to_bf16x2<true>(raw[i][1])};
    const u32x4 w1 = {fp8x2_to_bf16x2<false>(raw[i][2]), fp8x2_to_bf16x2<true>(raw[i][2]),
                      fp8x2_to_bf16x2<false>(raw[i][3]), fp8x2_to_bf16x2<true>(raw[i][3])};
    *reinterpret_cast<u32x4*>(tb + off + a0) = w0;
    *reinterpret_cast<u32x4*>(tb + off + a1) = w1;
  }
}

// Slots [S0, S1) of the tile of codes in staging buffer F into tile buffer T,
// six at a time (reads issued together, then converted).
template <int F, int T, int S0, int S1>
__device__ __forceinline__ void convert_staged(int lane) {
  if constexpr (S0 < S1) {
    constexpr int kN = S1 - S0 < 6 ? S1 - S0 : 6;
    constexpr int kHalf = kFpSlots / 2;
    u32x4 raw[kN];
#pragma unroll
    for (int i = 0; i < kN; ++i)
      raw[i] = code_buf<F>()[((S0 + i) / kHalf) * kFpBlockVec + ((S0 + i) % kHalf) * 64 + lane];
    convert_granules<T, S0, kN>(raw, lane);
    convert_staged<F, T, S0 + kN, S1>(lane);
  }
}

// The share loop with an fp8 cache. Wave WAVE of W copies slots
// [18 WAVE / W, 18 (WAVE + 1) / W) of every tile of codes (slot s: 1 KiB s % 9
// of block s / 9, lane L's 16 bytes at granule L) and converts the same
// slots, so the codes it reads are its own copies and only the converted
// tile needs the barrier. Step k (tile k, tile buffer k % 2) opens with the
// barrier behind which tile k is converted by every wave and every wave is
// done with tile k - 1; it copies tile k + 1's codes into staging buffer
// (k + 1) % 2, computes tile k, then waits for its copies and converts them
// into tile buffer (k + 1) % 2. One tile's codes are in flight while one is
// computed.
template <int W, int WAVE>
__device__ __forceinline__ void wide_share_fp8(const MlaArgs& a, int share, int seq, int tile, int units) {
  constexpr int kS0 = kFpSlots * WAVE / W, kS1 = kFpSlots * (WAVE + 1) / W;
  const DecodeArgs& d = a.d;
  const int hg = WAVE;

  WideWave<true> wv;
  wv.init(a, hg);
  const int lane = wv.lane;
  const char* cache = reinterpret_cast<const char*>(d.key_cache);

  ShareCursor cur(d, seq, tile, units);
  cur.fetch();
  constexpr int kLast = ShareCursor::kLast, kFirstOfSeq = ShareCursor::kFirstOfSeq,
                kLastOfSeq = ShareCursor::kLastOfSeq;

  // Copy slot s: lane L's 16 bytes are chunk 4 (s % 9) + L / 16 of token
  // L % 16 of tile half s / 9, at byte voff(s) of its cache block (as for
  // the bf16 copies, with 16-byte chunks and no swizzle).
  const int one = cur.one;
  const int blk_bytes = kFpBlockBytes << one;
  const int lane_off = (lane >> 4) * (256 << one) + (lane & 15) * 16;
  auto voff = [&](int s) {
    const int blk = s / (kFpSlots / 2), part = s % (kFpSlots / 2);
    return part * (1024 << one) + blk * 256 * one + lane_off;
  };

  // Tile 0: codes through registers (then staging buffer 1, not in use yet),
  // converted into tile buffer 0.
  {
    unsigned p0 = 0, p1 = 0;
    cur.template take<0>(p0, p1);   // a share holds at least one tile
#pragma unroll
    for (int s = kS0; s < kS1; ++s) {
      const int blk = s / (kFpSlots / 2), part = s % (kFpSlots / 2);
      code_buf<1>()[blk * kFpBlockVec + part * 64 + lane] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(cache + (int64_t)(blk ? p1 : p0) * blk_bytes + voff(s)));
    }
    convert_staged<1, 0, kS0, kS1>(lane);
  }
  cur.fetch();
  wv.load_q(a, seq, hg);
  wv.reset();
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // Copies the codes of the cursor's next tile into staging buffer F (its
  // descriptor in slot F); false when the share has no tile left.
  auto stage = [&](auto fsel) -> bool {
    constexpr int F = decltype(fsel)::value;
    unsigned p0, p1;
    if (!cur.template take<F>(p0, p1)) return false;
    const __amdgpu_buffer_rsrc_t r0 =
        __builtin_amdgcn_make_buffer_rsrc((void*)(cache + (int64_t)p0 * blk_bytes), 0, blk_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t r1 =
        __builtin_amdgcn_make_buffer_rsrc((void*)(cache + (int64_t)p1 * blk_bytes), 0, blk_bytes, kRsrcWord3);
#pragma unroll
    for (int s = kS0; s < kS1; ++s) {
      const int blk = s / (kFpSlots / 2), part = s % (kFpSlots / 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          blk ? r1 : r0, (__attribute__((address_space(3))) void*)(code_buf<F>() + blk * kFpBlockVec + part * 64), 16,
          voff(s), 0, 0, 2 /* nt */);
    }
    return true;
  };

  // Computes the tile in tile buffer B; false once the share is done.
  auto step = [&](auto bsel) -> bool {
    constexpr int B = decltype(bsel)::value, N = 1 - B;
    tile_barrier<0>();
    const bool has_next = stage(std::integral_constant<int, N>{});
    const int inf = cur.dinf[B];
    const int nvalid = inf & 63;
    if (nvalid < kTileTok)
      wv.template compute<B, true>(nvalid);
    else
      wv.template compute<B, false>(kTileTok);
    if (has_next) {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies of the next tile
      convert_staged<N, N, kS0, kS1>(lane);
    }
    cur.fetch();
    if (!(inf & kLast)) return true;
    wv.finish();
    const float m_end = wv.m, l_end = wv.lsum;
    if (has_next) wv.load_q(a, cur.dseq[N], hg);
    const int cseq = cur.dseq[B];
    const int nh = min(32, d.num_heads - hg * 32);
    if ((inf & kFirstOfSeq) && (inf & kLastOfSeq)) {
      wv.store_rows(reinterpret_cast<__bf16*>(d.out) + ((int64_t)cseq * d.num_heads + hg * 32) * kLatent, kLatent, nh);
    } else {
      const int64_t row = (int64_t)(cseq + share) * a.hpad + hg * 32;   // slot (seq + share)
      wv.store_rows(reinterpret_cast<__bf16*>(d.seg_out) + row * kLatent, kLatent, nh);
      float* mbase = d.seg_max;
      float* sbase = d.seg_sum;
      asm volatile("" : "+s"(mbase), "+s"(sbase));   // kept in scalar registers
      float* const mrow = mbase + row;
      float* const srow = sbase + row;
      if (wv.active && wv.half == 0) {
        mrow[lane & 31] = m_end;
        srow[lane & 31] = l_end;
      }
    }
    if (hg == 0 && lane == 0) {
      if (inf & kFirstOfSeq) d.seg_meta[2 * cseq] = share;
      if (inf & kLastOfSeq) d.seg_meta[2 * cseq + 1] = share;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (!has_next) return false;
    wv.reset();
    return true;
  };
  while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Grid: one workgroup of W waves (32 heads each) per stream-K share.
template <int W, bool FP8>
__global__ void __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(1, 1)))
pa_mla_wide_kernel(const MlaArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int share = blockIdx.x;
  int bsum = 0;
  const int T = count_blocks<kTileTok>(a.d, lane, bsum);
  if (T == 0) return;
  const int64_t U = ((int64_t)T + a.shares - 1) / a.shares;
  const int64_t u0 = (int64_t)share * U;
  const int64_t u1 = min((int64_t)T, u0 + U);
  if (u0 >= u1) return;   // uniform over the workgroup
  int seq = 0, tile = 0;
  locate_block<kTileTok>(a.d, lane, (int)u0, bsum, seq, tile);
  // Each wave runs its own instantiation (its copy slots); all meet the same barriers.
  const int n = (int)(u1 - u0);
  static_assert(W == 3 || W == 4, "three or four 32-head waves");
  if constexpr (FP8) {
    switch (wave) {
      case 0: wide_share_fp8<W, 0>(a, share, seq, tile, n); break;
      case 1: wide_share_fp8<W, 1>(a, share, seq, tile, n); break;
      case 2: wide_share_fp8<W, 2>(a, share, seq, tile, n); break;
      default: if constexpr (W > 3) wide_share_fp8<W, 3 % W>(a, share, seq, tile, n); break;
    }
  } else {
    switch (wave) {
      case 0: wide_share<W, 0>(a, share, seq, tile, n); break;
      case 1: wide_share<W, 1>(a, share, seq, tile, n); break;
      case 2: wide_share<W, 2>(a, share, seq, tile, n); break;
      default: if constexpr (W > 3) wide_share<W, 3 % W>(a, share, seq, tile, n); break;
    }
  }
}

}  // namespace

hipError_t launch_mla_wide(const MlaArgs& a, hipStream_t stream) {
  const dim3 grid(a.shares);
  switch (a.waves_per_wg * 2 + (a.fp8 ? 1 : 0)) {
    // 65 to 128 heads: three or four waves (the plan runs fewer heads on the
    // 16-heads-per-wave kernel).
    case 6: hipLaunchKernelGGL((pa_mla_wide_kernel<3, false>), grid, dim3(192), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((pa_mla_wide_kernel<4, false>), grid, dim3(256), 0, stream, a); break;
    case 7: hipLaunchKernelGGL((pa_mla_wide_kernel<3, true>), grid, dim3(192), 0, stream, a); break;
    case 9: hipLaunchKernelGGL((pa_mla_wide_kernel<4, true>), grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
