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
// Tiles go from HBM straight to LDS (global_load_lds_dwordx4, each wave a part
// of every tile) into two 36 KiB buffers used in turn; the next tile's copy is
// in flight while the current one is computed, and one barrier per tile
// separates them. The two buffers are distinct arrays named at compile time in
// the code that reads and the code that writes them, so the compiler orders
// reads of one only after copies into that one.
//
// Scheduling is the decode kernels' stream-K over (sequence, tile) units: every
// workgroup takes an equal share; a sequence cut by a share boundary writes
// partials that pa_mla_reduce_kernel combines.

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
  return B == 0 ? mla_wide_tile0 : mla_wide_tile1;
}

// Eight fp32 values to the bf16x8 operand (round to nearest even).
__device__ __forceinline__ bf16x8 pack8(const float (&p)[16], int v0) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(p[v0 + e]);
  return r;
}

// Start of a tile: this wave's copies of the tile have landed (vmcnt(0)), its
// reads of the previous tile are complete (release), every wave of the
// workgroup has reached this point (barrier), and no read of the new tile is
// moved above it (acquire). After it the tile is whole in LDS and the other
// buffer is free for the next copy.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Max / sum of this lane and lane l ^ 32 (v_permlane32_swap on two copies).
template <typename Op>
__device__ __forceinline__ float pair_reduce(float v, Op op) {
  const unsigned b = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

struct WideWave {
  bf16x8 q[kSteps];   // B operand of S: head i, d = 16 s + 8 h + e
  f32x16 o[kDt];      // O[32 dt + 8(v/4) + 4h + v%4][head i]
  float m, lsum, c;
  int lane, half, wave;
  bool active;        // this lane's head exists
  uint32_t k_off;     // byte offset of this lane's S operand (step 0) in a tile buffer
  uint32_t v_off;     // byte offset of this lane's transposing read (d-tile 0, block 0, first half)

  __device__ __forceinline__ void init(const MlaArgs& a, int hg) {
    lane = threadIdx.x & 63;
    half = lane >> 5;
    wave = hg;
    const int i = lane & 31;
    active = hg * 32 + i < a.d.num_heads;
    c = a.d.scale * kLog2e;
    // S operand: token i (block i / 16, slot i % 16), chunk 2 s + h.
    k_off = (uint32_t)((i >> 4) * kBlockBytes + (half * 16 + (i & 15)) * 16);
    // Transposing read: lane 4u + w of 16-lane group G reads the 8 bytes of
    // token 4 (G / 2) + u (+ 8 for the second half of the token order) at
    // d = 16 (G % 2) + 4 w (+ 32 dt); lane j of the group then receives that
    // token range's four values of d = 16 (G % 2) + j.
    const int G = lane >> 4, mm = lane & 15, u = mm >> 2, w = mm & 3;
    v_off = (uint32_t)((2 * (G & 1) + (w >> 1)) * 256 + (4 * (G >> 1) + u) * 16 + 8 * (w & 1));
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
      for (int j = 0; j < kG; ++j) k[j] = *reinterpret_cast<const bf16x8*>(base + k_off + 512 * (kG * g + j));
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
      m = m_new;
      lsum *= alpha;
      rescale(alpha);
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
        const uint32_t off = v_off + (uint32_t)((kV * g + j) * 1024 + b * kBlockBytes);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off + 128));
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

  // o / lsum for this lane's head: register v of tile dt is d = 32 dt +
  // 8 (v / 4) + 4 h + v % 4, four consecutive d per register group. Every
  // lane stages its tiles (the staging is per wave); inactive lanes store
  // nothing.
  template <typename T>
  __device__ __forceinline__ void store_rows(T* row_base, int64_t row_stride) const {
    T* dst = row_base + (int64_t)(lane & 31) * row_stride + 4 * half;
    const float f = 1.f / lsum;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) {
      const f32x16 x = through_lds(o[dt]);
      if (active) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store4(dst + 32 * dt + 8 * g, f32x4{x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]} * f);
      }
    }
  }
};

// A workgroup's share: tiles [u0, u0 + units) in (sequence, tile) order, one
// pipeline across the sequences it spans. Wave WAVE of W copies slots
// [36 WAVE / W, 36 (WAVE + 1) / W) of every tile (slot s: 1 KiB s % 18 of the
// tile's block s / 18). Each tile starts with a barrier: every wave has waited
// for its own copies of the tile, so after it the tile is whole in LDS, and
// every wave is past the previous tile, whose buffer the next copy refills.
template <int W, int WAVE>
__device__ __forceinline__ void wide_share(const MlaArgs& a, int share, int seq, int tile, int64_t units) {
  constexpr int kS0 = kCopySlots * WAVE / W, kS1 = kCopySlots * (WAVE + 1) / W;
  const DecodeArgs& d = a.d;
  const int S = d.num_seqs;
  const unsigned top = (unsigned)(d.num_blocks - 1);
  const int hg = WAVE;
  struct Seg {   // tiles [t0, t1) of sequence seq; L tokens in nblk blocks, ntiles tiles in all
    int seq, t0, t1, ntiles, nblk, L;
  };
  auto make_seg = [&](int s, int t0, int64_t left) {
    Seg g;
    g.seq = s;
    g.t0 = t0;
    g.L = clamp_len(d.seq_lens[s], d.max_seq_len);
    g.nblk = blocks_of<kBS>(g.L);
    g.ntiles = blocks_of<kTileTok>(g.L);
    g.t1 = t0 + (int)min((int64_t)(g.ntiles - t0), left);
    return g;
  };

  WideWave wv;
  wv.init(a, hg);
  const int lane = wv.lane;
  Seg cur = make_seg(seq, tile, units);
  int64_t left = units - (cur.t1 - cur.t0);
  wv.load_q(a, cur.seq, hg);
  wv.reset();
  const int32_t* trow = d.block_tables + (int64_t)cur.seq * d.max_blocks_per_seq;
  int chunk = 2 * cur.t0;   // lane i of tbl holds the table entry of block chunk + i (clamped to the last)
  int tbl = trow[min(chunk + lane, cur.nblk - 1)];

  // The share's next sequence (its length and first 64 table entries).
  Seg nx{};
  bool has_nx = false;
  int tbl_n = 0;
  auto prefetch = [&]() {
    has_nx = false;
    if (left <= 0) return;
    int s = cur.seq;
    do {
      ++s;
    } while (s < S && clamp_len(d.seq_lens[s], d.max_seq_len) == 0);
    if (s >= S) return;   // only with inconsistent inputs
    nx = make_seg(s, 0, left);
    has_nx = true;
    tbl_n = d.block_tables[(int64_t)nx.seq * d.max_blocks_per_seq + min(lane, nx.nblk - 1)];
  };
  prefetch();

  const char* cache = reinterpret_cast<const char*>(d.key_cache);
  // Copies this wave's slots of a tile (physical blocks p0, p1; p1 only when
  // the tile's second block holds tokens) into buffer B.
  auto stage = [&](auto bsel, unsigned p0, unsigned p1, bool two) {
    constexpr int B = decltype(bsel)::value;
    p0 = p0 < top ? p0 : top;
    p1 = p1 < top ? p1 : top;
#pragma unroll
    for (int s = kS0; s < kS1; ++s) {
      const int blk = s / (kCopySlots / 2), part = s % (kCopySlots / 2);
      if (blk == 1 && !two) continue;
      const char* src = cache + (int64_t)(blk ? p1 : p0) * kBlockBytes + part * 1024 + lane * 16;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(tile_buf<B>() + blk * kBlockVec +
                                                                                  part * 64),
                                       16, 0, 2 /* nt */);
    }
  };
  // Tile t of cur, or the first tile of the next sequence.
  auto stage_cur = [&](auto bsel, int t) {
    if (2 * t - chunk >= 64) {
      chunk += 64;
      tbl = trow[min(chunk + lane, cur.nblk - 1)];
    }
    const int nv = min(kTileTok, cur.L - t * kTileTok);
    stage(bsel, (unsigned)__builtin_amdgcn_readlane(tbl, 2 * t - chunk),
          (unsigned)__builtin_amdgcn_readlane(tbl, 2 * t + 1 - chunk), nv > kBS);
  };
  auto stage_next_seq = [&](auto bsel) {
    stage(bsel, (unsigned)__builtin_amdgcn_readlane(tbl_n, 0), (unsigned)__builtin_amdgcn_readlane(tbl_n, 1),
          nx.L > kBS);
  };

  int t = cur.t0;
  // Computes tile t of cur (in buffer B) after starting its successor's copy
  // into the other buffer; false once the share is done.
  auto step = [&](auto bsel) -> bool {
    constexpr int B = decltype(bsel)::value;
    using Next = std::integral_constant<int, 1 - B>;
    const bool more = t + 1 < cur.t1;
    tile_barrier();
    if (more)
      stage_cur(Next{}, t + 1);
    else if (has_nx)
      stage_next_seq(Next{});
    const int nvalid = min(kTileTok, cur.L - t * kTileTok);
    if (nvalid < kTileTok)
      wv.template compute<B, true>(nvalid);
    else
      wv.template compute<B, false>(kTileTok);
    if (more) {
      ++t;
      return true;
    }
    wv.finish();
    const int64_t h0 = (int64_t)cur.seq * d.num_heads + hg * 32;
    if (cur.t0 == 0 && cur.t1 == cur.ntiles) {
      wv.store_rows(reinterpret_cast<__bf16*>(d.out) + h0 * kLatent, kLatent);
    } else {
      const int64_t row = (int64_t)(cur.seq + share) * a.hpad + hg * 32;   // slot (seq + share)
      wv.store_rows(d.seg_out + row * kLatent, kLatent);
      if (wv.active && wv.half == 0) {
        d.seg_max[row + (lane & 31)] = wv.m;
        d.seg_sum[row + (lane & 31)] = wv.lsum;
      }
    }
    if (hg == 0 && lane == 0) {
      if (cur.t0 == 0) d.seg_meta[2 * cur.seq] = share;
      if (cur.t1 == cur.ntiles) d.seg_meta[2 * cur.seq + 1] = share;
    }
    if (!has_nx) return false;
    cur = nx;
    left -= cur.t1 - cur.t0;
    wv.load_q(a, cur.seq, hg);
    wv.reset();
    trow = d.block_tables + (int64_t)cur.seq * d.max_blocks_per_seq;
    chunk = 0;
    tbl = tbl_n;
    t = 0;
    prefetch();
    return true;
  };
  stage_cur(std::integral_constant<int, 0>{}, cur.t0);
  while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
  }
}

// Grid: one workgroup of W waves (32 heads each) per stream-K share.
template <int W>
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
  switch (wave) {
    case 0: wide_share<W, 0>(a, share, seq, tile, u1 - u0); break;
    case 1: if constexpr (W > 1) wide_share<W, 1 % W>(a, share, seq, tile, u1 - u0); break;
    case 2: if constexpr (W > 2) wide_share<W, 2 % W>(a, share, seq, tile, u1 - u0); break;
    default: if constexpr (W > 3) wide_share<W, 3 % W>(a, share, seq, tile, u1 - u0); break;
  }
}

}  // namespace

hipError_t launch_mla_wide(const MlaArgs& a, hipStream_t stream) {
  const dim3 grid(a.shares);
  switch (a.waves_per_wg) {
    case 1: hipLaunchKernelGGL(pa_mla_wide_kernel<1>, grid, dim3(64), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(pa_mla_wide_kernel<2>, grid, dim3(128), 0, stream, a); break;
    case 3: hipLaunchKernelGGL(pa_mla_wide_kernel<3>, grid, dim3(192), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(pa_mla_wide_kernel<4>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
