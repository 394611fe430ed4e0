// Paged MLA (multi-head latent attention) decode for gfx950.
//
// The 10100.com article on the retirement of vLLM's PagedAttention kernels
// (§2) names the case the old kernels cannot serve: every token stores one
// compressed row [c_kv, k_rope] instead of separate K and V. Decode in the
// absorbed form reads that row once and uses it twice: the whole row (width
// 576 = 512 latent + 64 rope) is the key of every query head, and its first
// 512 elements (c_kv) are the value. Logits are scale * q_h . row_t; the
// output of head h is the softmax-weighted sum of c_kv over the valid tokens.
//
// Cache layout: the pages' K layout (§2) with one kv head and x = 8 bf16,
// [num_blocks, 576/8, 16, 8]: 16 tokens of one 16-byte chunk are 256 bytes
// contiguous, and a block is one 18 KiB run. With 32-token blocks
// ([num_blocks, 72, 32, 8], 36 KiB) each block is two 16-token tiles, chunk c
// of tile h at 512 c + 256 h; the kernels work on 16-token tiles either way.
//
// One wave owns 16 query heads (the MFMA column count) of a run of blocks:
//   S[t][g] = sum_d row_t[d] q[g][d]: A = the latent tile (rows = tokens),
//     18 steps of v_mfma_f32_16x16x32_bf16; lane (t + 16*q4) of step s loads
//     chunk 4s + q4 of token t, so one load instruction reads 1 KiB
//     contiguous.
//   O[d][g] += sum_t c_kv_t[d] P[g][t]: the A operand needs four consecutive
//     tokens of one d per lane, but the loads hold eight consecutive d of one
//     token. The transpose is an MFMA with an identity B operand: C = A * I
//     returns the tile in the result layout, where lane (j + 16*q4) holds
//     tokens 4*q4 .. 4*q4+3 of column j, exactly the A layout of the next
//     product. Products with 1 and 0 and sums with zeros are exact, so the
//     bf16 values come back unchanged. The latent tile is read from HBM once
//     and serves as both K and V.
// Tiles go from HBM straight to LDS (global_load_lds_dwordx4) into two
// buffers per workgroup, so the next block's 18 KiB are in flight without
// holding registers. With 16 heads or fewer a workgroup is one wave, which
// reads back only what its own copies wrote: no barrier. With more heads, up
// to four 16-head groups are waves of one workgroup that share the buffers
// (each copies part of every tile; one barrier per block), and more groups
// take several workgroups per share, dispatched to the same XCD.
//
// Scheduling is stream-K over (sequence, block) tiles, as for the decode
// kernels: every share has the same number of blocks; a sequence cut by a
// share boundary writes partials that a merge kernel combines.
//
// fp8 latent cache (the pages' scaled fp8 storage, §4, one scale for the
// row): x = 16 codes per chunk, [num_blocks, 36, 16, 16], 9 KiB per block.
// A lane's 16-byte LDS slot then holds 16 consecutive d of one token, which
// become the A operands of two consecutive S steps after an exact e4m3 ->
// bf16 conversion: step s covers d = 64*(s/2) + 16*q4 + 8*(s%2) + u. The
// query is loaded in that d order, and everything after the conversion is
// the bf16 path; the scale multiplies the logits and the output.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_decode.h"
#include "pa_kernels.h"
#include "pa_sched.h"
#include "pa_wave.h"

namespace pa {

constexpr int kMlaLatent = PA_MLA_LATENT_DIM;                  // c_kv width
constexpr int kMlaWidth = PA_MLA_LATENT_DIM + PA_MLA_ROPE_DIM;  // row width
constexpr int kMlaBS = 16;
constexpr int kMlaSteps = kMlaWidth / 32;              // S steps (32 d each)
constexpr int kMlaVSteps = kMlaLatent / 32;            // steps that hold c_kv
constexpr int kMlaDt = kMlaLatent / 16;                // 16-row output tiles
// 1 KiB copies per tile (one cache block): 18 for bf16, 9 for fp8 codes.
template <bool FP8>
constexpr int kMlaSlots = FP8 ? kMlaSteps / 2 : kMlaSteps;
template <bool FP8>
constexpr int64_t kMlaTileBytes = (int64_t)kMlaSlots<FP8> * 1024;

// d offset of element u of this lane's S step s (lane quad q4), and of the
// first of the four rows r of output tile 2s + hf.
template <bool FP8>
__device__ __forceinline__ int mla_d(int s, int q4) {
  return FP8 ? 64 * (s >> 1) + 16 * q4 + 8 * (s & 1) : 32 * s + 8 * q4;
}

// s_waitcnt immediate (gfx9 encoding) of lgkmcnt(0) alone.
constexpr int kWaitLgkm0 = 0xC07F;

__device__ __forceinline__ s16x4 pack_bf16x4_pairs(f32x4 v) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const u32x2 w = {__builtin_bit_cast(unsigned, __builtin_convertvector((f32x2{v[0], v[1]}), bf16x2)),
                   __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2{v[2], v[3]}), bf16x2))};
  return __builtin_bit_cast(s16x4, w);
}

// One wave's attention state for 16 query heads. The latent tiles are staged
// in LDS by direct global->LDS loads (global_load_lds_dwordx4) in the cache
// layout, so slot s*64 + lane holds chunk 4s + q4 of token (lane & 15): the A
// operand of S step s for this lane (bf16), or of steps 2s and 2s + 1 (fp8).
template <bool FP8>
struct MlaWave {
  bf16x8 q[kMlaSteps];
  f32x4 o[kMlaDt];
  s16x4 ident;          // B operand of the transposing product
  float m, lsum, c;
  float vs;             // output multiplier: the fp8 scale, or 1
  int lane, q4;
  int sh;               // 16-token tiles per cache block: 1 << sh
  bool active;          // this lane's column is a real query head

  __device__ void init(const MlaArgs& a, int hg) {
    lane = threadIdx.x & 63;
    q4 = lane >> 4;
    const int j = lane & 15;
    active = hg * 16 + j < a.d.num_heads;
    vs = (FP8 && a.d.k_scale) ? *a.d.k_scale : 1.f;
    c = a.d.scale * kLog2e * vs;
    sh = a.d.block_size == 32 ? 1 : 0;
    // lane (j + 16*q4) holds I[4*q4 + u][j], u = 0..3.
    short e[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) e[u] = (4 * q4 + u == j) ? (short)0x3F80 : (short)0;
    ident = s16x4{e[0], e[1], e[2], e[3]};
  }

  // q rows of heads hg*16 + column, in the d-order of the tile: step s, lane
  // quad q4 -> d = mla_d(s, q4) + u.
  __device__ void load_q(const MlaArgs& a, int seq, int hg) {
    const int h = hg * 16 + (active ? (lane & 15) : 0);
    const __bf16* qh = reinterpret_cast<const __bf16*>(a.d.query) + ((int64_t)seq * a.d.num_heads + h) * kMlaWidth;
#pragma unroll
    for (int s = 0; s < kMlaSteps; ++s) {
      u32x4 w = {0, 0, 0, 0};
      if (active) w = *reinterpret_cast<const u32x4*>(qh + mla_d<FP8>(s, q4));
      q[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  __device__ void reset() {
    m = kNegInf;
    lsum = 0.f;
#pragma unroll
    for (int dt = 0; dt < kMlaDt; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Copy slots [S0, S1) of 16-token tile `half` of a cache block into buf:
  // instruction s moves chunks 4s .. 4s + 3 of the tile's tokens, lane L's
  // 16 bytes being chunk 4s + L / 16 of token L % 16, to buf + 64 s. A chunk
  // of a block spans 256 << sh bytes, so with 16-token blocks instruction s
  // reads bytes [1024 s, 1024 s + 1024) of the block.
  template <int S0, int S1>
  __device__ void stage(const char* block, int half, u32x4* buf) const {
    const char* src = block + (lane >> 4) * (256 << sh) + half * 256 + (lane & 15) * 16;
#pragma unroll
    for (int s = S0; s < S1; ++s)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(src + s * (1024 << sh)),
          (__attribute__((address_space(3))) void*)(buf + s * 64), 16, 0, 2 /* nt */);
  }

  // One block from buf, whose copy is the last but PENDING outstanding
  // vector-memory operations. Tokens >= nvalid (a sequence's partial last
  // block) get logit -inf by select, and their registers are zeroed before
  // the value product (stale slots may hold NaN, and 0 * NaN would poison
  // the sums).
  // The tile's copy is waited for and its 18 slots of this lane are read in
  // one asm block (which also waits for the reads): the compiler does not see
  // LDS reads it would otherwise order after every outstanding copy,
  // including the next block's. The outputs are early-clobber: a read's
  // destination must not be the address register the later reads use.
  template <int PENDING>
  __device__ static void read_tile(const u32x4* buf, u32x4 (&k)[kMlaSteps]) {
    const uint32_t addr = (uint32_t)(uintptr_t)buf;
    asm volatile(
        "s_waitcnt vmcnt(%18)\n\t"
        "ds_read_b128 %0, %19 offset:0\n\t"
        "ds_read_b128 %1, %19 offset:1024\n\t"
        "ds_read_b128 %2, %19 offset:2048\n\t"
        "ds_read_b128 %3, %19 offset:3072\n\t"
        "ds_read_b128 %4, %19 offset:4096\n\t"
        "ds_read_b128 %5, %19 offset:5120\n\t"
        "ds_read_b128 %6, %19 offset:6144\n\t"
        "ds_read_b128 %7, %19 offset:7168\n\t"
        "ds_read_b128 %8, %19 offset:8192\n\t"
        "ds_read_b128 %9, %19 offset:9216\n\t"
        "ds_read_b128 %10, %19 offset:10240\n\t"
        "ds_read_b128 %11, %19 offset:11264\n\t"
        "ds_read_b128 %12, %19 offset:12288\n\t"
        "ds_read_b128 %13, %19 offset:13312\n\t"
        "ds_read_b128 %14, %19 offset:14336\n\t"
        "ds_read_b128 %15, %19 offset:15360\n\t"
        "ds_read_b128 %16, %19 offset:16384\n\t"
        "ds_read_b128 %17, %19 offset:17408\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]), "=&v"(k[6]),
          "=&v"(k[7]), "=&v"(k[8]), "=&v"(k[9]), "=&v"(k[10]), "=&v"(k[11]), "=&v"(k[12]), "=&v"(k[13]),
          "=&v"(k[14]), "=&v"(k[15]), "=&v"(k[16]), "=&v"(k[17])
        : "n"(PENDING), "v"(addr + 16u * (threadIdx.x & 63))
        : "memory");
  }

  // The same for a tile of fp8 codes: nine slots.
  template <int PENDING>
  __device__ static void read_tile_fp8(const u32x4* buf, u32x4 (&k)[kMlaSteps / 2]) {
    const uint32_t addr = (uint32_t)(uintptr_t)buf;
    asm volatile(
        "s_waitcnt vmcnt(%9)\n\t"
        "ds_read_b128 %0, %10 offset:0\n\t"
        "ds_read_b128 %1, %10 offset:1024\n\t"
        "ds_read_b128 %2, %10 offset:2048\n\t"
        "ds_read_b128 %3, %10 offset:3072\n\t"
        "ds_read_b128 %4, %10 offset:4096\n\t"
        "ds_read_b128 %5, %10 offset:5120\n\t"
        "ds_read_b128 %6, %10 offset:6144\n\t"
        "ds_read_b128 %7, %10 offset:7168\n\t"
        "ds_read_b128 %8, %10 offset:8192\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]), "=&v"(k[6]),
          "=&v"(k[7]), "=&v"(k[8])
        : "n"(PENDING), "v"(addr + 16u * (threadIdx.x & 63))
        : "memory");
  }

  template <int PENDING>
  __device__ void consume(u32x4* buf, int nvalid) {
    const bool partial = nvalid < kMlaBS;
    u32x4 k[kMlaSteps];
    if constexpr (FP8) {
      // 16 codes (d .. d + 15 of one token) per slot -> steps 2i and 2i + 1.
      u32x4 raw[kMlaSteps / 2];
      read_tile_fp8<PENDING>(buf, raw);
      if (partial && (lane & 15) >= nvalid) {
#pragma unroll
        for (int i = 0; i < kMlaSteps / 2; ++i) raw[i] = u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < kMlaSteps / 2; ++i) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          k[2 * i + h] = u32x4{fp8x2_to_bf16x2<false>(raw[i][2 * h]), fp8x2_to_bf16x2<true>(raw[i][2 * h]),
                               fp8x2_to_bf16x2<false>(raw[i][2 * h + 1]), fp8x2_to_bf16x2<true>(raw[i][2 * h + 1])};
      }
    } else {
      read_tile<PENDING>(buf, k);
      if (partial && (lane & 15) >= nvalid) {
#pragma unroll
        for (int s = 0; s < kMlaSteps; ++s) k[s] = u32x4{0, 0, 0, 0};
      }
    }
    f32x4 z0 = {0.f, 0.f, 0.f, 0.f}, z1 = {0.f, 0.f, 0.f, 0.f};   // two chains in flight
#pragma unroll
    for (int s = 0; s < kMlaSteps; s += 2) {
      z0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[s]), q[s], z0, 0, 0, 0);
      z1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[s + 1]), q[s + 1], z1, 0, 0, 0);
    }
    f32x4 z = (z0 + z1) * c;
    if (partial) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * q4 + r >= nvalid) z[r] = kNegInf;
    }
    const float mx = quad_max(max4(z));
    if (wave_any(mx > m + kRescaleSlack)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2(m - m_new);
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < kMlaDt; ++dt) o[dt] *= alpha;
    }
    f32x4 p;
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fast_exp2(z[r] - m);
    lsum += (p[0] + p[1]) + (p[2] + p[3]);
    const s16x4 pb = pack_bf16x4_pairs(p);
    // Four transposes ahead of their value products.
#pragma unroll
    for (int s = 0; s < kMlaVSteps; s += 2) {
      f32x4 vt[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const u32x4 w = k[s + (t >> 1)];
        const u32x2 hw = {w[2 * (t & 1)], w[2 * (t & 1) + 1]};
        vt[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, hw), ident,
                                                         f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
        o[2 * s + t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pack_bf16x4_pairs(vt[t]), pb, o[2 * s + t], 0, 0, 0);
    }
  }

  __device__ void finish() { lsum = quad_sum(lsum); }

  // o * vs / lsum for this lane's head. Tile 2s + hf row 4*q4 + r is
  // d = mla_d(s, q4) + 4*hf + r: four consecutive d per tile.
  template <typename T>
  __device__ void store_rows(T* row_base, int64_t row_stride) const {
    if (!active) return;
    T* dst = row_base + (int64_t)(lane & 15) * row_stride;
    const float f = vs / lsum;
#pragma unroll
    for (int s = 0; s < kMlaVSteps; ++s)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) store4(dst + mla_d<FP8>(s, q4) + 4 * hf, o[2 * s + hf] * f);
  }
};

// A workgroup's share: tiles [u0, u0 + units) in (sequence, block) order, as
// one block pipeline across the sequences it spans. Its W waves (one per
// 16-head group) share two LDS tile buffers: while one block is computed,
// the next block's copy (also across a sequence boundary) is in flight into
// the other. Wave w copies slots [18 w / W, 18 (w + 1) / W) of each tile.
// With W > 1 each block starts with a barrier: each wave first waits for its
// own copies, so after it the tile is complete in LDS, and every wave is
// past the previous block, whose buffer the next copy overwrites.
template <int W, int WAVE, bool FP8>
__device__ __forceinline__ void mla_share(const MlaArgs& a, int share, int hg, int seq, int blk, int64_t units,
                                          u32x4* __restrict__ buf0, u32x4* __restrict__ buf1) {
  constexpr int kSlots = kMlaSlots<FP8>;
  constexpr int kS0 = kSlots * WAVE / W, kS1 = kSlots * (WAVE + 1) / W;
  const DecodeArgs& d = a.d;
  const int S = d.num_seqs;
  const unsigned top = (unsigned)(d.num_blocks - 1);
  struct Seg {
    int seq, b0, b1, nbs, L;
  };
  auto make_seg = [&](int s, int b0, int64_t left) {
    Seg g;
    g.seq = s;
    g.b0 = b0;
    g.L = clamp_len(d.seq_lens[s], d.max_seq_len);
    g.nbs = blocks_of<kMlaBS>(g.L);
    g.b1 = b0 + (int)min((int64_t)(g.nbs - b0), left);
    return g;
  };

  MlaWave<FP8> wv;
  wv.init(a, hg);
  const int lane = wv.lane;
  Seg cur = make_seg(seq, blk, units);
  int64_t left = units - (cur.b1 - cur.b0);
  wv.load_q(a, cur.seq, hg);
  wv.reset();
  // Lane i of tbl holds the table entry of tile chunk + i (tile g is in
  // block g >> sh).
  const int sh = wv.sh;
  const int32_t* trow = d.block_tables + (int64_t)cur.seq * d.max_blocks_per_seq;
  int chunk = cur.b0;
  int tbl = trow[min((chunk + lane) >> sh, (cur.b1 - 1) >> sh)];

  // The share's next sequence (seq_len and first 64 table entries).
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
    tbl_n = d.block_tables[(int64_t)nx.seq * d.max_blocks_per_seq + min(lane >> sh, (nx.b1 - 1) >> sh)];
  };
  prefetch();

  const char* base = reinterpret_cast<const char*>(d.key_cache);
  auto stage_block = [&](unsigned phys, int half, u32x4* buf) {
    phys = phys < top ? phys : top;
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // earlier LDS reads of buf are complete
    wv.template stage<kS0, kS1>(base + (int64_t)phys * (kMlaTileBytes<FP8> << sh), half, buf);
  };
  auto stage_cur = [&](int g, u32x4* buf) {
    if (g - chunk >= 64) {
      chunk += 64;
      tbl = trow[min((chunk + lane) >> sh, (cur.b1 - 1) >> sh)];
    }
    stage_block((unsigned)__builtin_amdgcn_readlane(tbl, g - chunk), g & sh, buf);
  };

  int g = cur.b0;
  // Computes block g of cur (in bc) after starting its successor's copy into
  // bn; false once the share is done.
  auto step = [&](u32x4* bc, u32x4* bn) -> bool {
    const bool more = g + 1 < cur.b1;
    const int nvalid = min(kMlaBS, cur.L - g * kMlaBS);
    // The tile reads wait for all but the successor's copy (one wave), or
    // not at all (several waves: the barrier has).
    constexpr int kPending = W == 1 ? kS1 - kS0 : 63;
    if constexpr (W > 1) {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies of bc
      __builtin_amdgcn_s_barrier();
    }
    if (more) {
      stage_cur(g + 1, bn);
      wv.template consume<kPending>(bc, nvalid);
    } else if (has_nx) {
      stage_block((unsigned)__builtin_amdgcn_readlane(tbl_n, 0), 0, bn);
      wv.template consume<kPending>(bc, nvalid);
    } else {
      wv.template consume<W == 1 ? 0 : 63>(bc, nvalid);
    }
    if (more) {
      ++g;
      return true;
    }
    wv.finish();
    const int64_t h0 = (int64_t)cur.seq * d.num_heads + hg * 16;
    if (cur.b0 == 0 && cur.b1 == cur.nbs) {
      wv.store_rows(reinterpret_cast<__bf16*>(d.out) + h0 * kMlaLatent, kMlaLatent);
    } else {
      const int64_t row = (int64_t)(cur.seq + share) * a.hpad + hg * 16;   // slot (seq + share)
      wv.store_rows(reinterpret_cast<__bf16*>(d.seg_out) + row * kMlaLatent, kMlaLatent);
      if (wv.active && wv.q4 == 0) {
        d.seg_max[row + (lane & 15)] = wv.m;
        d.seg_sum[row + (lane & 15)] = wv.lsum;
      }
    }
    if (hg == 0 && lane == 0) {
      if (cur.b0 == 0) d.seg_meta[2 * cur.seq] = share;
      if (cur.b1 == cur.nbs) d.seg_meta[2 * cur.seq + 1] = share;
    }
    if (!has_nx) return false;
    cur = nx;
    left -= cur.b1 - cur.b0;
    wv.load_q(a, cur.seq, hg);
    wv.reset();
    trow = d.block_tables + (int64_t)cur.seq * d.max_blocks_per_seq;
    chunk = 0;
    tbl = tbl_n;
    g = 0;
    prefetch();
    return true;
  };

  stage_cur(cur.b0, buf0);
  while (step(buf0, buf1) && step(buf1, buf0)) {
  }
}

// Grid: shares * chunks workgroups of W waves (36 KiB of LDS each). Wave w of
// workgroup i takes share 8*(i / (8*chunks)) + i % 8 and head group
// ((i / 8) % chunks) * W + w, so the chunks of a share are 8 workgroup ids
// apart: the same XCD under the round-robin dispatch of workgroups to the
// eight XCDs. A wave past the last head group runs with no active lane (it
// still copies its slots and meets the barriers).
template <int W, bool FP8>
__global__ void __launch_bounds__(64 * W) pa_mla_streamk_kernel(const MlaArgs a) {
  // two tile buffers: 18 KiB each (bf16), 9 KiB (fp8)
  __shared__ u32x4 tiles0[kMlaSlots<FP8> * 64], tiles1[kMlaSlots<FP8> * 64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = blockIdx.x;
  const int chunks = a.chunks;
  const int share = 8 * (i / (8 * chunks)) + i % 8;
  const int hg = ((i / 8) % chunks) * W + wave;
  if (share >= a.shares) return;   // uniform over the workgroup

  int bsum = 0;
  const int T = count_blocks<kMlaBS>(a.d, lane, bsum);
  if (T == 0) return;
  const int64_t U = ((int64_t)T + a.shares - 1) / a.shares;
  const int64_t u0 = (int64_t)share * U;
  const int64_t u1 = min((int64_t)T, u0 + U);
  if (u0 >= u1) return;
  int seq = 0, blk = 0;
  locate_block<kMlaBS>(a.d, lane, (int)u0, bsum, seq, blk);
  // Each wave runs its own instantiation (its copy slots); all meet the same barriers.
  switch (wave) {
    case 0: mla_share<W, 0, FP8>(a, share, hg, seq, blk, u1 - u0, tiles0, tiles1); break;
    case 1: if constexpr (W > 1) mla_share<W, 1 % W, FP8>(a, share, hg, seq, blk, u1 - u0, tiles0, tiles1); break;
    case 2: if constexpr (W > 2) mla_share<W, 2 % W, FP8>(a, share, hg, seq, blk, u1 - u0, tiles0, tiles1); break;
    default: if constexpr (W > 3) mla_share<W, 3 % W, FP8>(a, share, hg, seq, blk, u1 - u0, tiles0, tiles1); break;
  }
}

// Merge of the segments of cut sequences, zero rows of empty ones. A
// segment's row is stored in bf16, the output type (its max and sum stay
// fp32): half the bytes written and read back, for one more rounding of at
// most 2^-9 relative per row. Grid
// (num_seqs, ceil(num_heads / 4)), four waves of 64; one (sequence, head) row
// per wave, eight of its 512 values per lane. The segments' weights are
// computed one per lane; their rows are read eight segments at a time with
// the loads in flight together, and added in segment order.
__global__ void __launch_bounds__(256) pa_mla_reduce_kernel(const MlaArgs a) {
  const DecodeArgs& d = a.d;
  const int seq = blockIdx.x;
  const int h = blockIdx.y * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (h >= d.num_heads) return;
  const int64_t hpad = a.hpad;
  // The length and the segment bounds are read together (the bounds are
  // only used when the length is non-zero).
  const int len = d.seq_lens[seq];
  const int m0 = d.seg_meta[2 * seq], m1 = d.seg_meta[2 * seq + 1];
  const int L = clamp_len(len, d.max_seq_len);
  __bf16* out = reinterpret_cast<__bf16*>(d.out) + ((int64_t)seq * d.num_heads + h) * kMlaLatent + 8 * lane;
  if (L == 0) {
    store4(out, f32x4{0.f, 0.f, 0.f, 0.f});
    store4(out + 4, f32x4{0.f, 0.f, 0.f, 0.f});
    return;
  }
  const int w0 = max(0, m0);
  const int w1 = min(a.shares - 1, m1);
  if (w0 >= w1) return;   // one segment: written directly
  auto row = [&](int w) { return (int64_t)(seq + w) * hpad + h; };
  // Up to 64 segments: lane i keeps segment w0 + i's max and sum from one
  // read. More: the maxima are gathered first, the sums read per chunk.
  const bool one_chunk = w1 - w0 < 64;
  float sm = kNegInf, ss = 0.f;
  if (one_chunk && w0 + lane <= w1) {
    sm = d.seg_max[row(w0 + lane)];
    ss = d.seg_sum[row(w0 + lane)];
  }
  float big_m = sm;
  if (!one_chunk)
    for (int w = w0 + lane; w <= w1; w += 64) big_m = fmaxf(big_m, d.seg_max[row(w)]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) big_m = fmaxf(big_m, __shfl_xor(big_m, off, 64));
  float tot = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int c = w0; c <= w1; c += 64) {
    const int n = min(64, w1 - c + 1);
    float f = 0.f;
    if (lane < n) {
      if (one_chunk)
        f = fast_exp2(sm - big_m) * ss;
      else
        f = fast_exp2(d.seg_max[row(c + lane)] - big_m) * d.seg_sum[row(c + lane)];
    }
    tot += f;
    constexpr int kU = 8;
    for (int u = 0; u < n; u += kU) {
      f32x4 v0[kU], v1[kU];
      float fw[kU];
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        const int idx = min(u + k, n - 1);
        fw[k] = u + k < n ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), idx)) : 0.f;
        const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const __bf16*>(d.seg_out) +
                                                        row(c + idx) * kMlaLatent + 8 * lane);
        v0[k] = f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u), __uint_as_float(w[1] << 16),
                      __uint_as_float(w[1] & 0xFFFF0000u)};
        v1[k] = f32x4{__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xFFFF0000u), __uint_as_float(w[3] << 16),
                      __uint_as_float(w[3] & 0xFFFF0000u)};
      }
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        acc0 += fw[k] * v0[k];
        acc1 += fw[k] * v1[k];
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off, 64);
  const float inv = 1.f / tot;
  store4(out, acc0 * inv);
  store4(out + 4, acc1 * inv);
}

hipError_t launch_mla(const MlaArgs& a, hipStream_t stream, const LaunchHooks& hooks) {
  if (hooks.before_partition) hooks.before_partition(stream);
  hipError_t err = hipSuccess;
  if (a.wide) {
    err = launch_mla_wide(a, stream);
  } else {
    const dim3 grid(a.shares * a.chunks);
    const int key = a.waves_per_wg * 2 + (a.fp8 ? 1 : 0);
    switch (key) {
      case 2: hipLaunchKernelGGL((pa_mla_streamk_kernel<1, false>), grid, dim3(64), 0, stream, a); break;
      case 4: hipLaunchKernelGGL((pa_mla_streamk_kernel<2, false>), grid, dim3(128), 0, stream, a); break;
      case 6: hipLaunchKernelGGL((pa_mla_streamk_kernel<3, false>), grid, dim3(192), 0, stream, a); break;
      case 8: hipLaunchKernelGGL((pa_mla_streamk_kernel<4, false>), grid, dim3(256), 0, stream, a); break;
      case 3: hipLaunchKernelGGL((pa_mla_streamk_kernel<1, true>), grid, dim3(64), 0, stream, a); break;
      case 5: hipLaunchKernelGGL((pa_mla_streamk_kernel<2, true>), grid, dim3(128), 0, stream, a); break;
      case 7: hipLaunchKernelGGL((pa_mla_streamk_kernel<3, true>), grid, dim3(192), 0, stream, a); break;
      case 9: hipLaunchKernelGGL((pa_mla_streamk_kernel<4, true>), grid, dim3(256), 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    err = hipGetLastError();
  }
  if (hooks.after_partition) hooks.after_partition(stream);
  if (err != hipSuccess) return err;
  if (hooks.before_reduce) hooks.before_reduce(stream);
  hipLaunchKernelGGL(pa_mla_reduce_kernel, dim3(a.d.num_seqs, (a.d.num_heads + 3) / 4), dim3(256), 0, stream, a);
  err = hipGetLastError();
  if (hooks.after_reduce) hooks.after_reduce(stream);
  return err;
}

}  // namespace pa
