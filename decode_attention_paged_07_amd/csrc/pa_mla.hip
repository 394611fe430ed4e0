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
// contiguous, and a block is one 18 KiB run.
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
//     and serves as both K and V. The only LDS use is each lane's own copy of
//     its q pieces (a register extension; no barriers).
// With more than 16 heads every 16-head group has its own wave on the same
// share of blocks: two groups share a workgroup, more are split over
// workgroups dispatched to the same XCD, so a tile's reads after the first
// hit in L1 or L2.
//
// Scheduling is stream-K over (sequence, block) tiles, as for the decode
// kernels: every share has the same number of blocks; a sequence cut by a
// share boundary writes partials that a merge kernel combines.

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
constexpr int64_t kMlaBlockBytes = (int64_t)kMlaWidth * kMlaBS * 2;

// Dynamic LDS: kMlaSteps * 64 16-byte slots per wave, each lane's own q
// pieces (written and read back by the same lane; no barrier).
extern __shared__ u32x4 mla_q_lds[];

struct MlaWave {
  u32x4* qs;            // this wave's q slots in LDS
  f32x4 o[kMlaDt];
  s16x4 ident;          // B operand of the transposing product
  float m, lsum, c;
  uint32_t koff;        // this lane's byte offset in a tile (step 0)
  int lane, q4;
  bool active;          // this lane's column is a real query head

  __device__ void init(const MlaArgs& a, int hg) {
    lane = threadIdx.x & 63;
    q4 = lane >> 4;
    const int j = lane & 15;
    active = hg * 16 + j < a.d.num_heads;
    koff = (uint32_t)(q4 * kMlaBS * 16 + j * 16);
    c = a.d.scale * kLog2e;
    qs = mla_q_lds + (threadIdx.x >> 6) * (kMlaSteps * 64);
    // lane (j + 16*q4) holds I[4*q4 + u][j], u = 0..3.
    short e[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) e[u] = (4 * q4 + u == j) ? (short)0x3F80 : (short)0;
    ident = s16x4{e[0], e[1], e[2], e[3]};
  }

  // q rows of heads hg*16 + column, in the d-order of the tile loads: step
  // s, lane quad q4 -> d = 8*(4s + q4) + u.
  __device__ void load_q(const MlaArgs& a, int seq, int hg) {
    const int h = hg * 16 + (active ? (lane & 15) : 0);
    const __bf16* qh = reinterpret_cast<const __bf16*>(a.d.query) + ((int64_t)seq * a.d.num_heads + h) * kMlaWidth;
#pragma unroll
    for (int s = 0; s < kMlaSteps; ++s) {
      u32x4 w = {0, 0, 0, 0};
      if (active) w = *reinterpret_cast<const u32x4*>(qh + 8 * (4 * s + q4));
      qs[s * 64 + lane] = w;
    }
  }

  __device__ void reset() {
    m = kNegInf;
    lsum = 0.f;
#pragma unroll
    for (int dt = 0; dt < kMlaDt; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  __device__ void load_tile(const char* tile, u32x4 (&k)[kMlaSteps]) const {
#pragma unroll
    for (int s = 0; s < kMlaSteps; ++s)
      k[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(tile + koff + s * 4 * kMlaBS * 16));
  }

  // One block; tokens >= nvalid (a sequence's partial last block) are masked
  // by select: their logits become -inf and their values 0, since stale
  // slots may hold NaN and 0 * NaN would poison the sums.
  __device__ void consume(const u32x4 (&k)[kMlaSteps], int nvalid) {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kMlaSteps; ++s)
      z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[s]),
                                                  __builtin_bit_cast(bf16x8, qs[s * 64 + lane]), z, 0, 0, 0);
    z *= c;
    const bool partial = nvalid < kMlaBS;
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
    const s16x4 pb = pack_bf16x4(p);
#pragma unroll
    for (int s = 0; s < kMlaVSteps; ++s)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const u32x2 half = {k[s][2 * hf], k[s][2 * hf + 1]};
        f32x4 vt = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, half), ident,
                                                             f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        if (partial) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (4 * q4 + r >= nvalid) vt[r] = 0.f;
        }
        o[2 * s + hf] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pack_bf16x4(vt), pb, o[2 * s + hf], 0, 0, 0);
      }
  }

  __device__ void finish() { lsum = quad_sum(lsum); }

  // o / lsum for this lane's head. Tile 2s + hf row 4*q4 + r is
  // d = 32s + 8*q4 + 4*hf + r: four consecutive d per tile.
  template <typename T>
  __device__ void store_rows(T* row_base, int64_t row_stride) const {
    if (!active) return;
    T* dst = row_base + (int64_t)(lane & 15) * row_stride + 8 * q4;
    const float f = 1.f / lsum;
#pragma unroll
    for (int s = 0; s < kMlaVSteps; ++s)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) store4(dst + 32 * s + 4 * hf, o[2 * s + hf] * f);
  }
};

// One wave's share: tiles [u0, u0 + units) in (sequence, block) order, as one
// block pipeline across the sequences it spans (the next block's loads are
// in flight while the current one is computed, also across a sequence
// boundary).
__device__ void mla_share(const MlaArgs& a, int share, int hg, int seq, int blk, int64_t units) {
  const DecodeArgs& d = a.d;
  const int S = d.num_seqs;
  const unsigned top = (unsigned)(d.num_blocks - 1);
  const int hpad = a.head_groups * 16;
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

  MlaWave wv;
  wv.init(a, hg);
  const int lane = wv.lane;
  Seg cur = make_seg(seq, blk, units);
  int64_t left = units - (cur.b1 - cur.b0);
  wv.load_q(a, cur.seq, hg);
  wv.reset();
  const int32_t* trow = d.block_tables + (int64_t)cur.seq * d.max_blocks_per_seq;
  int chunk = cur.b0;
  int tbl = trow[min(chunk + lane, cur.b1 - 1)];

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
    tbl_n = d.block_tables[(int64_t)nx.seq * d.max_blocks_per_seq + min(lane, nx.b1 - 1)];
  };
  prefetch();

  const char* base = reinterpret_cast<const char*>(d.key_cache);
  auto load_block = [&](unsigned phys, u32x4 (&k)[kMlaSteps]) {
    phys = phys < top ? phys : top;
    wv.load_tile(base + (int64_t)phys * kMlaBlockBytes, k);
  };
  auto issue_cur = [&](int g, u32x4 (&k)[kMlaSteps]) {
    if (g - chunk >= 64) {
      chunk += 64;
      tbl = trow[min(chunk + lane, cur.b1 - 1)];
    }
    load_block((unsigned)__builtin_amdgcn_readlane(tbl, g - chunk), k);
  };

  int g = cur.b0;
  auto step = [&](u32x4 (&kr)[kMlaSteps], u32x4 (&kn)[kMlaSteps]) -> bool {
    const bool more = g + 1 < cur.b1;
    if (more)
      issue_cur(g + 1, kn);
    else if (has_nx)
      load_block((unsigned)__builtin_amdgcn_readlane(tbl_n, 0), kn);
    const int nvalid = min(kMlaBS, cur.L - g * kMlaBS);
    wv.consume(kr, nvalid);
    if (more) {
      ++g;
      return true;
    }
    wv.finish();
    const int64_t h0 = (int64_t)cur.seq * d.num_heads + hg * 16;
    if (cur.b0 == 0 && cur.b1 == cur.nbs) {
      wv.store_rows(reinterpret_cast<__bf16*>(d.out) + h0 * kMlaLatent, kMlaLatent);
    } else {
      const int64_t row = (int64_t)(cur.seq + share) * hpad + hg * 16;   // slot (seq + share)
      wv.store_rows(d.seg_out + row * kMlaLatent, kMlaLatent);
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

  u32x4 ka[kMlaSteps], kb[kMlaSteps];
  issue_cur(cur.b0, ka);
  while (step(ka, kb) && step(kb, ka)) {
  }
}

// Grid: shares * chunks workgroups of waves_per_wg waves. Workgroup i takes
// share 8*(i / (8*chunks)) + i % 8 and head-group chunk (i / 8) % chunks, so
// the chunks of a share are 8 workgroup ids apart: the same XCD under the
// round-robin dispatch of workgroups to the eight XCDs.
__global__ void __launch_bounds__(256) pa_mla_streamk_kernel(const MlaArgs a) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x;
  const int chunks = a.chunks;
  const int share = 8 * (i / (8 * chunks)) + i % 8;
  const int chunk = (i / 8) % chunks;
  const int hg = chunk * a.waves_per_wg + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (hg >= a.head_groups || share >= a.shares) return;

  int bsum = 0;
  const int T = count_blocks<kMlaBS>(a.d, lane, bsum);
  if (T == 0) return;
  const int64_t U = ((int64_t)T + a.shares - 1) / a.shares;
  const int64_t u0 = (int64_t)share * U;
  const int64_t u1 = min((int64_t)T, u0 + U);
  if (u0 >= u1) return;
  int seq = 0, blk = 0;
  locate_block<kMlaBS>(a.d, lane, (int)u0, bsum, seq, blk);
  mla_share(a, share, hg, seq, blk, u1 - u0);
}

// Merge of the segments of cut sequences, zero rows of empty ones: grid
// (head_groups, num_seqs), 256 threads; one (sequence, 16-head group) each.
__global__ void __launch_bounds__(256) pa_mla_reduce_kernel(const MlaArgs a) {
  const DecodeArgs& d = a.d;
  const int hg = blockIdx.x;
  const int seq = blockIdx.y;
  const int hpad = a.head_groups * 16;
  const int nh = min(16, d.num_heads - hg * 16);
  const int L = clamp_len(d.seq_lens[seq], d.max_seq_len);
  __bf16* out = reinterpret_cast<__bf16*>(d.out) + ((int64_t)seq * d.num_heads + hg * 16) * kMlaLatent;
  if (L == 0) {
    for (int e = threadIdx.x; e < nh * kMlaLatent; e += 256) out[e] = static_cast<__bf16>(0.f);
    return;
  }
  const int w0 = max(0, d.seg_meta[2 * seq]);
  const int w1 = min(a.shares - 1, d.seg_meta[2 * seq + 1]);
  if (w0 >= w1) return;   // one segment: written directly
  for (int e = threadIdx.x; e < nh * (kMlaLatent / 4); e += 256) {
    const int h = e / (kMlaLatent / 4);
    const int d4 = e - h * (kMlaLatent / 4);
    float big_m = kNegInf;
    for (int w = w0; w <= w1; ++w) big_m = fmaxf(big_m, d.seg_max[(int64_t)(seq + w) * hpad + hg * 16 + h]);
    float tot = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int w = w0; w <= w1; ++w) {
      const int64_t row = (int64_t)(seq + w) * hpad + hg * 16 + h;
      const float f = fast_exp2(d.seg_max[row] - big_m) * d.seg_sum[row];
      tot += f;
      acc += f * *reinterpret_cast<const f32x4*>(d.seg_out + row * kMlaLatent + 4 * d4);
    }
    store4(out + (int64_t)h * kMlaLatent + 4 * d4, acc * (1.f / tot));
  }
}

hipError_t launch_mla(const MlaArgs& a, hipStream_t stream, const LaunchHooks& hooks) {
  if (hooks.before_partition) hooks.before_partition(stream);
  const size_t lds = (size_t)a.waves_per_wg * kMlaSteps * 64 * sizeof(u32x4);
  hipLaunchKernelGGL(pa_mla_streamk_kernel, dim3(a.shares * a.chunks), dim3(a.waves_per_wg * 64), lds, stream, a);
  hipError_t err = hipGetLastError();
  if (hooks.after_partition) hooks.after_partition(stream);
  if (err != hipSuccess) return err;
  if (hooks.before_reduce) hooks.before_reduce(stream);
  hipLaunchKernelGGL(pa_mla_reduce_kernel, dim3(a.head_groups, a.d.num_seqs), dim3(256), 0, stream, a);
  err = hipGetLastError();
  if (hooks.after_reduce) hooks.after_reduce(stream);
  return err;
}

}  // namespace pa
