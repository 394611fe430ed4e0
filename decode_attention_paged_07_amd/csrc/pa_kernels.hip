// Paged decode-attention kernels for gfx950 (CDNA4, wave64, MFMA).
//
// Unit of work: one wave streams a run of consecutive logical blocks of one
// (sequence, kv head) pair and keeps an online-softmax state for all query
// heads of that kv head (GQA packing). K and V tiles of a block are loaded
// straight from HBM into MFMA operand registers; every K and V byte is read
// once, in a single traversal with the K and V loads of a block in flight
// together. (The pages' prior-art CUDA kernel walked the table twice, K and
// softmax first and V second, with a barrier in between: 10100.com
// retirement article, §3.)
//
// Two schedulers feed that unit:
//  * split grid: one wave per (sequence, kv head, split of split_tokens
//    tokens); multi-split sequences write the per-split partial output, max
//    logit and exp-sum (the 256-token partitions and buffers of the PR #47361
//    report's benchmark snippet) and a reduce kernel merges them;
//  * stream-K (the default): a persistent grid in which every wave takes an
//    equal, contiguous share of all (block, kv head) tiles of the batch,
//    ordered kv head, sequence, block, and runs it as one block pipeline
//    across the pairs it spans; a pair cut by a share boundary is finished by
//    a merge kernel. Ragged lengths then leave every wave the same work.
//
// Contraction mapping (per 16 tokens of a block; 16x16 fp32 MFMA results):
//   S[t][g] = sum_d K[t][d] q[g][d]: A = K tile (rows = tokens), B = q
//     (columns = query heads of the group, zero-padded to 16). Result lane
//     (g + 16*q4) holds S[4*q4 + r][g], r = 0..3.
//   O[d][g] += sum_t V[t][d] P[g][t]: A = V^T tile (rows = head dims),
//     B = P. B's lane layout for a 16-deep product equals S's result layout,
//     so P stays in its registers.
// Any permutation of a reduction index is valid when both operands agree: the
// d-order of the K operand is chosen so each lane's 16-byte K load is
// contiguous in the cache and one wave load instruction covers 1 KiB
// contiguous. V loads of one d-tile cover 512 B (bf16), 1 KiB (f32) or
// 256 B (fp8) contiguous.
//
// Softmax runs in the log2 domain: z = S*(scale*log2 e [*k_scale]) +
// slope*log2 e*(t - (L-1)); p = exp2(z - m). The running max m is raised only
// when a block's max exceeds it by more than kRescaleSlack (so p <= 2^8) and
// the accumulator rescale is then done once for the whole wave; the result is
// the same softmax. Tokens t >= L in a sequence's last block get z = -inf by
// select and their V elements are zeroed by select (stale slots may hold NaN,
// and 0 * NaN would poison the sum).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_kernels.h"
#include "pa_sched.h"
#include "pa_wave.h"

namespace pa {

// ---------------------------------------------------------------------------
// Split grid: grid (ceil(num_kv_heads / kWaves), num_seqs, num_splits). The
// split index varies slowest, so every sequence's first split is dispatched
// before any second one: with ragged lengths the grid (sized by max_seq_len)
// ends in splits past most sequences' ends, which exit at once, instead of
// interleaving them with the work.
// ---------------------------------------------------------------------------

template <typename P, int D, int NB, bool ALIBI>
__global__ void __launch_bounds__(kWaves * 64)
pa_split_kernel(const DecodeArgs a) {
  split_unit<P, D, NB, ALIBI>(a, blockIdx.z, blockIdx.x, blockIdx.y);
}

// Merge of the split partials: grid (num_heads, num_seqs), 64 threads.
template <typename OutElem, int D>
__global__ void __launch_bounds__(64)
pa_split_reduce_kernel(const DecodeArgs a) {
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int lane = threadIdx.x;
  const int L = clamp_len(a.seq_lens[seq], a.max_seq_len);
  const int n = (L + a.split_tokens - 1) / a.split_tokens;
  if (n <= 1) return;
  const int64_t row0 = ((int64_t)seq * a.num_heads + h) * a.num_splits;
  const float* ml = a.max_logits + row0;
  const float* es = a.exp_sums + row0;
  float big_m = kNegInf;
  for (int p = lane; p < n; p += 64) big_m = fmaxf(big_m, ml[p]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) big_m = fmaxf(big_m, __shfl_xor(big_m, off, 64));
  float tot = 0.f;
  for (int p = lane; p < n; p += 64) tot += es[p] * fast_exp2((ml[p] - big_m) * kLog2e);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off, 64);
  constexpr int kPer = D >= 64 ? D / 64 : 1;     // head elements per lane
  if (lane * kPer >= D) return;                  // D = 32: lanes 32..63 idle
  float acc[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) acc[k] = 0.f;
  const float* tmp = a.tmp_out + row0 * D + lane * kPer;
  // Eight splits per step, their loads in flight together (index clamped,
  // weight zeroed past n); the valid splits add in order p = 0, 1, ...
  constexpr int kU = 8;
  for (int p0 = 0; p0 < n; p0 += kU) {
    float wgt[kU], part[kU][kPer];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int p = min(p0 + u, n - 1);
      wgt[u] = es[p] * fast_exp2((ml[p] - big_m) * kLog2e) * (float)(p0 + u < n);
#pragma unroll
      for (int k = 0; k < kPer; ++k) part[u][k] = tmp[(int64_t)p * D + k];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int k = 0; k < kPer; ++k) acc[k] += wgt[u] * part[u][k];
  }
  const float inv = 1.f / tot;
  OutElem* out = reinterpret_cast<OutElem*>(a.out) + ((int64_t)seq * a.num_heads + h) * D + lane * kPer;
#pragma unroll
  for (int k = 0; k < kPer; ++k) out[k] = from_f32<OutElem>(acc[k] * inv);
}

// ---------------------------------------------------------------------------
// Stream-K: grid (num_workgroups), kWaves waves each; wave w of W in total
// owns tiles [w*U, min(total, (w+1)*U)) with U = ceil(total / W) of the
// total = num_kv_heads * T tiles, T = sum_s ceil(L_s / BS) (one tile per
// BS-token block), ordered
// (kv head, sequence, block). Pair p = kvh*S + s cut into several segments
// writes segment partials at slot p + w (unique: both p and w grow along the
// order) and records its first and last wave in seg_meta[p].
// ---------------------------------------------------------------------------


// Register-set copy: arrays element by element, anything else by assignment.
template <typename T>
__device__ __forceinline__ void assign(T& d, const T& s) { d = s; }
template <typename T, int N>
__device__ __forceinline__ void assign(T (&d)[N], const T (&s)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) assign(d[i], s[i]);
}

// One wave's stream-K share as a single block pipeline. The (sequence, kv
// head) pairs of the share follow one another without a pause: the next
// pair's q rows and first 64 table entries are loaded when the current pair
// starts, and its first block's K/V loads are issued before the current
// pair's last block is computed, the way a pair's own next block is.
template <typename P, int D, bool ALIBI>
__device__ __forceinline__ void streamk_share(const DecodeArgs& a, int w, int seq, int kvh, int blk, int64_t units,
                                              float v_scale) {
  using OutElem = typename P::OutElem;
  using KRegs = typename P::KRegs;
  using VRegs = typename P::VRegs;
  constexpr int kBS = P::kBS;
  constexpr int kShift = kBS == 32 ? 5 : 4;
  const int S = a.num_seqs;
  const unsigned top = (unsigned)(a.num_blocks - 1);

  struct Seg {   // blocks [b0, b1) of the pair (seq, kvh); nbs blocks of L tokens in all
    int seq, kvh, b0, b1, nbs, L;
  };
  auto make_seg = [&](int s, int k, int b0, int64_t left) {
    Seg g;
    g.seq = s;
    g.kvh = k;
    g.b0 = b0;
    g.L = clamp_len(a.seq_lens[s], a.max_seq_len);
    g.nbs = blocks_of<kBS>(g.L);
    g.b1 = b0 + (int)min((int64_t)(g.nbs - b0), left);
    return g;
  };

  WaveAttn<P, D, 1, ALIBI> wa;
  wa.init_lane(a);
  const int lane = wa.lane;

  Seg cur = make_seg(seq, kvh, blk, units);
  int64_t left = units - (cur.b1 - cur.b0);   // units of the share after cur
  float sl;
  wa.load_pair_q(a, cur.seq, cur.kvh, wa.q, sl);
  wa.reset(sl);
  const int32_t* trow = a.block_tables + (int64_t)cur.seq * a.max_blocks_per_seq;
  int chunk = cur.b0;   // lane i of tbl holds the entry of block chunk + i
  int tbl = trow[min(chunk + lane, cur.b1 - 1)];

  // The share's next pair, prefetched.
  Seg nx{};
  bool has_nx = false;
  typename P::QRegs qn;
  float sln = 0.f;
  int tbl_n = 0;
  auto prefetch = [&]() {
    has_nx = false;
    if (left <= 0) return;
    int s = cur.seq, k = cur.kvh;
    do {
      if (++s == S) {
        s = 0;
        ++k;
      }
    } while (k < a.num_kv_heads && clamp_len(a.seq_lens[s], a.max_seq_len) == 0);
    if (k >= a.num_kv_heads) return;   // only with inconsistent inputs
    nx = make_seg(s, k, 0, left);
    has_nx = true;
    wa.load_pair_q(a, nx.seq, nx.kvh, qn, sln);
    tbl_n = a.block_tables[(int64_t)nx.seq * a.max_blocks_per_seq + min(lane, nx.b1 - 1)];
  };
  prefetch();

  const char* kbase = reinterpret_cast<const char*>(a.key_cache);
  const char* vbase = reinterpret_cast<const char*>(a.value_cache);
  auto load_block = [&](int k, unsigned phys, KRegs (&kr)[1], VRegs (&vr)[1]) {
    phys = phys < top ? phys : top;
    const int64_t off = (int64_t)phys * a.k_block_stride_bytes;   // K and V tiles share strides
    P::load_k(kbase + (int64_t)k * a.k_head_stride_bytes + off, wa.lo, kr[0]);
    P::load_v(vbase + (int64_t)k * a.v_head_stride_bytes + off, wa.lo, vr[0]);
  };
  auto issue_cur = [&](int g, KRegs (&kr)[1], VRegs (&vr)[1]) {   // block g of cur
    if (g - chunk >= 64) {
      chunk += 64;
      tbl = trow[min(chunk + lane, cur.b1 - 1)];
    }
    load_block(cur.kvh, (unsigned)__builtin_amdgcn_readlane(tbl, g - chunk), kr, vr);
  };

  int last_blk = (cur.L - 1) >> kShift;
  int tail = cur.L - (last_blk << kShift);   // valid slots in the last block, 1..kBS
  int g = cur.b0;
  // Computes block g of cur (in kr/vr) after issuing its successor into
  // kn/vn; false once the share is done.
  auto step = [&](KRegs (&kr)[1], VRegs (&vr)[1], KRegs (&kn)[1], VRegs (&vn)[1]) -> bool {
    const bool more = g + 1 < cur.b1;
    if (more)
      issue_cur(g + 1, kn, vn);
    else if (has_nx)
      load_block(nx.kvh, (unsigned)__builtin_amdgcn_readlane(tbl_n, 0), kn, vn);
    wa.consume(kr, vr, g, 1, cur.L, last_blk, tail);
    if (more) {
      ++g;
      return true;
    }
    wa.finish();
    const int64_t pair = (int64_t)cur.kvh * S + cur.seq;
    const int64_t h0 = (int64_t)cur.seq * a.num_heads + cur.kvh * a.group;
    if (cur.b0 == 0 && cur.b1 == cur.nbs) {
      wa.store_rows(reinterpret_cast<OutElem*>(a.out) + h0 * D, D, v_scale);
    } else {
      const int64_t slot = pair + w;
      wa.store_rows(a.seg_out + slot * a.group * D, D, v_scale);
      if (wa.active && wa.q4 == 0) {
        a.seg_max[slot * a.group + (lane & 15)] = wa.m;
        a.seg_sum[slot * a.group + (lane & 15)] = wa.lsum;
      }
    }
    if (lane == 0) {
      if (cur.b0 == 0) a.seg_meta[2 * pair] = w;
      if (cur.b1 == cur.nbs) a.seg_meta[2 * pair + 1] = w;
    }
    if (!has_nx) return false;
    // On to the prefetched pair, whose first block is already in kn/vn.
    cur = nx;
    left -= cur.b1 - cur.b0;
    assign(wa.q, qn);
    wa.reset(sln);
    trow = a.block_tables + (int64_t)cur.seq * a.max_blocks_per_seq;
    chunk = 0;
    tbl = tbl_n;
    last_blk = (cur.L - 1) >> kShift;
    tail = cur.L - (last_blk << kShift);
    g = 0;
    prefetch();
    return true;
  };

  KRegs ka[1], kb[1];
  VRegs va[1], vb[1];
  issue_cur(cur.b0, ka, va);
  while (step(ka, va, kb, vb) && step(kb, vb, ka, va)) {
  }
}

template <typename P, int D, int NB, bool ALIBI>
__global__ void __launch_bounds__(kWaves * 64)
pa_streamk_kernel(const DecodeArgs a) {
  using OutElem = typename P::OutElem;
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = gridDim.x * kWaves;
  const int S = a.num_seqs;

  constexpr int kBS = P::kBS;
  int bsum = 0;
  const int T = count_blocks<kBS>(a, lane, bsum);
  const int64_t total = (int64_t)a.num_kv_heads * T;
  if (total == 0) return;
  const int64_t U = (total + nwaves - 1) / nwaves;
  const int64_t u0 = (int64_t)w * U;
  const int64_t u1 = min(total, u0 + U);
  if (u0 >= u1) return;

  // Locate tile u0: kv head, then the sequence whose block range holds r.
  int kvh = (int)(u0 / T);
  const int r = (int)(u0 - (int64_t)kvh * T);
  int seq = 0, blk = 0;
  locate_block<kBS>(a, lane, r, bsum, seq, blk);

  float v_scale = 1.f;
  if (a.v_scale) v_scale = *a.v_scale;
  if constexpr (NB == 1) {
    streamk_share<P, D, ALIBI>(a, w, seq, kvh, blk, u1 - u0, v_scale);
  } else {
    // Several blocks per iteration: one pair at a time.
    int64_t u = u0;
    while (true) {
      const int L = clamp_len(a.seq_lens[seq], a.max_seq_len);
      const int nbs = blocks_of<P::kBS>(L);
      const int n = (int)min((int64_t)(nbs - blk), u1 - u);
      WaveAttn<P, D, NB, ALIBI> wa;
      wa.begin(a, seq, kvh);
      const char* kh = reinterpret_cast<const char*>(a.key_cache) + (int64_t)kvh * a.k_head_stride_bytes;
      const char* vh = reinterpret_cast<const char*>(a.value_cache) + (int64_t)kvh * a.v_head_stride_bytes;
      wa.run(a, kh, vh, a.block_tables + (int64_t)seq * a.max_blocks_per_seq, blk, blk + n, L);
      wa.finish();
      const int64_t pair = (int64_t)kvh * S + seq;
      const int64_t h0 = (int64_t)seq * a.num_heads + kvh * a.group;
      if (blk == 0 && n == nbs) {
        wa.store_rows(reinterpret_cast<OutElem*>(a.out) + h0 * D, D, v_scale);
      } else {
        const int64_t slot = pair + w;
        wa.store_rows(a.seg_out + slot * a.group * D, D, v_scale);
        if (wa.active && wa.q4 == 0) {
          a.seg_max[slot * a.group + (lane & 15)] = wa.m;
          a.seg_sum[slot * a.group + (lane & 15)] = wa.lsum;
        }
      }
      if (lane == 0) {
        if (blk == 0) a.seg_meta[2 * pair] = w;
        if (blk + n == nbs) a.seg_meta[2 * pair + 1] = w;
      }
      u += n;
      if (u >= u1) break;
      // Next pair with at least one block (one exists: u < u1 <= total; the
      // kv-head bound only guards against inconsistent inputs).
      blk = 0;
      do {
        if (++seq == S) {
          seq = 0;
          ++kvh;
        }
      } while (kvh < a.num_kv_heads && clamp_len(a.seq_lens[seq], a.max_seq_len) == 0);
      if (kvh >= a.num_kv_heads) break;
    }
  }
}

// Merge of stream-K segments and zero rows of empty sequences: grid
// (num_kv_heads, num_seqs), 256 threads; one (sequence, kv head) pair each.
template <typename OutElem, int D>
__global__ void __launch_bounds__(256)
pa_streamk_reduce_kernel(const DecodeArgs a) {
  const int kvh = blockIdx.x;
  const int seq = blockIdx.y;
  const int G = a.group;
  const int L = clamp_len(a.seq_lens[seq], a.max_seq_len);
  OutElem* out = reinterpret_cast<OutElem*>(a.out) + ((int64_t)seq * a.num_heads + kvh * G) * D;
  if (L == 0) {
    for (int e = threadIdx.x; e < G * D; e += 256) out[e] = from_f32<OutElem>(0.f);
    return;
  }
  const int64_t pair = (int64_t)kvh * a.num_seqs + seq;
  const int nwaves = a.streamk_workgroups * kWaves;
  const int w0 = max(0, a.seg_meta[2 * pair]);
  const int w1 = min(nwaves - 1, a.seg_meta[2 * pair + 1]);
  if (w0 >= w1) return;                       // single segment: written directly
  for (int e = threadIdx.x; e < G * (D / 4); e += 256) {
    const int g = e / (D / 4);
    const int d4 = e - g * (D / 4);
    float big_m = kNegInf;
    for (int w = w0; w <= w1; ++w) big_m = fmaxf(big_m, a.seg_max[(pair + w) * G + g]);
    float tot = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int w = w0; w <= w1; ++w) {
      const int64_t slot = pair + w;
      const float f = fast_exp2(a.seg_max[slot * G + g] - big_m) * a.seg_sum[slot * G + g];
      tot += f;
      acc += f * *reinterpret_cast<const f32x4*>(a.seg_out + (slot * G + g) * D + 4 * d4);
    }
    store4(out + (int64_t)g * D + 4 * d4, acc * (1.f / tot));
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers.
// ---------------------------------------------------------------------------

template <typename P, int D, int NB, bool ALIBI>
static hipError_t launch_mode(const DecodeArgs& a, hipStream_t stream, const LaunchHooks& hooks) {
  using OutElem = typename P::OutElem;
  hipError_t err;
  if (hooks.before_partition) hooks.before_partition(stream);
  if (a.streamk_workgroups > 0) {
    hipLaunchKernelGGL((pa_streamk_kernel<P, D, NB, ALIBI>), dim3(a.streamk_workgroups), dim3(kWaves * 64), 0,
                       stream, a);
  } else {
    hipLaunchKernelGGL((pa_split_kernel<P, D, NB, ALIBI>),
                       dim3((a.num_kv_heads + kWaves - 1) / kWaves, a.num_seqs, a.num_splits), dim3(kWaves * 64), 0,
                       stream, a);
  }
  err = hipGetLastError();
  if (hooks.after_partition) hooks.after_partition(stream);
  if (err != hipSuccess) return err;
  if (a.streamk_workgroups > 0) {
    if (hooks.before_reduce) hooks.before_reduce(stream);
    hipLaunchKernelGGL((pa_streamk_reduce_kernel<OutElem, D>), dim3(a.num_kv_heads, a.num_seqs), dim3(256), 0,
                       stream, a);
  } else {
    if (a.num_splits <= 1 || a.first_block) return hipSuccess;   // shared-prefix mode merges elsewhere
    if (hooks.before_reduce) hooks.before_reduce(stream);
    hipLaunchKernelGGL((pa_split_reduce_kernel<OutElem, D>), dim3(a.num_heads, a.num_seqs), dim3(64), 0, stream,
                       a);
  }
  err = hipGetLastError();
  if (hooks.after_reduce) hooks.after_reduce(stream);
  return err;
}

template <typename P, int D, int NB>
static hipError_t launch_alibi(const DecodeArgs& a, hipStream_t stream, const LaunchHooks& hooks) {
  return a.alibi_slopes ? launch_mode<P, D, NB, true>(a, stream, hooks)
                        : launch_mode<P, D, NB, false>(a, stream, hooks);
}

template <int BS>
static hipError_t launch_decode_bs(const DecodeArgs& a, int kind, hipStream_t stream, const LaunchHooks& hooks) {
  // A 32-token block is already two 16-row sub-tiles: one block per issue.
  constexpr int nb_f32 = BS == 32 ? 1 : PA_NB_F32;
  constexpr int nb_bf16 = BS == 32 ? 1 : PA_NB_BF16;
  constexpr int nb_fp8 = BS == 32 ? 1 : PA_NB_FP8;
  switch (kind * 1000 + a.head_size) {
    case KIND_F32 * 1000 + 32: return launch_alibi<PolicyF32<32, BS>, 32, nb_f32>(a, stream, hooks);
    case KIND_F32 * 1000 + 64: return launch_alibi<PolicyF32<64, BS>, 64, nb_f32>(a, stream, hooks);
    case KIND_F32 * 1000 + 128: return launch_alibi<PolicyF32<128, BS>, 128, nb_f32>(a, stream, hooks);
    case KIND_BF16 * 1000 + 32: return launch_alibi<PolicyBf16<32, BS>, 32, nb_bf16>(a, stream, hooks);
    case KIND_BF16 * 1000 + 64: return launch_alibi<PolicyBf16<64, BS>, 64, nb_bf16>(a, stream, hooks);
    case KIND_BF16 * 1000 + 128: return launch_alibi<PolicyBf16<128, BS>, 128, nb_bf16>(a, stream, hooks);
    case KIND_FP8 * 1000 + 32: return launch_alibi<PolicyFp8<32, BS>, 32, nb_fp8>(a, stream, hooks);
    case KIND_FP8 * 1000 + 64: return launch_alibi<PolicyFp8<64, BS>, 64, nb_fp8>(a, stream, hooks);
    case KIND_FP8 * 1000 + 128: return launch_alibi<PolicyFp8<128, BS>, 128, nb_fp8>(a, stream, hooks);
    case KIND_FP8MX * 1000 + 32: return launch_alibi<PolicyFp8Mx<32, BS>, 32, 1>(a, stream, hooks);
    case KIND_FP8MX * 1000 + 64: return launch_alibi<PolicyFp8Mx<64, BS>, 64, 1>(a, stream, hooks);
    case KIND_FP8MX * 1000 + 128: return launch_alibi<PolicyFp8Mx<128, BS>, 128, 1>(a, stream, hooks);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs& a, int kind, hipStream_t stream, const LaunchHooks& hooks) {
  switch (a.block_size) {
    case 16: return launch_decode_bs<16>(a, kind, stream, hooks);
    case 32: return launch_decode_bs<32>(a, kind, stream, hooks);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
