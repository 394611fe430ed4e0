// Shared-prefix paged decode for gfx950: when several sequences map their
// first blocks to the same physical blocks (a forked prompt: parallel
// sampling, beam search, a common system prompt — the sharing of "vLLM 0.25.0
// 解读" §1), each shared K/V tile is read once for all of them.
//
// Two launches:
//  1. one kernel with two kinds of workgroups:
//     - prefix items, one wave per (group chunk, kv head, prefix split). The
//       query heads of up to 16*NCT/G members of a group form NCT tiles of
//       16 MFMA columns; each K and V tile of the shared prefix is loaded
//       once and multiplied against every column tile. Writes per (member,
//       head, split) partials (normalised output, max logit, exp-sum);
//     - split-grid items over each sequence's own blocks after the prefix
//       (DecodeArgs::first_block), always writing partials;
//  2. merge: log-sum-exp combination of the prefix and suffix partials of
//     every (sequence, head) into out.
// Prefix blocks hold only valid tokens (the prefix is whole blocks every
// member fills), so no tail masking happens in the prefix kernel. Softmax
// bookkeeping is the decode kernel's: log2 domain, lazily raised per-column
// running max.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_kernels.h"
#include "pa_wave.h"

namespace pa {

namespace {

template <typename P, int D, int NCT, bool ALIBI>
struct GroupAttn {
  static constexpr int kDt = P::kDt;
  static constexpr int kBS = P::kBS;
  static constexpr int kSub = P::kSub;
  typename P::QRegs q[NCT];
  typename P::Lane lo;
  f32x4 o[NCT][kDt];
  float m[NCT], m_true[NCT], lsum[NCT];
  float slope2[NCT], lane_bias[NCT][4];
  int col_seq[NCT], col_head[NCT];
  bool active[NCT];
  float c;
  int lane, q4;

  // Column 16*t + (lane & 15) of tile t is member (col / G), head g = col % G
  // of kv head kvh; columns past the chunk's members are zero and inactive.
  __device__ void begin(const SharedArgs& s, const int32_t* members, int count, int kvh) {
    const DecodeArgs& a = s.d;
    lane = threadIdx.x & 63;
    q4 = lane >> 4;
    lo = P::lane_offsets(lane);
    float k_scale = 1.f;
    if (a.k_scale) k_scale = *a.k_scale;
    c = a.scale * kLog2e * k_scale;
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
      const int col = 16 * t + (lane & 15);
      const int mi = col / a.group;
      const int g = col - mi * a.group;
      active[t] = mi < count;
      col_seq[t] = min(max(members[active[t] ? mi : 0], 0), a.num_seqs - 1);
      col_head[t] = kvh * a.group + g;
      const auto* qh = reinterpret_cast<const typename P::QElem*>(a.query) +
                       ((int64_t)col_seq[t] * a.num_heads + col_head[t]) * D;
      P::load_q(qh, active[t], q4, q[t]);
      slope2[t] = 0.f;
      if constexpr (ALIBI) {
        const int L = clamp_len(a.seq_lens[col_seq[t]], a.max_seq_len);
        if (active[t]) slope2[t] = a.alibi_slopes[col_head[t]] * kLog2e;
#pragma unroll
        for (int r = 0; r < 4; ++r) lane_bias[t][r] = slope2[t] * (float)(tile_token<kBS>(0, q4, r) - (L - 1));
      }
      m[t] = m_true[t] = kNegInf;
      lsum[t] = 0.f;
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // Phase by phase over the column tiles (all q.K^T products, then all
  // maxima, one uniform test for any rescale, then all P.V), so the tiles'
  // independent MFMA chains interleave instead of running one tile at a time
  // between branches. Each tile's rescale decision is the same as tile by tile.
  __device__ void consume(const typename P::KRegs& kr, typename P::VRegs& vr, int blk) {
    P::prepare_v(vr);
    f32x4 z[NCT][kSub];
    float mx[NCT];
#pragma unroll
    for (int t = 0; t < NCT; ++t)
#pragma unroll
      for (int st = 0; st < kSub; ++st) {
        const f32x4 sc = P::qk(kr, q[t], st);
        if constexpr (ALIBI) {
          const float base = (float)(blk * kBS + 8 * st);
#pragma unroll
          for (int r = 0; r < 4; ++r) z[t][st][r] = fmaf(sc[r], c, fmaf(slope2[t], base, lane_bias[t][r]));
        } else {
          z[t][st] = sc * c;
        }
      }
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
      float v = max4(z[t][0]);
#pragma unroll
      for (int st = 1; st < kSub; ++st) v = fmaxf(v, max4(z[t][st]));
      mx[t] = quad_max(v);
      m_true[t] = fmaxf(m_true[t], mx[t]);
    }
    if constexpr (Fp8Math<P>::value) {
#pragma unroll
      for (int t = 0; t < NCT; ++t) fp8_block_update<P>(vr, z[t], mx[t], m[t], lsum[t], o[t]);
    } else {
      bool need = false;
#pragma unroll
      for (int t = 0; t < NCT; ++t) need = need || mx[t] > m[t] + kRescaleSlack;
      if (wave_any(need)) {
#pragma unroll
        for (int t = 0; t < NCT; ++t) {
          if (wave_any(mx[t] > m[t] + kRescaleSlack)) {
            const float m_new = fmaxf(m[t], mx[t]);
            const float alpha = fast_exp2(m[t] - m_new);
            m[t] = m_new;
            lsum[t] *= alpha;
#pragma unroll
            for (int dt = 0; dt < kDt; ++dt) o[t][dt] *= alpha;
          }
        }
      }
#pragma unroll
      for (int t = 0; t < NCT; ++t)
#pragma unroll
        for (int st = 0; st < kSub; ++st) {
          f32x4 p;
#pragma unroll
          for (int r = 0; r < 4; ++r) p[r] = fast_exp2(z[t][st][r] - m[t]);
          lsum[t] += (p[0] + p[1]) + (p[2] + p[3]);
          P::pv(vr, p, o[t], st);
        }
    }
  }

  // Blocks [b0, b1) of the shared table row. Table entries are read 64 at a
  // time into one VGPR (lane i = entry base + i) and broadcast per block; the
  // asm statement consumes a fresh window at once so that its wait happens
  // once per 64 blocks rather than before every block's loads. The next
  // block's K/V loads are in flight while the current block is computed
  // (four query tiles make the compute long enough to hide behind them).
  __device__ void run(const DecodeArgs& a, const char* kh, const char* vh, const int32_t* table_row, int b0,
                      int b1) {
    const unsigned top = (unsigned)(a.num_blocks - 1);
    int base = b0;
    int win = (b0 + lane < b1) ? table_row[b0 + lane] : 0;
    asm volatile("" ::"v"(win));
    auto addr = [&](int blk) -> int64_t {
      if (blk - base >= 64) {
        base += 64;
        win = (base + lane < b1) ? table_row[base + lane] : 0;
        asm volatile("" ::"v"(win));
      }
      unsigned phys = (unsigned)__builtin_amdgcn_readlane(win, blk - base);
      phys = phys < top ? phys : top;
      return (int64_t)phys * a.k_block_stride_bytes;
    };
    typename P::KRegs ka, kb;
    typename P::VRegs va, vb;
    auto issue = [&](int blk, typename P::KRegs& kr, typename P::VRegs& vr) {
      const int64_t off = addr(blk);
      P::load_k(kh + off, lo, kr);
      P::load_v(vh + off, lo, vr);
    };
    // Every load in the loop is unconditional (past the end it re-reads the
    // last block, whose data is still in L2), so each wait covers exactly the
    // block it needs; only two consume sites keep the register count down.
    issue(b0, ka, va);
    issue(min(b0 + 1, b1 - 1), kb, vb);
    for (int i = b0;; i += 2) {
      consume(ka, va, i);
      if (i + 1 >= b1) break;
      issue(min(i + 2, b1 - 1), ka, va);
      consume(kb, vb, i + 1);
      if (i + 2 >= b1) break;
      issue(min(i + 3, b1 - 1), kb, vb);
    }
#pragma unroll
    for (int t = 0; t < NCT; ++t) lsum[t] = quad_sum(lsum[t]);
  }
};

// One (group chunk, group of kWaves kv heads, prefix split) item.
template <typename P, int D, int NCT, bool ALIBI>
__device__ __forceinline__ void prefix_unit(const SharedArgs& s, int group, int chunk, int kvh_group, int split) {
  const DecodeArgs& a = s.d;
  const int kvh = kvh_group * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (group >= s.num_groups || kvh >= a.num_kv_heads) return;
  // Group offsets and member ids are the caller's contract; clamp them so a
  // violation cannot address memory outside the arrays.
  const int g0 = min(max(s.group_start[group], 0), s.num_members);
  const int g1 = min(max(s.group_start[group + 1], g0), s.num_members);
  const int m0 = g0 + chunk * s.members_per_chunk;
  if (m0 >= g1) return;
  const int count = min(s.members_per_chunk, g1 - m0);
  const int pblocks = min(max(s.group_prefix_blocks[group], 0), min(a.max_blocks_per_seq, a.max_first_block));
  const int b0 = split * s.prefix_split_blocks;
  const int b1 = min(pblocks, b0 + s.prefix_split_blocks);
  if (b0 >= b1) return;
  const int32_t* members = s.group_seqs + m0;

  GroupAttn<P, D, NCT, ALIBI> w;
  w.begin(s, members, count, kvh);
  const char* kh = reinterpret_cast<const char*>(a.key_cache) + (int64_t)kvh * a.k_head_stride_bytes;
  const char* vh = reinterpret_cast<const char*>(a.value_cache) + (int64_t)kvh * a.v_head_stride_bytes;
  w.run(a, kh, vh, a.block_tables + (int64_t)w.col_seq[0] * a.max_blocks_per_seq, b0, b1);

  float v_scale = 1.f;
  if (a.v_scale) v_scale = *a.v_scale;
#pragma unroll
  for (int t = 0; t < NCT; ++t) {
    if (!w.active[t]) continue;
    const int64_t row = ((int64_t)w.col_seq[t] * a.num_heads + w.col_head[t]) * s.max_prefix_splits + split;
    float* dst = s.pre_out + row * D + 4 * w.q4;
    const float f = v_scale / w.lsum[t];
#pragma unroll
    for (int dt = 0; dt < P::kDt; ++dt) *reinterpret_cast<f32x4*>(dst + 16 * dt) = w.o[t][dt] * f;
    if (w.q4 == 0) {
      s.pre_max[row] = w.m_true[t] * kLn2;
      s.pre_sum[row] = w.lsum[t] * fast_exp2(w.m[t] - w.m_true[t]);
    }
  }
}

// One launch for both parts, so the sequences' own blocks fill the machine
// around the prefix work: workgroups [0, prefix_wgs) are prefix items
// (group, chunk, kv-head group, split), the rest split-grid items (split,
// kv-head group, sequence) over each sequence's blocks after its prefix.
template <typename P, int D, int NCT, bool ALIBI>
__global__ void __launch_bounds__(kWaves * 64) pa_shared_kernel(const SharedArgs s, int prefix_wgs) {
  const int kv_groups = (s.d.num_kv_heads + kWaves - 1) / kWaves;
  int x = blockIdx.x;
  if (x < prefix_wgs) {
    const int split = x % s.max_prefix_splits;
    x /= s.max_prefix_splits;
    const int kvg = x % kv_groups;
    x /= kv_groups;
    prefix_unit<P, D, NCT, ALIBI>(s, x / s.max_chunks, x % s.max_chunks, kvg, split);
  } else {
    // Split index slowest: split 0 (the first tokens after each sequence's
    // prefix, where every grouped sequence's own tokens start) is dispatched
    // right after the prefix items; the higher splits, empty unless a
    // sequence is long past its prefix, come last and mostly exit at once.
    x -= prefix_wgs;
    const int per_split = kv_groups * s.d.num_seqs;
    const int split = x / per_split;
    x -= split * per_split;
    split_unit<P, D, 1, ALIBI>(s.d, split, x % kv_groups, x / kv_groups);
  }
}

// Merge of prefix and suffix partials: grid (num_kv_heads, num_seqs), 256
// threads; thread e covers 4 consecutive dims (16-byte loads) of query head
// kvh*G + e / (D/4).
template <typename OutElem, int D>
__global__ void __launch_bounds__(256) pa_shared_merge_kernel(const SharedArgs s, const int32_t* seq_prefix_blocks) {
  const DecodeArgs& a = s.d;
  const int kvh = blockIdx.x;
  const int seq = blockIdx.y;
  const int G = a.group;
  const int L = clamp_len(a.seq_lens[seq], a.max_seq_len);
  OutElem* out = reinterpret_cast<OutElem*>(a.out) + ((int64_t)seq * a.num_heads + kvh * G) * D;
  const int first = min(max(seq_prefix_blocks[seq], 0), min(L / a.block_size, a.max_first_block));
  const int n_pre = first > 0 ? (first + s.prefix_split_blocks - 1) / s.prefix_split_blocks : 0;
  const int t0 = first * a.block_size;
  const int n_suf = L > t0 ? (L - t0 + a.split_tokens - 1) / a.split_tokens : 0;
  const int n = n_pre + n_suf;
  for (int e = threadIdx.x; e < G * (D / 4); e += 256) {
    const int g = e / (D / 4);
    const int d4 = e - g * (D / 4);
    OutElem* dst = out + (int64_t)g * D + 4 * d4;
    if (n == 0) {
      store4(dst, f32x4{0.f, 0.f, 0.f, 0.f});
      continue;
    }
    const int64_t row = (int64_t)seq * a.num_heads + kvh * G + g;
    const int64_t pre_row = row * s.max_prefix_splits;
    const int64_t suf_row = row * a.num_splits;
    auto ml = [&](int i) { return i < n_pre ? s.pre_max[pre_row + i] : a.max_logits[suf_row + i - n_pre]; };
    auto es = [&](int i) { return i < n_pre ? s.pre_sum[pre_row + i] : a.exp_sums[suf_row + i - n_pre]; };
    float big_m = kNegInf;
    for (int i = 0; i < n; ++i) big_m = fmaxf(big_m, ml(i));
    float tot = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < n; ++i) {
      const float wgt = es(i) * fast_exp2((ml(i) - big_m) * kLog2e);
      tot += wgt;
      const float* src = i < n_pre ? s.pre_out + (pre_row + i) * D : a.tmp_out + (suf_row + i - n_pre) * D;
      acc += wgt * *reinterpret_cast<const f32x4*>(src + 4 * d4);
    }
    store4(dst, acc * (1.f / tot));
  }
}

template <typename P, int D, int NCT>
hipError_t launch_prefix(const SharedArgs& s, hipStream_t stream) {
  const int64_t kv_groups = (s.d.num_kv_heads + kWaves - 1) / kWaves;
  const int64_t prefix_wgs = (int64_t)s.num_groups * s.max_chunks * kv_groups * s.max_prefix_splits;
  const int64_t suffix_wgs = (int64_t)s.d.num_splits * kv_groups * s.d.num_seqs;
  if (prefix_wgs + suffix_wgs >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(prefix_wgs + suffix_wgs));
  if (s.d.alibi_slopes)
    hipLaunchKernelGGL((pa_shared_kernel<P, D, NCT, true>), grid, dim3(kWaves * 64), 0, stream, s, (int)prefix_wgs);
  else
    hipLaunchKernelGGL((pa_shared_kernel<P, D, NCT, false>), grid, dim3(kWaves * 64), 0, stream, s, (int)prefix_wgs);
  return hipGetLastError();
}

template <typename P, int D>
hipError_t launch_prefix_nct(const SharedArgs& s, int nct, hipStream_t stream) {
  switch (nct) {
    case 1: return launch_prefix<P, D, 1>(s, stream);
    case 2: return launch_prefix<P, D, 2>(s, stream);
    default:
      if constexpr (max_column_tiles(sizeof(typename P::QElem), P::kKvElemBytes, D, P::kBS) >= 4)
        return launch_prefix<P, D, 4>(s, stream);
      return hipErrorInvalidValue;
  }
}

}  // namespace

template <int BS>
hipError_t launch_shared_main(const SharedArgs& s, int kind, int column_tiles, hipStream_t stream) {
  switch (kind * 1000 + s.d.head_size) {
    case KIND_F32 * 1000 + 32: return launch_prefix_nct<PolicyF32<32, BS>, 32>(s, column_tiles, stream);
    case KIND_F32 * 1000 + 64: return launch_prefix_nct<PolicyF32<64, BS>, 64>(s, column_tiles, stream);
    case KIND_F32 * 1000 + 128: return launch_prefix_nct<PolicyF32<128, BS>, 128>(s, column_tiles, stream);
    case KIND_BF16 * 1000 + 32: return launch_prefix_nct<PolicyBf16<32, BS>, 32>(s, column_tiles, stream);
    case KIND_BF16 * 1000 + 64: return launch_prefix_nct<PolicyBf16<64, BS>, 64>(s, column_tiles, stream);
    case KIND_BF16 * 1000 + 128: return launch_prefix_nct<PolicyBf16<128, BS>, 128>(s, column_tiles, stream);
    case KIND_FP8 * 1000 + 32: return launch_prefix_nct<PolicyFp8<32, BS>, 32>(s, column_tiles, stream);
    case KIND_FP8 * 1000 + 64: return launch_prefix_nct<PolicyFp8<64, BS>, 64>(s, column_tiles, stream);
    case KIND_FP8 * 1000 + 128: return launch_prefix_nct<PolicyFp8<128, BS>, 128>(s, column_tiles, stream);
    case KIND_FP8MX * 1000 + 32: return launch_prefix_nct<PolicyFp8Mx<32, BS>, 32>(s, column_tiles, stream);
    case KIND_FP8MX * 1000 + 64: return launch_prefix_nct<PolicyFp8Mx<64, BS>, 64>(s, column_tiles, stream);
    case KIND_FP8MX * 1000 + 128: return launch_prefix_nct<PolicyFp8Mx<128, BS>, 128>(s, column_tiles, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_shared(const SharedArgs& s, int kind, int column_tiles, hipStream_t stream) {
  hipError_t err = s.d.block_size == 32 ? launch_shared_main<32>(s, kind, column_tiles, stream)
                   : s.d.block_size == 16 ? launch_shared_main<16>(s, kind, column_tiles, stream)
                                          : hipErrorInvalidValue;
  if (err != hipSuccess) return err;
  const dim3 grid(s.d.num_kv_heads, s.d.num_seqs);
  const bool f32 = kind == KIND_F32;
  switch (s.d.head_size) {
    case 32:
      if (f32) hipLaunchKernelGGL((pa_shared_merge_kernel<float, 32>), grid, dim3(256), 0, stream, s, s.d.first_block);
      else hipLaunchKernelGGL((pa_shared_merge_kernel<__bf16, 32>), grid, dim3(256), 0, stream, s, s.d.first_block);
      break;
    case 64:
      if (f32) hipLaunchKernelGGL((pa_shared_merge_kernel<float, 64>), grid, dim3(256), 0, stream, s, s.d.first_block);
      else hipLaunchKernelGGL((pa_shared_merge_kernel<__bf16, 64>), grid, dim3(256), 0, stream, s, s.d.first_block);
      break;
    default:
      if (f32) hipLaunchKernelGGL((pa_shared_merge_kernel<float, 128>), grid, dim3(256), 0, stream, s, s.d.first_block);
      else hipLaunchKernelGGL((pa_shared_merge_kernel<__bf16, 128>), grid, dim3(256), 0, stream, s, s.d.first_block);
  }
  return hipGetLastError();
}

}  // namespace pa
