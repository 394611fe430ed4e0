// Paged decode-attention kernels for gfx950 (CDNA4, wave64, MFMA).
//
// One workgroup of kWaves waves handles one (sequence, kv head, split): the
// split's KV blocks are dealt to the waves in groups of NB consecutive
// blocks; each wave keeps its own online-softmax state for all the query heads
// of the group (GQA packing) and streams K and V of each block straight from
// HBM into MFMA operand registers. A single traversal reads every K and V
// byte once, with K and V loads of a block in flight together; the pages'
// prior-art CUDA kernel walked the table twice, first for K and softmax, then
// for V, with a barrier in between (10100.com retirement article, §3).
//
// Contraction mapping (per 16-token block, all tiles 16x16 fp32 results):
//   logits S[t][g] = sum_d K[t][d] q[g][d]: A = K tile (rows = tokens),
//     B = q (columns = query heads of the group, zero-padded to 16).
//     Result lane (g + 16*q4) holds S[4*q4 + r][g], r = 0..3.
//   O[d][g] += sum_t V[t][d] P[g][t]: A = V^T tile (rows = head dims),
//     B = P. B's lane layout for a 16-deep product is exactly S's result
//     layout, so P never leaves its registers.
// Any permutation of the reduction index is valid when both operands agree;
// the d-order of the K operand is chosen so that each lane's 16-byte K load is
// contiguous in the cache and a wave's load instruction covers one contiguous
// run (1 KiB for bf16/f32, 1 KiB for fp8). V loads of one d-tile cover 512 B
// (bf16), 1 KiB (f32) or 256 B (fp8) contiguous.
//
// Softmax runs in the log2 domain: z = S * (scale*log2(e)[*k_scale]) +
// slope*log2(e)*(t - (L-1)); p = exp2(z - m). Tokens t >= L get z = -inf by
// select, and their V elements are zeroed by select (stale slots may hold
// NaN; 0 * NaN would poison the sum).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_kernels.h"

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 16;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float wave_max_across_quads(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

__device__ __forceinline__ float wave_sum_across_quads(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ s16x4 pack_bf16x4(f32x4 v) {
  bf16x4 b = __builtin_convertvector(v, bf16x4);
  return __builtin_bit_cast(s16x4, b);
}

// Two e4m3fn codes (bytes 0-1 or 2-3 of w) -> two bf16, exact (every e4m3
// value is a bf16 value); scale 1 so the conversion itself does not round.
template <bool HI>
__device__ __forceinline__ unsigned fp8x2_to_bf16x2(unsigned w) {
  bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(unsigned, r);
}

// ---------------------------------------------------------------------------
// Per-element-type policies: register shapes, loads and the two contractions.
// ---------------------------------------------------------------------------

// bf16 query, bf16 cache (x = 8): K chunk c = 8 consecutive d at one token.
template <int D>
struct PolicyBf16 {
  static constexpr int kElem = 2;
  static constexpr int kKLoads = D / 32;     // 16x16x32 steps, one uint4 each
  static constexpr int kDt = D / 16;         // d-tiles of the PV product
  static constexpr int NB = 4;               // blocks per wave iteration
  using KRegs = u32x4[kKLoads];
  using VRegs = u32x2[kDt];                  // 4 bf16 tokens of one d per tile
  using QRegs = bf16x8[kKLoads];
  using QElem = __bf16;
  using OutElem = __bf16;

  // lane l = i + 16*q4 loads chunk (4s + q4) at token i: uint4 index 64s + l.
  __device__ static void load_k(const char* blk, int lane, KRegs& k) {
    const u32x4* p = reinterpret_cast<const u32x4*>(blk);
#pragma unroll
    for (int s = 0; s < kKLoads; ++s) k[s] = __builtin_nontemporal_load(p + 64 * s + lane);
  }
  // V[d][t] rows of 16 tokens: lane (i + 16*q4) of tile dt reads tokens
  // 4*q4..4*q4+3 of d = 16*dt + i.
  __device__ static void load_v(const char* blk, int lane, VRegs& v) {
    const u32x2* p = reinterpret_cast<const u32x2*>(blk);
    const int i = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) v[dt] = __builtin_nontemporal_load(p + (16 * dt + i) * 4 + q4);
  }
  // q element order matching load_k: step s, lane quad q4 -> d = 8*(4s+q4) + u.
  __device__ static void load_q(const QElem* qh, bool active, int q4, QRegs& q) {
#pragma unroll
    for (int s = 0; s < kKLoads; ++s) {
      u32x4 w = {0, 0, 0, 0};
      if (active) w = *reinterpret_cast<const u32x4*>(qh + 8 * (4 * s + q4));
      q[s] = __builtin_bit_cast(bf16x8, w);
    }
  }
  __device__ static f32x4 qk(const KRegs& k, const QRegs& q) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kKLoads; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[s]), q[s], acc, 0, 0, 0);
    return acc;
  }
  // Zero V of tokens 4*q4+u >= nvalid (only called on a partial last block).
  __device__ static void mask_v(VRegs& v, int q4, int nvalid) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) {
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        unsigned x = v[dt][w];
        const int t0 = 4 * q4 + 2 * w;
        if (t0 >= nvalid) x &= 0xFFFF0000u;
        if (t0 + 1 >= nvalid) x &= 0x0000FFFFu;
        v[dt][w] = x;
      }
    }
  }
  __device__ static void pv(const VRegs& v, f32x4 p, f32x4 (&o)[kDt]) {
    const s16x4 pb = pack_bf16x4(p);
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, v[dt]), pb, o[dt], 0, 0, 0);
  }
};

// fp32 query, fp32 cache (x = 4): fp32 MFMA keeps full fp32 products.
template <int D>
struct PolicyF32 {
  static constexpr int kElem = 4;
  static constexpr int kKLoads = D / 16;     // uint4 = 4 d at one token
  static constexpr int kDt = D / 16;
  static constexpr int NB = 2;
  using KRegs = f32x4[kKLoads];
  using VRegs = f32x4[kDt];                  // 4 fp32 tokens of one d per tile
  using QRegs = f32x4[kKLoads];
  using QElem = float;
  using OutElem = float;

  __device__ static void load_k(const char* blk, int lane, KRegs& k) {
    const f32x4* p = reinterpret_cast<const f32x4*>(blk);
#pragma unroll
    for (int s = 0; s < kKLoads; ++s) k[s] = __builtin_nontemporal_load(p + 64 * s + lane);
  }
  __device__ static void load_v(const char* blk, int lane, VRegs& v) {
    const f32x4* p = reinterpret_cast<const f32x4*>(blk);
    const int i = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) v[dt] = __builtin_nontemporal_load(p + (16 * dt + i) * 4 + q4);
  }
  // load s holds d = 4*(4s+q4) + u, u = 0..3 (one MFMA step per u).
  __device__ static void load_q(const QElem* qh, bool active, int q4, QRegs& q) {
#pragma unroll
    for (int s = 0; s < kKLoads; ++s) {
      f32x4 w = {0.f, 0.f, 0.f, 0.f};
      if (active) w = *reinterpret_cast<const f32x4*>(qh + 4 * (4 * s + q4));
      q[s] = w;
    }
  }
  __device__ static f32x4 qk(const KRegs& k, const QRegs& q) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kKLoads; ++s)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k[s][u], q[s][u], acc, 0, 0, 0);
    return acc;
  }
  __device__ static void mask_v(VRegs& v, int q4, int nvalid) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (4 * q4 + u >= nvalid) v[dt][u] = 0.f;
  }
  // 16x16x4: reduction slot q4 of step r is token 4*q4 + r.
  __device__ static void pv(const VRegs& v, f32x4 p, f32x4 (&o)[kDt]) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(v[dt][r], p[r], o[dt], 0, 0, 0);
  }
};

// bf16 query, fp8 e4m3fn cache (x = 16): codes are converted to bf16 in
// registers (exact); k_scale and v_scale are applied as scalars outside.
template <int D>
struct PolicyFp8 {
  static constexpr int kElem = 1;
  static constexpr int kKLoads = D / 64;     // uint4 = 16 d at one token
  static constexpr int kDt = D / 16;
  static constexpr int NB = 4;
  using KRegs = u32x4[kKLoads];
  using VRegs = unsigned[kDt];               // 4 codes: tokens 4*q4..+3 of one d
  using QRegs = bf16x8[2 * kKLoads];
  using QElem = __bf16;
  using OutElem = __bf16;

  __device__ static void load_k(const char* blk, int lane, KRegs& k) {
    const u32x4* p = reinterpret_cast<const u32x4*>(blk);
#pragma unroll
    for (int h = 0; h < kKLoads; ++h) k[h] = __builtin_nontemporal_load(p + 64 * h + lane);
  }
  __device__ static void load_v(const char* blk, int lane, VRegs& v) {
    const unsigned* p = reinterpret_cast<const unsigned*>(blk);
    const int i = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) v[dt] = __builtin_nontemporal_load(p + (16 * dt + i) * 4 + q4);
  }
  // load h of lane quad q4 is chunk 4h + q4 (16 d); step 2h + half uses its
  // 8 d starting at 16*(4h+q4) + 8*half.
  __device__ static void load_q(const QElem* qh, bool active, int q4, QRegs& q) {
#pragma unroll
    for (int h = 0; h < kKLoads; ++h)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 w = {0, 0, 0, 0};
        if (active) w = *reinterpret_cast<const u32x4*>(qh + 16 * (4 * h + q4) + 8 * half);
        q[2 * h + half] = __builtin_bit_cast(bf16x8, w);
      }
  }
  __device__ static f32x4 qk(const KRegs& k, const QRegs& q) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < kKLoads; ++h)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 a;
        a[0] = fp8x2_to_bf16x2<false>(k[h][2 * half]);
        a[1] = fp8x2_to_bf16x2<true>(k[h][2 * half]);
        a[2] = fp8x2_to_bf16x2<false>(k[h][2 * half + 1]);
        a[3] = fp8x2_to_bf16x2<true>(k[h][2 * half + 1]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), q[2 * h + half], acc, 0, 0, 0);
      }
    return acc;
  }
  __device__ static void mask_v(VRegs& v, int q4, int nvalid) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) {
      unsigned x = v[dt];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (4 * q4 + u >= nvalid) x &= ~(0xFFu << (8 * u));
      v[dt] = x;
    }
  }
  __device__ static void pv(const VRegs& v, f32x4 p, f32x4 (&o)[kDt]) {
    const s16x4 pb = pack_bf16x4(p);
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) {
      u32x2 a;
      a[0] = fp8x2_to_bf16x2<false>(v[dt]);
      a[1] = fp8x2_to_bf16x2<true>(v[dt]);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), pb, o[dt], 0, 0, 0);
    }
  }
};

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float v) { return static_cast<__bf16>(v); }

// ---------------------------------------------------------------------------
// Partition kernel: grid (num_splits, num_kv_heads, num_seqs), kThreads threads.
// ---------------------------------------------------------------------------

template <typename P, int D>
__global__ void __launch_bounds__(kThreads)
pa_partition_kernel(const DecodeArgs a) {
  constexpr int kDt = P::kDt;
  constexpr int NB = P::NB;
  using QElem = typename P::QElem;
  using OutElem = typename P::OutElem;

  // LDS for the cross-wave merge: per wave, per query head of the group,
  // head_size floats padded by 4 to spread rows over banks.
  constexpr int kRow = D + 4;
  __shared__ float s_o[kWaves][PA_MAX_GROUP_DEV][kRow];
  __shared__ float s_m[kWaves][PA_MAX_GROUP_DEV];
  __shared__ float s_l[kWaves][PA_MAX_GROUP_DEV];

  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15;
  const int q4 = lane >> 4;
  const int G = a.group;

  int L = a.seq_lens[seq];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int t_begin = split * a.split_tokens;
  if (L == 0) {
    // Empty sequence: split 0 writes the zero row for the group's heads.
    if (split == 0) {
      OutElem* out = reinterpret_cast<OutElem*>(a.out);
      for (int e = threadIdx.x; e < G * D; e += kThreads) {
        const int g = e / D, d = e - g * D;
        out[((int64_t)seq * a.num_heads + kvh * G + g) * D + d] = from_f32<OutElem>(0.f);
      }
    }
    return;
  }
  if (t_begin >= L) return;
  const int t_end = min(L, t_begin + a.split_tokens);
  const int nsplit_seq = (L + a.split_tokens - 1) / a.split_tokens;
  const int blk_begin = t_begin / kBlock;
  const int blk_end = (t_end + kBlock - 1) / kBlock;
  const int last_blk = (L - 1) / kBlock;     // logical block holding token L-1
  const int last_valid = L - last_blk * kBlock;  // valid slots in it (1..16)

  // Query rows of the group (zero for padded columns g >= G).
  const int g = i;
  const bool active = g < G;
  const int h = kvh * G + (active ? g : 0);
  const QElem* qh = reinterpret_cast<const QElem*>(a.query) + ((int64_t)seq * a.num_heads + h) * D;
  typename P::QRegs qreg;
  P::load_q(qh, active, q4, qreg);

  float k_scale = 1.f, v_scale = 1.f;
  if (a.k_scale) k_scale = *a.k_scale;
  if (a.v_scale) v_scale = *a.v_scale;
  const float c = a.scale * kLog2e * k_scale;
  float slope2 = 0.f;
  if (a.alibi_slopes && active) slope2 = a.alibi_slopes[h] * kLog2e;

  const int32_t* table = a.block_tables + (int64_t)seq * a.max_blocks_per_seq;
  const char* kbase = reinterpret_cast<const char*>(a.key_cache) + (int64_t)kvh * a.k_head_stride_bytes;
  const char* vbase = reinterpret_cast<const char*>(a.value_cache) + (int64_t)kvh * a.v_head_stride_bytes;

  float m = -__builtin_huge_valf();
  float lsum = 0.f;
  f32x4 o[kDt];
#pragma unroll
  for (int dt = 0; dt < kDt; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int base = blk_begin + wave * NB; base < blk_end; base += kWaves * NB) {
    typename P::KRegs kr[NB];
    typename P::VRegs vr[NB];
    // Issue every load of the group before any use.
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int blk = base + j;
      if (blk < blk_end) {
        unsigned phys = (unsigned)table[blk];
        phys = phys < (unsigned)a.num_blocks ? phys : (unsigned)(a.num_blocks - 1);
        P::load_k(kbase + (int64_t)phys * a.k_block_stride_bytes, lane, kr[j]);
        P::load_v(vbase + (int64_t)phys * a.v_block_stride_bytes, lane, vr[j]);
      }
    }
    f32x4 z[NB];
    float mx = -__builtin_huge_valf();
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int blk = base + j;
      if (blk < blk_end) {
        const f32x4 s = P::qk(kr[j], qreg);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = blk * kBlock + 4 * q4 + r;
          const float zz = fmaf(s[r], c, slope2 * (float)(t - (L - 1)));
          z[j][r] = t < L ? zz : -__builtin_huge_valf();
          mx = fmaxf(mx, z[j][r]);
        }
      } else {
        z[j] = f32x4{-__builtin_huge_valf(), -__builtin_huge_valf(), -__builtin_huge_valf(),
                     -__builtin_huge_valf()};
      }
    }
    mx = wave_max_across_quads(mx);
    const float m_new = fmaxf(m, mx);
    const float alpha = fast_exp2(m - m_new);
    m = m_new;
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) o[dt] *= alpha;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int blk = base + j;
      if (blk < blk_end) {
        f32x4 p;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[r] = fast_exp2(z[j][r] - m_new);
          lsum += p[r];
        }
        if (blk == last_blk && last_valid < kBlock) P::mask_v(vr[j], q4, last_valid);
        P::pv(vr[j], p, o);
      }
    }
  }
  lsum = wave_sum_across_quads(lsum);

  // Cross-wave merge.
  if (active) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
      *reinterpret_cast<f32x4*>(&s_o[wave][g][16 * dt + 4 * q4]) = o[dt];
    if (q4 == 0) {
      s_m[wave][g] = m;
      s_l[wave][g] = lsum;
    }
  }
  __syncthreads();

  const bool direct = nsplit_seq == 1;
  for (int e = threadIdx.x; e < G * (D / 4); e += kThreads) {
    const int gg = e / (D / 4);
    const int d4 = e - gg * (D / 4);
    float big_m = s_m[0][gg];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) big_m = fmaxf(big_m, s_m[w][gg]);
    float tot = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(s_m[w][gg] - big_m);
      tot += f * s_l[w][gg];
      acc += f * *reinterpret_cast<const f32x4*>(&s_o[w][gg][4 * d4]);
    }
    const float inv = v_scale / tot;
    acc *= inv;
    const int hh = kvh * G + gg;
    if (direct) {
      OutElem* out = reinterpret_cast<OutElem*>(a.out) + ((int64_t)seq * a.num_heads + hh) * D + 4 * d4;
#pragma unroll
      for (int r = 0; r < 4; ++r) out[r] = from_f32<OutElem>(acc[r]);
    } else {
      const int64_t row = ((int64_t)seq * a.num_heads + hh) * a.num_splits + split;
      *reinterpret_cast<f32x4*>(a.tmp_out + row * D + 4 * d4) = acc;
      if (d4 == 0) {
        a.max_logits[row] = big_m * kLn2;
        a.exp_sums[row] = tot;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Reduce kernel: grid (num_heads, num_seqs), 64 threads. Merges the per-split
// partials of sequences that span more than one split.
// ---------------------------------------------------------------------------

template <typename OutElem, int D>
__global__ void __launch_bounds__(64)
pa_reduce_kernel(const DecodeArgs a) {
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int lane = threadIdx.x;
  int L = a.seq_lens[seq];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int n = (L + a.split_tokens - 1) / a.split_tokens;
  if (n <= 1) return;
  const int64_t row0 = ((int64_t)seq * a.num_heads + h) * a.num_splits;
  const float* ml = a.max_logits + row0;
  const float* es = a.exp_sums + row0;

  float big_m = -__builtin_huge_valf();
  for (int p = lane; p < n; p += 64) big_m = fmaxf(big_m, ml[p]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) big_m = fmaxf(big_m, __shfl_xor(big_m, off, 64));
  float tot = 0.f;
  for (int p = lane; p < n; p += 64) tot += es[p] * fast_exp2((ml[p] - big_m) * kLog2e);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off, 64);

  constexpr int kPer = D / 64;   // elements per lane
  float acc[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) acc[k] = 0.f;
  const float* tmp = a.tmp_out + row0 * D + lane * kPer;
  for (int p = 0; p < n; ++p) {
    const float w = es[p] * fast_exp2((ml[p] - big_m) * kLog2e);
#pragma unroll
    for (int k = 0; k < kPer; ++k) acc[k] += w * tmp[(int64_t)p * D + k];
  }
  const float inv = 1.f / tot;
  OutElem* out = reinterpret_cast<OutElem*>(a.out) + ((int64_t)seq * a.num_heads + h) * D + lane * kPer;
#pragma unroll
  for (int k = 0; k < kPer; ++k) out[k] = from_f32<OutElem>(acc[k] * inv);
}

// ---------------------------------------------------------------------------
// Host-side launchers.
// ---------------------------------------------------------------------------

template <typename P, int D>
static hipError_t launch_pair(const DecodeArgs& a, hipStream_t stream, const LaunchHooks& hooks) {
  if (hooks.before_partition) hooks.before_partition(stream);
  hipLaunchKernelGGL((pa_partition_kernel<P, D>), dim3(a.num_splits, a.num_kv_heads, a.num_seqs),
                     dim3(kThreads), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (hooks.after_partition) hooks.after_partition(stream);
  if (err != hipSuccess || a.num_splits <= 1) return err;
  if (hooks.before_reduce) hooks.before_reduce(stream);
  hipLaunchKernelGGL((pa_reduce_kernel<typename P::OutElem, D>), dim3(a.num_heads, a.num_seqs),
                     dim3(64), 0, stream, a);
  err = hipGetLastError();
  if (hooks.after_reduce) hooks.after_reduce(stream);
  return err;
}

hipError_t launch_decode(const DecodeArgs& a, int kind, hipStream_t stream, const LaunchHooks& hooks) {
  switch (kind * 1000 + a.head_size) {
    case KIND_F32 * 1000 + 64: return launch_pair<PolicyF32<64>, 64>(a, stream, hooks);
    case KIND_F32 * 1000 + 128: return launch_pair<PolicyF32<128>, 128>(a, stream, hooks);
    case KIND_BF16 * 1000 + 64: return launch_pair<PolicyBf16<64>, 64>(a, stream, hooks);
    case KIND_BF16 * 1000 + 128: return launch_pair<PolicyBf16<128>, 128>(a, stream, hooks);
    case KIND_FP8 * 1000 + 64: return launch_pair<PolicyFp8<64>, 64>(a, stream, hooks);
    case KIND_FP8 * 1000 + 128: return launch_pair<PolicyFp8<128>, 128>(a, stream, hooks);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
