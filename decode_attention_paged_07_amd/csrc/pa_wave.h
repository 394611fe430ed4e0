// Device-side building blocks shared by the decode kernels (pa_kernels.hip,
// pa_shared.hip): vector types, wave reductions, and the element-type
// policies that load K/V tiles straight into MFMA operand registers.
//
// Contraction mapping (per 16-token block; 16x16 fp32 MFMA results):
//   S[t][g] = sum_d K[t][d] q[g][d]: A = K tile (rows = tokens), B = q
//     (columns = query heads, zero-padded to 16). Result lane (g + 16*q4)
//     holds S[4*q4 + r][g], r = 0..3.
//   O[d][g] += sum_t V[t][d] P[g][t]: A = V^T tile (rows = head dims),
//     B = P. B's lane layout for a 16-deep product equals S's result layout,
//     so P stays in its registers.
// Any permutation of a reduction index is valid when both operands agree: the
// d-order of the K operand is chosen so each lane's 16-byte K load is
// contiguous in the cache and one wave load instruction covers 1 KiB
// contiguous. V loads of one d-tile cover 512 B (bf16), 1 KiB (f32) or
// 256 B (fp8) contiguous.
#pragma once

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
constexpr int kWaves = PA_WAVES;          // waves per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;     // log2 units
constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------------------
// Wave-level helpers.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float quad_max(float v) {   // over lanes l, l^16, l^32, l^48
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float quad_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float max4(f32x4 v) { return fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])); }

__device__ __forceinline__ s16x4 pack_bf16x4(f32x4 v) {
  return __builtin_bit_cast(s16x4, __builtin_convertvector(v, bf16x4));
}

// Two e4m3fn codes (bytes 0-1, or 2-3 when HI, of w) -> two bf16, exact (every
// e4m3 value is a bf16 value); scale 1 so the conversion itself cannot round.
template <bool HI>
__device__ __forceinline__ unsigned fp8x2_to_bf16x2(unsigned w) {
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

__device__ __forceinline__ int clamp_len(int L, int max_seq_len) {
  return L < 0 ? 0 : (L > max_seq_len ? max_seq_len : L);
}

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float v) { return static_cast<__bf16>(v); }

template <typename T>
__device__ __forceinline__ void store4(T* p, f32x4 v) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4*>(p) = v;
  } else {
    *reinterpret_cast<s16x4*>(p) = pack_bf16x4(v);
  }
}

// ---------------------------------------------------------------------------
// Element-type policies: register shapes, lane offsets, loads, contractions.
// Loads take a wave-uniform tile address plus this lane's byte offset, so the
// address is one SGPR pair plus a loop-invariant VGPR.
// ---------------------------------------------------------------------------

// bf16 query, bf16 cache (x = 8): K chunk c = 8 consecutive d at one token.
template <int D>
struct PolicyBf16 {
  static constexpr int kKLoads = D / 32;     // 16x16x32 steps, one 16-byte load each
  static constexpr int kDt = D / 16;         // d-tiles of the PV product
  using KRegs = u32x4[kKLoads];
  using VRegs = u32x2[kDt];                  // 4 bf16 tokens of one d per tile
  using QRegs = bf16x8[kKLoads];
  using QElem = __bf16;
  using OutElem = __bf16;
  struct Lane { uint32_t k, v; };

  // K: lane l = i + 16*q4 reads chunk (4s + q4) at token i, byte (64s + l)*16.
  // V: lane (i + 16*q4) of tile dt reads tokens 4*q4..+3 of d = 16*dt + i.
  __device__ static Lane lane_offsets(int lane) {
    return {(uint32_t)lane * 16u, (uint32_t)((lane & 15) * 32 + (lane >> 4) * 8)};
  }
  __device__ static void load_k(const char* t, const Lane& lo, KRegs& k) {
#pragma unroll
    for (int s = 0; s < kKLoads; ++s)
      k[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(t + lo.k + s * 1024));
  }
  __device__ static void load_v(const char* t, const Lane& lo, VRegs& v) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
      v[dt] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(t + lo.v + dt * 512));
  }
  // q in the d-order of load_k: step s, lane quad q4 -> d = 8*(4s+q4) + u.
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
  // Zero V of tokens 4*q4+u >= nvalid (only on a sequence's partial last block).
  __device__ static void mask_v(VRegs& v, int q4, int nvalid) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        unsigned x = v[dt][w];
        const int t0 = 4 * q4 + 2 * w;
        if (t0 >= nvalid) x &= 0xFFFF0000u;
        if (t0 + 1 >= nvalid) x &= 0x0000FFFFu;
        v[dt][w] = x;
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
  static constexpr int kKLoads = D / 16;     // 16 bytes = 4 d at one token
  static constexpr int kDt = D / 16;
  using KRegs = f32x4[kKLoads];
  using VRegs = f32x4[kDt];                  // 4 fp32 tokens of one d per tile
  using QRegs = f32x4[kKLoads];
  using QElem = float;
  using OutElem = float;
  struct Lane { uint32_t k, v; };

  __device__ static Lane lane_offsets(int lane) {
    return {(uint32_t)lane * 16u, (uint32_t)((lane & 15) * 64 + (lane >> 4) * 16)};
  }
  __device__ static void load_k(const char* t, const Lane& lo, KRegs& k) {
#pragma unroll
    for (int s = 0; s < kKLoads; ++s)
      k[s] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(t + lo.k + s * 1024));
  }
  __device__ static void load_v(const char* t, const Lane& lo, VRegs& v) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
      v[dt] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(t + lo.v + dt * 1024));
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
      for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k[s][u], q[s][u], acc, 0, 0, 0);
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
      for (int r = 0; r < 4; ++r) o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(v[dt][r], p[r], o[dt], 0, 0, 0);
  }
};

// bf16 query, fp8 e4m3fn cache (x = 16): codes are converted to bf16 in
// registers (exact); k_scale and v_scale are applied as scalars outside.
template <int D>
struct PolicyFp8 {
  static constexpr int kKLoads = D / 64;     // 16 bytes = 16 d at one token
  static constexpr int kDt = D / 16;
  using KRegs = u32x4[kKLoads];
  using VRegs = unsigned[kDt];               // 4 codes: tokens 4*q4..+3 of one d
  using QRegs = bf16x8[2 * kKLoads];
  using QElem = __bf16;
  using OutElem = __bf16;
  struct Lane { uint32_t k, v; };

  __device__ static Lane lane_offsets(int lane) {
    return {(uint32_t)lane * 16u, (uint32_t)((lane & 15) * 16 + (lane >> 4) * 4)};
  }
  __device__ static void load_k(const char* t, const Lane& lo, KRegs& k) {
#pragma unroll
    for (int h = 0; h < kKLoads; ++h)
      k[h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(t + lo.k + h * 1024));
  }
  __device__ static void load_v(const char* t, const Lane& lo, VRegs& v) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
      v[dt] = __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(t + lo.v + dt * 256));
  }
  // load h of lane quad q4 is chunk 4h + q4 (16 d); step 2h + half uses the
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

// ---------------------------------------------------------------------------
// One wave's attention over a run of blocks of one (sequence, kv head).
// ---------------------------------------------------------------------------

template <typename P, int D, int NB, bool ALIBI>
struct WaveAttn {
  static constexpr int kDt = P::kDt;
  typename P::QRegs q;
  typename P::Lane lo;
  f32x4 o[kDt];
  float m, m_true, lsum;
  float c, slope2;
  float lane_bias[4];   // slope2 * (4*q4 + r), ALiBi only
  int lane, q4;
  bool active;          // this lane's column g is a real query head

  // Query rows of heads kvh*G + g (zero for padded columns g >= G).
  __device__ void begin(const DecodeArgs& a, int seq, int kvh) {
    lane = threadIdx.x & 63;
    q4 = lane >> 4;
    const int g = lane & 15;
    active = g < a.group;
    const int h = kvh * a.group + (active ? g : 0);
    lo = P::lane_offsets(lane);
    const auto* qh = reinterpret_cast<const typename P::QElem*>(a.query) + ((int64_t)seq * a.num_heads + h) * D;
    P::load_q(qh, active, q4, q);
    float k_scale = 1.f;
    if (a.k_scale) k_scale = *a.k_scale;
    c = a.scale * kLog2e * k_scale;
    slope2 = 0.f;
    if constexpr (ALIBI) {
      if (active) slope2 = a.alibi_slopes[h] * kLog2e;
#pragma unroll
      for (int r = 0; r < 4; ++r) lane_bias[r] = slope2 * (float)(4 * q4 + r);
    }
    m = m_true = kNegInf;
    lsum = 0.f;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Logical blocks [b0, b1) of a sequence of length L; kh / vh address this kv
  // head's tile inside physical block 0. Table entries are read 64 at a time
  // into one VGPR (lane k = entry chunk + k) and broadcast per block.
  struct Cursor {
    int chunk, tbl;
  };

  __device__ int issue(const DecodeArgs& a, const char* kh, const char* vh, const int32_t* table_row, int g0,
                       int b1, Cursor& cur, typename P::KRegs (&kr)[NB], typename P::VRegs (&vr)[NB]) {
    if (g0 - cur.chunk >= 64) {
      cur.chunk += 64;
      cur.tbl = (cur.chunk + lane < b1) ? table_row[cur.chunk + lane] : 0;
    }
    const unsigned top = (unsigned)(a.num_blocks - 1);
    const int n = min(NB, b1 - g0);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (j < n) {
        unsigned phys = (unsigned)__builtin_amdgcn_readlane(cur.tbl, g0 + j - cur.chunk);
        phys = phys < top ? phys : top;
        const int64_t off = (int64_t)phys * a.k_block_stride_bytes;   // K and V tiles share strides
        P::load_k(kh + off, lo, kr[j]);
        P::load_v(vh + off, lo, vr[j]);
      }
    }
    return n;
  }

  __device__ void run(const DecodeArgs& a, const char* kh, const char* vh, const int32_t* table_row, int b0,
                      int b1, int L) {
    const int last_blk = (L - 1) >> 4;
    const int tail = L - (last_blk << 4);                 // valid slots in the last block, 1..16
    Cursor cur{b0, (b0 + lane < b1) ? table_row[b0 + lane] : 0};
    if constexpr (PA_PIPE) {
      // Two register buffers: the next group's loads are in flight while the
      // current group is computed.
      typename P::KRegs ka[NB], kb[NB];
      typename P::VRegs va[NB], vb[NB];
      int g0 = b0;
      if (g0 >= b1) return;
      int na = issue(a, kh, vh, table_row, g0, b1, cur, ka, va);
      while (true) {
        const int g1 = g0 + NB;
        int nb = 0;
        if (g1 < b1) nb = issue(a, kh, vh, table_row, g1, b1, cur, kb, vb);
        consume(ka, va, g0, na, L, last_blk, tail);
        if (g1 >= b1) break;
        const int g2 = g1 + NB;
        if (g2 < b1) na = issue(a, kh, vh, table_row, g2, b1, cur, ka, va);
        consume(kb, vb, g1, nb, L, last_blk, tail);
        if (g2 >= b1) break;
        g0 = g2;
      }
    } else {
      for (int g0 = b0; g0 < b1; g0 += NB) {
        typename P::KRegs kr[NB];
        typename P::VRegs vr[NB];
        const int n = issue(a, kh, vh, table_row, g0, b1, cur, kr, vr);
        consume(kr, vr, g0, n, L, last_blk, tail);
      }
    }
  }

  __device__ void consume(typename P::KRegs (&kr)[NB], typename P::VRegs (&vr)[NB], int g0, int n, int L,
                          int last_blk, int tail) {
    f32x4 z[NB];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (j < n) {
        const f32x4 s = P::qk(kr[j], q);
        const int blk = g0 + j;
        if constexpr (ALIBI) {
          const float base = (float)(blk * kBlock - (L - 1));
#pragma unroll
          for (int r = 0; r < 4; ++r) z[j][r] = fmaf(s[r], c, fmaf(slope2, base, lane_bias[r]));
        } else {
          z[j] = s * c;
        }
        if (blk == last_blk && tail < kBlock) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (4 * q4 + r >= tail) z[j][r] = kNegInf;
          P::mask_v(vr[j], q4, tail);
        }
        mx = fmaxf(mx, max4(z[j]));
      }
    }
    mx = quad_max(mx);
    m_true = fmaxf(m_true, mx);
    if (wave_any(mx > m + kRescaleSlack)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2(m - m_new);
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) o[dt] *= alpha;
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (j < n) {
        f32x4 p;
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = fast_exp2(z[j][r] - m);
        lsum += (p[0] + p[1]) + (p[2] + p[3]);
        P::pv(vr[j], p, o);
      }
    }
  }

  __device__ void finish() { lsum = quad_sum(lsum); }

  // o / lsum * mult for this lane's column, 4 consecutive d per tile.
  template <typename T>
  __device__ void store_rows(T* row_base, int64_t row_stride, float mult) const {
    if (!active) return;
    T* dst = row_base + (int64_t)(lane & 15) * row_stride + 4 * q4;
    const float f = mult / lsum;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) store4(dst + 16 * dt, o[dt] * f);
  }
};

template <typename OutElem, int D>
__device__ void write_zero_rows(const DecodeArgs& a, int seq, int kvh, int lane) {
  OutElem* out = reinterpret_cast<OutElem*>(a.out) + ((int64_t)seq * a.num_heads + kvh * a.group) * D;
  for (int e = lane; e < a.group * D; e += 64) out[e] = from_f32<OutElem>(0.f);
}


// One (split, group of kWaves kv heads, sequence) item of the split grid;
// also called from the shared-prefix kernel for the sequences' own blocks.
template <typename P, int D, int NB, bool ALIBI>
__device__ __forceinline__ void split_unit(const DecodeArgs& a, int split, int kvh_group, int seq) {
  using OutElem = typename P::OutElem;
  const int kvh = kvh_group * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (kvh >= a.num_kv_heads) return;
  const int lane = threadIdx.x & 63;
  const int L = clamp_len(a.seq_lens[seq], a.max_seq_len);
  if (L == 0) {
    if (split == 0) write_zero_rows<OutElem, D>(a, seq, kvh, lane);
    return;
  }
  // With a shared prefix (first_block set), this kernel covers only the
  // sequence's own tokens after the prefix's first_block full blocks and
  // always writes partials, which a merge combines with the prefix's.
  const int first = a.first_block ? min(max(a.first_block[seq], 0), min(L / kBlock, a.max_first_block)) : 0;
  const int t0 = first * kBlock;
  const int t_begin = t0 + split * a.split_tokens;
  if (t_begin >= L) return;
  const int b0 = t_begin / kBlock;
  const int b1 = min((L + kBlock - 1) / kBlock, (t_begin + a.split_tokens) / kBlock);
  const int nsplit_seq = a.first_block ? 0 : (L + a.split_tokens - 1) / a.split_tokens;

  WaveAttn<P, D, NB, ALIBI> w;
  w.begin(a, seq, kvh);
  const char* kh = reinterpret_cast<const char*>(a.key_cache) + (int64_t)kvh * a.k_head_stride_bytes;
  const char* vh = reinterpret_cast<const char*>(a.value_cache) + (int64_t)kvh * a.v_head_stride_bytes;
  w.run(a, kh, vh, a.block_tables + (int64_t)seq * a.max_blocks_per_seq, b0, b1, L);
  w.finish();

  float v_scale = 1.f;
  if (a.v_scale) v_scale = *a.v_scale;
  const int64_t h0 = (int64_t)seq * a.num_heads + kvh * a.group;
  if (nsplit_seq == 1) {
    w.store_rows(reinterpret_cast<OutElem*>(a.out) + h0 * D, D, v_scale);
  } else {
    // Per-split partials: normalised output, true max logit (natural units)
    // and the exp-sum relative to it.
    w.store_rows(a.tmp_out + (h0 * a.num_splits + split) * D, (int64_t)a.num_splits * D, v_scale);
    if (w.active && w.q4 == 0) {
      const int64_t row = (h0 + (lane & 15)) * a.num_splits + split;
      a.max_logits[row] = w.m_true * kLn2;
      a.exp_sums[row] = w.lsum * fast_exp2(w.m - w.m_true);
    }
  }
}

}  // namespace pa
