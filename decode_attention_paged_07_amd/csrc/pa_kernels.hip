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
//    ordered kv head, sequence, block; a pair cut by a share boundary is
//    finished by a merge kernel. Ragged lengths then cost no tail imbalance.
//
// Contraction mapping (per 16-token block; 16x16 fp32 MFMA results):
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

// ---------------------------------------------------------------------------
// Split grid: grid (num_splits, ceil(num_kv_heads / kWaves), num_seqs).
// ---------------------------------------------------------------------------

template <typename P, int D, int NB, bool ALIBI>
__global__ void __launch_bounds__(kWaves * 64)
pa_split_kernel(const DecodeArgs a) {
  using OutElem = typename P::OutElem;
  const int split = blockIdx.x;
  const int seq = blockIdx.z;
  const int kvh = blockIdx.y * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (kvh >= a.num_kv_heads) return;
  const int lane = threadIdx.x & 63;
  const int L = clamp_len(a.seq_lens[seq], a.max_seq_len);
  if (L == 0) {
    if (split == 0) write_zero_rows<OutElem, D>(a, seq, kvh, lane);
    return;
  }
  const int t_begin = split * a.split_tokens;
  if (t_begin >= L) return;
  const int b0 = t_begin / kBlock;
  const int b1 = min((L + kBlock - 1) / kBlock, (t_begin + a.split_tokens) / kBlock);
  const int nsplit_seq = (L + a.split_tokens - 1) / a.split_tokens;

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
  constexpr int kPer = D / 64;
  float acc[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) acc[k] = 0.f;
  const float* tmp = a.tmp_out + row0 * D + lane * kPer;
  for (int p = 0; p < n; ++p) {
    const float wgt = es[p] * fast_exp2((ml[p] - big_m) * kLog2e);
#pragma unroll
    for (int k = 0; k < kPer; ++k) acc[k] += wgt * tmp[(int64_t)p * D + k];
  }
  const float inv = 1.f / tot;
  OutElem* out = reinterpret_cast<OutElem*>(a.out) + ((int64_t)seq * a.num_heads + h) * D + lane * kPer;
#pragma unroll
  for (int k = 0; k < kPer; ++k) out[k] = from_f32<OutElem>(acc[k] * inv);
}

// ---------------------------------------------------------------------------
// Stream-K: grid (num_workgroups), kWaves waves each; wave w of W in total
// owns tiles [w*U, min(total, (w+1)*U)) with U = ceil(total / W) of the
// total = num_kv_heads * T tiles, T = sum_s ceil(L_s / 16), ordered
// (kv head, sequence, block). Pair p = kvh*S + s cut into several segments
// writes segment partials at slot p + w (unique: both p and w grow along the
// order) and records its first and last wave in seg_meta[p].
// ---------------------------------------------------------------------------

__device__ __forceinline__ int blocks_of(int L) { return (L + kBlock - 1) / kBlock; }

template <typename P, int D, int NB, bool ALIBI>
__global__ void __launch_bounds__(kWaves * 64)
pa_streamk_kernel(const DecodeArgs a) {
  using OutElem = typename P::OutElem;
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = gridDim.x * kWaves;
  const int S = a.num_seqs;

  int T = 0;
  for (int c0 = 0; c0 < S; c0 += 64) {
    const int s = c0 + lane;
    T += wave_sum(s < S ? blocks_of(clamp_len(a.seq_lens[s], a.max_seq_len)) : 0);
  }
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
  int running = 0;
  for (int c0 = 0; c0 < S; c0 += 64) {
    const int s = c0 + lane;
    const int nb = s < S ? blocks_of(clamp_len(a.seq_lens[s], a.max_seq_len)) : 0;
    const int incl = wave_incl_scan(nb, lane) + running;
    const int excl = incl - nb;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(nb > 0 && excl <= r && r < incl);
    if (hit) {
      const int ln = __builtin_ctzll(hit);
      seq = c0 + ln;
      blk = r - __builtin_amdgcn_readlane(excl, ln);
      break;
    }
    running = __builtin_amdgcn_readlane(incl, 63);
  }

  float v_scale = 1.f;
  if (a.v_scale) v_scale = *a.v_scale;
  int64_t u = u0;
  while (true) {
    const int L = clamp_len(a.seq_lens[seq], a.max_seq_len);
    const int nbs = blocks_of(L);
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
                       dim3(a.num_splits, (a.num_kv_heads + kWaves - 1) / kWaves, a.num_seqs), dim3(kWaves * 64), 0,
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
    if (a.num_splits <= 1) return hipSuccess;
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

hipError_t launch_decode(const DecodeArgs& a, int kind, hipStream_t stream, const LaunchHooks& hooks) {
  switch (kind * 1000 + a.head_size) {
    case KIND_F32 * 1000 + 64: return launch_alibi<PolicyF32<64>, 64, PA_NB_F32>(a, stream, hooks);
    case KIND_F32 * 1000 + 128: return launch_alibi<PolicyF32<128>, 128, PA_NB_F32>(a, stream, hooks);
    case KIND_BF16 * 1000 + 64: return launch_alibi<PolicyBf16<64>, 64, PA_NB_BF16>(a, stream, hooks);
    case KIND_BF16 * 1000 + 128: return launch_alibi<PolicyBf16<128>, 128, PA_NB_BF16>(a, stream, hooks);
    case KIND_FP8 * 1000 + 64: return launch_alibi<PolicyFp8<64>, 64, PA_NB_FP8>(a, stream, hooks);
    case KIND_FP8 * 1000 + 128: return launch_alibi<PolicyFp8<128>, 128, PA_NB_FP8>(a, stream, hooks);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
