// Device-side building blocks shared by the decode kernels (pa_kernels.hip,
// pa_shared.hip): vector types, wave reductions, and the element-type
// policies that load K/V tiles straight into MFMA operand registers.
//
// Contraction mapping (per 16 tokens of a block; 16x16 fp32 MFMA results):
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

constexpr int kWaves = PA_WAVES;          // waves per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;     // log2 units
constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------------------
// Wave-level helpers.
// ---------------------------------------------------------------------------

// Reductions over lanes l, l^16, l^32, l^48 (the four lane quads of a
// 16-column MFMA result) on gfx950's VALU row swaps, no LDS round trip:
// v_permlane16_swap on two copies of v leaves rows (0, 0, 2, 2) in one and
// (1, 1, 3, 3) in the other, so combining them pairs each lane with lane
// l^16; v_permlane32_swap then leaves (lo, lo) and (hi, hi), pairing l with
// l^32. Every lane of the wave must be active.
template <typename Op>
__device__ __forceinline__ float quad_reduce(float v, Op op) {
  const unsigned b = __float_as_uint(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  v = op(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const unsigned c = __float_as_uint(v);
  const auto r32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return op(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}
__device__ __forceinline__ float quad_max(float v) {
  return quad_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}
// The sum is formed in the same order on every lane: (row0 + row1) + (row2 + row3).
__device__ __forceinline__ float quad_sum(float v) {
  return quad_reduce(v, [](float x, float y) { return x + y; });
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
//
// A policy covers one (physical block, kv head) tile of BS = 16 or 32 tokens
// as BS/16 sub-tiles of 16 S rows; row 4*q4 + r of sub-tile t holds token
// tile_token<BS>(t, q4, r). With 32-token blocks the two sub-tiles interleave
// in runs of 8 tokens: a K load instruction then reads whole 128-byte lines
// (8 tokens of a 16-byte chunk), and a V load gives each lane 8 consecutive
// tokens of one head dim, so one instruction reads whole V rows; a row swap
// between lane quads (split_rows) then hands each sub-tile its tokens.
// Reading the two 16-token halves separately would split every cache line
// between two instructions, which measured markedly slower.
// ---------------------------------------------------------------------------

template <int BS>
__device__ __forceinline__ constexpr int tile_token(int t, int q4, int r) {
  return BS == 16 ? 4 * q4 + r : 16 * (q4 >> 1) + 8 * t + 4 * (q4 & 1) + r;
}
// Token of K row rho (= 4*q4 + r) of sub-tile 0; sub-tile t adds 8*t.
template <int BS>
__device__ __forceinline__ constexpr int k_row_token(int rho) {
  return BS == 16 ? rho : 16 * (rho >> 3) + (rho & 7);
}

// lo / hi: tokens 8*q4 .. +3 / 8*q4+4 .. +7 of lane quad q4 (a 32-token
// tile). Afterwards lo holds sub-tile 0's tokens of this lane and hi sub-tile
// 1's: quads 2k and 2k+1 exchange one half (v_permlane16_swap: odd rows of
// the first operand trade places with even rows of the second).
__device__ __forceinline__ void split_rows(unsigned& lo, unsigned& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(lo, hi, false, false);
  lo = r[0];
  hi = r[1];
}

template <bool C, typename A, typename B> struct Pick { using type = A; };
template <typename A, typename B> struct Pick<false, A, B> { using type = B; };

// bf16 query, bf16 cache (x = 8): K chunk c = 8 consecutive d at one token.
template <int D, int BS = 16>
struct PolicyBf16 {
  static constexpr int kBS = BS;
  static constexpr int kKvElemBytes = 2;
  static constexpr int kSub = BS / 16;       // 16-row sub-tiles per tile
  static constexpr int kKLoads = D / 32;     // per sub-tile: 16x16x32 steps, one 16-byte load each
  static constexpr int kDt = D / 16;         // d-tiles of the PV product
  using VVec = typename Pick<BS == 16, u32x2, u32x4>::type;   // 2 bf16 tokens per dword
  using KRegs = u32x4[kSub][kKLoads];
  using VRegs = VVec[kDt];
  using QRegs = bf16x8[kKLoads];
  using QElem = __bf16;
  using OutElem = __bf16;
  struct Lane { uint32_t k, v; };

  // K: lane (rho + 16*q4) of step s reads chunk (4s + q4) at token
  //    k_row_token(rho) + 8t. V: lane (i + 16*q4) of tile dt reads BS/4
  //    consecutive tokens from 4*q4 (BS/4 * q4) of d = 16*dt + i.
  __device__ static Lane lane_offsets(int lane) {
    const int q4 = lane >> 4, rho = lane & 15;
    return {(uint32_t)(q4 * BS * 16 + k_row_token<BS>(rho) * 16), (uint32_t)(rho * BS * 2 + q4 * (BS / 4) * 2)};
  }
  __device__ static void load_k(const char* t, const Lane& lo, KRegs& k) {
#pragma unroll
    for (int st = 0; st < kSub; ++st)
#pragma unroll
      for (int s = 0; s < kKLoads; ++s)
        k[st][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(t + lo.k + s * 4 * BS * 16 + st * 128));
  }
  __device__ static void load_v(const char* t, const Lane& lo, VRegs& v) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
      v[dt] = __builtin_nontemporal_load(reinterpret_cast<const VVec*>(t + lo.v + dt * 16 * BS * 2));
  }
  // After the loads have landed: dwords (2t, 2t+1) of v[dt] become sub-tile t's.
  __device__ static void prepare_v(VRegs& v) {
    if constexpr (BS == 32) {
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) {
        unsigned w0 = v[dt][0], w1 = v[dt][1], w2 = v[dt][2], w3 = v[dt][3];
        split_rows(w0, w2);
        split_rows(w1, w3);
        v[dt] = VVec{w0, w1, w2, w3};
      }
    }
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
  __device__ static f32x4 qk(const KRegs& k, const QRegs& q, int st) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kKLoads; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[st][s]), q[s], acc, 0, 0, 0);
    return acc;
  }
  // Zero V of tokens >= nvalid (only on a sequence's partial last block).
  __device__ static void mask_v(VRegs& v, int q4, int nvalid) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
      for (int w = 0; w < 2 * kSub; ++w) {
        unsigned x = v[dt][w];
        const int t0 = tile_token<BS>(w >> 1, q4, 2 * (w & 1));
        if (t0 >= nvalid) x &= 0xFFFF0000u;
        if (t0 + 1 >= nvalid) x &= 0x0000FFFFu;
        v[dt][w] = x;
      }
  }
  __device__ static void pv(const VRegs& v, f32x4 p, f32x4 (&o)[kDt], int st) {
    const s16x4 pb = pack_bf16x4(p);
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) {
      const u32x2 a = {v[dt][2 * st], v[dt][2 * st + 1]};
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), pb, o[dt], 0, 0, 0);
    }
  }
};

// fp32 query, fp32 cache (x = 4): fp32 MFMA keeps full fp32 products.
template <int D, int BS = 16>
struct PolicyF32 {
  static constexpr int kBS = BS;
  static constexpr int kKvElemBytes = 4;
  static constexpr int kSub = BS / 16;
  static constexpr int kKLoads = D / 16;     // per sub-tile: 16 bytes = 4 d at one token
  static constexpr int kDt = D / 16;
  using KRegs = f32x4[kSub][kKLoads];
  using VRegs = f32x4[kSub][kDt];            // 4 fp32 tokens of one d per tile and sub-tile
  using QRegs = f32x4[kKLoads];
  using QElem = float;
  using OutElem = float;
  struct Lane { uint32_t k, v; };

  // V: lane (i + 16*q4) of tile dt, sub-tile t reads tokens
  // tile_token(t, q4, 0..3) (consecutive) of d = 16*dt + i. With 32-token
  // blocks a V row is 128 bytes and one instruction reads half of each.
  __device__ static Lane lane_offsets(int lane) {
    const int q4 = lane >> 4, rho = lane & 15;
    return {(uint32_t)(q4 * BS * 16 + k_row_token<BS>(rho) * 16),
            (uint32_t)(rho * BS * 4 + tile_token<BS>(0, q4, 0) * 4)};
  }
  __device__ static void load_k(const char* t, const Lane& lo, KRegs& k) {
#pragma unroll
    for (int st = 0; st < kSub; ++st)
#pragma unroll
      for (int s = 0; s < kKLoads; ++s)
        k[st][s] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(t + lo.k + s * 4 * BS * 16 + st * 128));
  }
  __device__ static void load_v(const char* t, const Lane& lo, VRegs& v) {
#pragma unroll
    for (int st = 0; st < kSub; ++st)
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt)
        v[st][dt] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(t + lo.v + dt * 16 * BS * 4 + st * 32));
  }
  __device__ static void prepare_v(VRegs&) {}
  // load s holds d = 4*(4s+q4) + u, u = 0..3 (one MFMA step per u).
  __device__ static void load_q(const QElem* qh, bool active, int q4, QRegs& q) {
#pragma unroll
    for (int s = 0; s < kKLoads; ++s) {
      f32x4 w = {0.f, 0.f, 0.f, 0.f};
      if (active) w = *reinterpret_cast<const f32x4*>(qh + 4 * (4 * s + q4));
      q[s] = w;
    }
  }
  __device__ static f32x4 qk(const KRegs& k, const QRegs& q, int st) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kKLoads; ++s)
#pragma unroll
      for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k[st][s][u], q[s][u], acc, 0, 0, 0);
    return acc;
  }
  __device__ static void mask_v(VRegs& v, int q4, int nvalid) {
#pragma unroll
    for (int st = 0; st < kSub; ++st)
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (tile_token<BS>(st, q4, u) >= nvalid) v[st][dt][u] = 0.f;
  }
  // 16x16x4: reduction slot q4 of step r is row 4*q4 + r.
  __device__ static void pv(const VRegs& v, f32x4 p, f32x4 (&o)[kDt], int st) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(v[st][dt][r], p[r], o[dt], 0, 0, 0);
  }
};

// bf16 query, fp8 e4m3fn cache (x = 16): codes are converted to bf16 in
// registers (exact); k_scale and v_scale are applied as scalars outside.
// The V side is common to every head size.
template <int D, int BS>
struct Fp8VPart {
  static constexpr int kBS = BS;
  static constexpr int kKvElemBytes = 1;
  static constexpr int kSub = BS / 16;
  static constexpr int kDt = D / 16;
  using VVec = typename Pick<BS == 16, unsigned, u32x2>::type;   // 4 codes per dword
  using VRegs = VVec[kDt];
  using QElem = __bf16;
  using OutElem = __bf16;
  struct Lane { uint32_t k, v; };

  // Dword of sub-tile st: codes of tokens tile_token(st, q4, 0..3).
  __device__ static unsigned vword(const VVec& w, int st) {
    if constexpr (BS == 16) return w;
    else return w[st];
  }
  __device__ static void set_vword(VVec& w, int st, unsigned x) {
    if constexpr (BS == 16) w = x;
    else w[st] = x;
  }
  // lane (i + 16*q4) of tile dt reads BS/4 consecutive codes of d = 16*dt + i.
  __device__ static uint32_t v_offset(int lane) { return (uint32_t)((lane & 15) * BS + (lane >> 4) * (BS / 4)); }
  __device__ static void load_v(const char* t, const Lane& lo, VRegs& v) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
      v[dt] = __builtin_nontemporal_load(reinterpret_cast<const VVec*>(t + lo.v + dt * 16 * BS));
  }
  __device__ static void prepare_v(VRegs& v) {
    if constexpr (BS == 32) {
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) {
        unsigned w0 = v[dt][0], w1 = v[dt][1];
        split_rows(w0, w1);
        v[dt] = VVec{w0, w1};
      }
    }
  }
  __device__ static void mask_v(VRegs& v, int q4, int nvalid) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
      for (int st = 0; st < kSub; ++st) {
        unsigned x = vword(v[dt], st);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (tile_token<BS>(st, q4, u) >= nvalid) x &= ~(0xFFu << (8 * u));
        set_vword(v[dt], st, x);
      }
  }
  __device__ static void pv(const VRegs& v, f32x4 p, f32x4 (&o)[kDt], int st) {
    const s16x4 pb = pack_bf16x4(p);
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) {
      const unsigned w = vword(v[dt], st);
      u32x2 a;
      a[0] = fp8x2_to_bf16x2<false>(w);
      a[1] = fp8x2_to_bf16x2<true>(w);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), pb, o[dt], 0, 0, 0);
    }
  }
};

template <int D, int BS = 16>
struct PolicyFp8 : Fp8VPart<D, BS> {
  using Base = Fp8VPart<D, BS>;
  using Lane = typename Base::Lane;
  using QElem = typename Base::QElem;
  static constexpr int kSub = Base::kSub;
  static constexpr int kKLoads = D / 64;     // per sub-tile: 16 bytes = 16 d at one token
  using KRegs = u32x4[kSub][kKLoads];
  using QRegs = bf16x8[2 * kKLoads];

  __device__ static Lane lane_offsets(int lane) {
    const int q4 = lane >> 4, rho = lane & 15;
    return {(uint32_t)(q4 * BS * 16 + k_row_token<BS>(rho) * 16), Base::v_offset(lane)};
  }
  __device__ static void load_k(const char* t, const Lane& lo, KRegs& k) {
#pragma unroll
    for (int st = 0; st < kSub; ++st)
#pragma unroll
      for (int h = 0; h < kKLoads; ++h)
        k[st][h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(t + lo.k + h * 4 * BS * 16 + st * 128));
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
  __device__ static f32x4 qk(const KRegs& k, const QRegs& q, int st) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < kKLoads; ++h)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 a;
        a[0] = fp8x2_to_bf16x2<false>(k[st][h][2 * half]);
        a[1] = fp8x2_to_bf16x2<true>(k[st][h][2 * half]);
        a[2] = fp8x2_to_bf16x2<false>(k[st][h][2 * half + 1]);
        a[3] = fp8x2_to_bf16x2<true>(k[st][h][2 * half + 1]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), q[2 * h + half], acc, 0, 0, 0);
      }
    return acc;
  }
};

// Head size 32 with an fp8 cache: a token has only two 16-byte K chunks, so
// each lane quad reads half a chunk. Quad q4 takes d = 8*q4 .. 8*q4 + 7
// (chunk q4 >> 1, bytes 8*(q4 & 1)); one 16x16x32 step covers all 32 d.
template <int BS>
struct PolicyFp8<32, BS> : Fp8VPart<32, BS> {
  using Base = Fp8VPart<32, BS>;
  using Lane = typename Base::Lane;
  using QElem = typename Base::QElem;
  static constexpr int kSub = Base::kSub;
  using KRegs = u32x2[kSub][1];
  using QRegs = bf16x8[1];

  __device__ static Lane lane_offsets(int lane) {
    const int q4 = lane >> 4, rho = lane & 15;
    return {(uint32_t)((q4 >> 1) * BS * 16 + k_row_token<BS>(rho) * 16 + (q4 & 1) * 8), Base::v_offset(lane)};
  }
  __device__ static void load_k(const char* t, const Lane& lo, KRegs& k) {
#pragma unroll
    for (int st = 0; st < kSub; ++st)
      k[st][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(t + lo.k + st * 128));
  }
  __device__ static void load_q(const QElem* qh, bool active, int q4, QRegs& q) {
    u32x4 w = {0, 0, 0, 0};
    if (active) w = *reinterpret_cast<const u32x4*>(qh + 8 * q4);
    q[0] = __builtin_bit_cast(bf16x8, w);
  }
  __device__ static f32x4 qk(const KRegs& k, const QRegs& q, int st) {
    u32x4 a;
    a[0] = fp8x2_to_bf16x2<false>(k[st][0][0]);
    a[1] = fp8x2_to_bf16x2<true>(k[st][0][0]);
    a[2] = fp8x2_to_bf16x2<false>(k[st][0][1]);
    a[3] = fp8x2_to_bf16x2<true>(k[st][0][1]);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), q[0], f32x4{0.f, 0.f, 0.f, 0.f},
                                                   0, 0, 0);
  }
};

// bf16 query, fp8 e4m3fn cache, fp8 arithmetic (the pages' fp8-compute
// variant, 10100.com §4: the decode runs on fp8 operands and converts once
// at the output). q is quantised to MX fp8 (blocks of 32 consecutive head
// dims, one power-of-two scale each); S = K q^T runs on the block-scaled
// v_mfma_scale_f32_16x16x128_f8f6f4, whose B scales carry q's MX exponents,
// and O += V^T P on v_mfma_f32_16x16x32_fp8_fp8. Each block's P is quantised
// to e4m3 relative to 2^ceil(block max); no operand is converted to a wider
// type.
//
// Operand layout of the 16x16x128 MFMA (checked on the GPU with a one-wave
// probe): lane (i + 16*q4) supplies k = 16*q4 + j from bytes j = 0..15 and
// k = 64 + 16*q4 + (j - 16) from bytes 16..31; the scale of row i, k-block b
// (32 consecutive k) comes from lane (i + 16*b). With d = k, lane quad q4's
// bytes are K chunks q4 and 4 + q4 (the 16-byte loads of PolicyFp8) and its
// scale is that of q's MX block q4.
typedef int i32x8 __attribute__((ext_vector_type(8)));

// E4M3FN code of y: nearest, ties to even, magnitude saturated at 448,
// NaN -> 0x7F, sign kept.
__device__ __forceinline__ unsigned e4m3_code(float y) {
  if (__builtin_isnan(y)) return 0x7Fu;
  const float mag = fminf(__builtin_fabsf(y), 448.0f);
  const unsigned c = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(mag, 0.0f, 0, false) & 0x7Fu;
  return c | ((__float_as_uint(y) >> 24) & 0x80u);
}

// MX shared exponent of a block with largest magnitude amax (OCP MX rule for
// e4m3, whose largest power of two is 2^8): floor(log2 amax) - 8, clamped to
// the e8m0 range; -127 for an all-zero block, 127 for an infinite amax.
__device__ __forceinline__ int mx_exponent(float amax) {
  if (amax == 0.f) return -127;
  if (__builtin_isinf(amax)) return 127;
  const int e = __builtin_amdgcn_frexp_expf(amax) - 1 - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

template <int D, int BS = 16>
struct PolicyFp8Mx : Fp8VPart<D, BS> {
  using Base = Fp8VPart<D, BS>;
  using Lane = typename Base::Lane;
  using QElem = typename Base::QElem;
  using VRegs = typename Base::VRegs;
  static constexpr bool kFp8Math = true;
  static constexpr int kSub = Base::kSub;
  static constexpr int kDt = Base::kDt;
  static constexpr int kKLoads = D == 128 ? 2 : 1;
  using KRegs = u32x4[kSub][kKLoads];
  struct QRegs {
    i32x8 codes;   // MX e4m3 codes of this lane's 32 k slots
    int scale;     // e8m0 scale of q's MX block q4
  };

  // Lane quad q4 reads K chunk q4 (and 4 + q4 at D = 128). At D = 32 only
  // chunks 0 and 1 exist: quads 2 and 3 re-read chunk q4 & 1, which their
  // zero q codes cancel.
  __device__ static Lane lane_offsets(int lane) {
    const int q4 = lane >> 4, rho = lane & 15;
    const int chunk = D == 32 ? (q4 & 1) : q4;
    return {(uint32_t)(chunk * BS * 16 + k_row_token<BS>(rho) * 16), Base::v_offset(lane)};
  }
  __device__ static void load_k(const char* t, const Lane& lo, KRegs& k) {
#pragma unroll
    for (int st = 0; st < kSub; ++st)
#pragma unroll
      for (int h = 0; h < kKLoads; ++h)
        k[st][h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(t + lo.k + h * 4 * BS * 16 + st * 128));
  }

  // Quantise the lane's slots of q (d = 16*q4 + j and, at D = 128,
  // 64 + 16*q4 + j) with the exponent of the MX block each belongs to; quads
  // 2k and 2k+1 together hold a block, so one exchange gives its amax.
  __device__ static void load_q(const QElem* qh, bool active, int q4, QRegs& q) {
    float a[16], b[16];
    const bool has_a = active && 16 * q4 < D, has_b = active && D == 128;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 wa = {0, 0, 0, 0}, wb = {0, 0, 0, 0};
      if (has_a) wa = *reinterpret_cast<const u32x4*>(qh + 16 * q4 + 8 * h);
      if (has_b) wb = *reinterpret_cast<const u32x4*>(qh + 64 + 16 * q4 + 8 * h);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[8 * h + 2 * u] = __uint_as_float(wa[u] << 16);
        a[8 * h + 2 * u + 1] = __uint_as_float(wa[u] & 0xFFFF0000u);
        b[8 * h + 2 * u] = __uint_as_float(wb[u] << 16);
        b[8 * h + 2 * u + 1] = __uint_as_float(wb[u] & 0xFFFF0000u);
      }
    }
    float ma = 0.f, mb = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      ma = fmaxf(ma, __builtin_fabsf(a[j]));
      mb = fmaxf(mb, __builtin_fabsf(b[j]));
    }
    ma = fmaxf(ma, __shfl_xor(ma, 16, 64));
    mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
    const int xa = mx_exponent(ma), xb = mx_exponent(mb);   // blocks q4 >> 1 and 2 + (q4 >> 1)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      unsigned ca = 0, cb = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        ca |= e4m3_code(__builtin_ldexpf(a[4 * w + u], -xa)) << (8 * u);
        cb |= e4m3_code(__builtin_ldexpf(b[4 * w + u], -xb)) << (8 * u);
      }
      q.codes[w] = (int)ca;
      q.codes[4 + w] = (int)cb;
    }
    // Block q4's exponent: quad 0 holds block 0 (its a), quad 3 block 3 (its
    // b); block 1 is quad 2's a, block 2 quad 1's b.
    const int lane = threadIdx.x & 63;
    const int from_up = __shfl(xa, (lane + 16) & 63, 64);
    const int from_down = __shfl(xb, (lane + 48) & 63, 64);
    const int x = q4 == 0 ? xa : q4 == 1 ? from_up : q4 == 2 ? from_down : xb;
    q.scale = 32 * q4 < D ? 127 + x : 127;
  }
  __device__ static f32x4 qk(const KRegs& k, const QRegs& q, int st) {
    i32x8 a = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 4; ++u) a[u] = (int)k[st][0][u];
    if constexpr (kKLoads == 2) {
#pragma unroll
      for (int u = 0; u < 4; ++u) a[4 + u] = (int)k[st][1][u];
    }
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, q.codes, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0,
                                                            q.scale);
  }
  // O += 2^e * V^T P on v_mfma_f32_16x16x32_fp8_fp8 (k = 8*q4 + j from byte j
  // of lane quad q4): bytes 0-3 of A and B are sub-tile 0's four rows of the
  // quad, bytes 4-7 sub-tile 1's (zero with 16-token blocks). Each block's
  // product is formed from zero and added to O in fp32 with the exact factor
  // 2^e, so the sum over blocks is an fp32 sum.
  __device__ static void pv8(const VRegs& v, unsigned p0, unsigned p1, float f, f32x4 (&o)[kDt]) {
    const long b = (long)(((unsigned long)p1 << 32) | p0);
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) {
      const unsigned w1 = kSub == 2 ? Base::vword(v[dt], kSub - 1) : 0u;
      const long a = (long)(((unsigned long)w1 << 32) | Base::vword(v[dt], 0));
      const f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) o[dt][r] = fmaf(t[r], f, o[dt][r]);
    }
  }
};

// Whether a policy runs the fp8 arithmetic (PolicyFp8Mx).
template <typename P, typename = void> struct Fp8Math { static constexpr bool value = false; };
template <typename P> struct Fp8Math<P, decltype((void)P::kFp8Math)> { static constexpr bool value = P::kFp8Math; };

// fp8 arithmetic, one block of one query column tile: P is quantised to e4m3
// relative to mb = ceil(block max mx) (so every p <= 1), multiplied with V on
// fp8 operands, and brought to the running reference m by the exact factor
// 2^(mb - m); m stays an integer and is raised lazily like the other paths'.
template <typename P>
__device__ __forceinline__ void fp8_block_update(const typename P::VRegs& vr, const f32x4 (&z)[P::kSub], float mx,
                                                 float& m, float& lsum, f32x4 (&o)[P::kDt]) {
  const float mb = ceilf(mx);
  if (wave_any(mb > m + kRescaleSlack)) {
    const float m_new = fmaxf(m, mb);
    const float alpha = m == kNegInf ? 0.f : __builtin_ldexpf(1.f, (int)(m - m_new));
    m = m_new;
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < P::kDt; ++dt) o[dt] *= alpha;
  }
  unsigned pw[2] = {0u, 0u};
  float s = 0.f;
#pragma unroll
  for (int st = 0; st < P::kSub; ++st) {
    f32x4 p;
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fast_exp2(z[st][r] - mb);
    unsigned w = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
    w = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], (int)w, true);
    pw[st] = w;
    s += (__builtin_amdgcn_cvt_f32_fp8((int)w, 0) + __builtin_amdgcn_cvt_f32_fp8((int)w, 1)) +
         (__builtin_amdgcn_cvt_f32_fp8((int)w, 2) + __builtin_amdgcn_cvt_f32_fp8((int)w, 3));
  }
  const int e = (int)(mb - m);
  P::pv8(vr, pw[0], pw[1], __builtin_ldexpf(1.f, e), o);
  lsum += __builtin_ldexpf(s, e);
}

// ---------------------------------------------------------------------------
// One wave's attention over a run of blocks of one (sequence, kv head).
// ---------------------------------------------------------------------------

template <typename P, int D, int NB, bool ALIBI>
struct WaveAttn {
  static constexpr int kDt = P::kDt;
  static constexpr int kBS = P::kBS;      // tokens per block (tile)
  static constexpr int kSub = P::kSub;    // 16-row sub-tiles per tile
  typename P::QRegs q;
  typename P::Lane lo;
  f32x4 o[kDt];
  float m, m_true, lsum;
  float c, slope2;
  float lane_bias[4];   // slope2 * (token of row 4*q4 + r in sub-tile 0), ALiBi only
  int lane, q4;
  bool active;          // this lane's column g is a real query head

  // Query rows of heads kvh*G + g (zero for padded columns g >= G).
  __device__ void begin(const DecodeArgs& a, int seq, int kvh) {
    init_lane(a);
    float sl;
    load_pair_q(a, seq, kvh, q, sl);
    reset(sl);
  }

  // The part of the set-up that is the same for every (sequence, kv head).
  __device__ void init_lane(const DecodeArgs& a) {
    lane = threadIdx.x & 63;
    q4 = lane >> 4;
    active = (lane & 15) < a.group;
    lo = P::lane_offsets(lane);
    float k_scale = 1.f;
    if (a.k_scale) k_scale = *a.k_scale;
    c = a.scale * kLog2e * k_scale;
  }

  // q rows of the pair's query heads into qq, and this column's ALiBi slope
  // (log2 units; 0 without ALiBi) into sl.
  __device__ void load_pair_q(const DecodeArgs& a, int seq, int kvh, typename P::QRegs& qq, float& sl) const {
    const int h = kvh * a.group + (active ? (lane & 15) : 0);
    const auto* qh = reinterpret_cast<const typename P::QElem*>(a.query) + ((int64_t)seq * a.num_heads + h) * D;
    P::load_q(qh, active, q4, qq);
    sl = 0.f;
    if constexpr (ALIBI) {
      if (active) sl = a.alibi_slopes[h] * kLog2e;
    }
  }

  // Empty softmax state for a new pair with ALiBi slope sl.
  __device__ void reset(float sl) {
    slope2 = sl;
    if constexpr (ALIBI) {
#pragma unroll
      for (int r = 0; r < 4; ++r) lane_bias[r] = slope2 * (float)tile_token<kBS>(0, q4, r);
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
    constexpr int kShift = kBS == 32 ? 5 : 4;
    const int last_blk = (L - 1) >> kShift;
    const int tail = L - (last_blk << kShift);           // valid slots in the last block, 1..kBS
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
    f32x4 z[NB][kSub];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (j < n) {
        P::prepare_v(vr[j]);
        const int blk = g0 + j;
#pragma unroll
        for (int st = 0; st < kSub; ++st) {
          const f32x4 s = P::qk(kr[j], q, st);
          if constexpr (ALIBI) {
            const float base = (float)(blk * kBS + 8 * st - (L - 1));
#pragma unroll
            for (int r = 0; r < 4; ++r) z[j][st][r] = fmaf(s[r], c, fmaf(slope2, base, lane_bias[r]));
          } else {
            z[j][st] = s * c;
          }
        }
        if (blk == last_blk && tail < kBS) {
#pragma unroll
          for (int st = 0; st < kSub; ++st)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (tile_token<kBS>(st, q4, r) >= tail) z[j][st][r] = kNegInf;
          P::mask_v(vr[j], q4, tail);
        }
#pragma unroll
        for (int st = 0; st < kSub; ++st) mx = fmaxf(mx, max4(z[j][st]));
      }
    }
    mx = quad_max(mx);
    m_true = fmaxf(m_true, mx);
    if constexpr (Fp8Math<P>::value) {
      consume_fp8(vr[0], z[0], mx);
    } else {
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
#pragma unroll
          for (int st = 0; st < kSub; ++st) {
            f32x4 p;
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = fast_exp2(z[j][st][r] - m);
            lsum += (p[0] + p[1]) + (p[2] + p[3]);
            P::pv(vr[j], p, o, st);
          }
        }
      }
    }
  }

  __device__ void consume_fp8(const typename P::VRegs& vr, const f32x4 (&z)[kSub], float mx) {
    static_assert(NB == 1, "the fp8 arithmetic takes one block per issue");
    fp8_block_update<P>(vr, z, mx, m, lsum, o);
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
  constexpr int kBS = P::kBS;
  const int first = a.first_block ? min(max(a.first_block[seq], 0), min(L / kBS, a.max_first_block)) : 0;
  const int t0 = first * kBS;
  const int t_begin = t0 + split * a.split_tokens;
  if (t_begin >= L) return;
  const int b0 = t_begin / kBS;
  const int b1 = min((L + kBS - 1) / kBS, (t_begin + a.split_tokens) / kBS);
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
