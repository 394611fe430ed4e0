// KV-cache append for gfx950: store the new tokens' K and V rows in the
// paged cache, the step that precedes attention in every decode iteration
// (the cache grows one token per step; vLLM 0.25.0 解读 §1). Token j of
// sequence s goes to logical position p = positions[s] + j, i.e. physical
// block block_tables[s, p / B], slot p % B for blocks of B = 16 or 32 tokens
// (10100.com retirement article, §1), in the pages' layouts (same article, §2):
//   K [num_blocks][num_kv_heads][D/x][B][x],  V [num_blocks][num_kv_heads][D][B].
// With an fp8 cache each element is stored as the E4M3FN code nearest to
// x / scale (ties to even, saturating at 448; same article, §4, for the
// scaled fp8 storage).
//
// One wave per (sequence, kv head, physical block touched): the wave stores
// the run of new tokens that falls in that block. The run's input rows are
// read along the rows into LDS first; the stores then walk the run with the
// token index fastest, so each store instruction covers consecutive slots:
// for K, 16-byte rows of one chunk (contiguous 16*run bytes); for V, elements
// of one dim row (contiguous run*elem bytes). A single token per block (the
// decode step) can only write 16-byte K pieces and single V elements.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_kernels.h"

namespace pa {

namespace {

typedef unsigned u32x4a __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(unsigned short b) { return __uint_as_float((unsigned)b << 16); }

// E4M3FN code of v / scale: IEEE float32 quotient, nearest code with ties to
// even (the hardware conversion rounds to nearest even), magnitude saturated
// at 448, NaN -> 0x7F, sign bit taken from the quotient.
__device__ __forceinline__ unsigned quant_e4m3(float v, float scale) {
  const float y = v / scale;
  if (__builtin_isnan(y)) return 0x7Fu;
  const float mag = fminf(__builtin_fabsf(y), 448.0f);
  const unsigned c = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(mag, 0.0f, 0, false) & 0x7Fu;
  return c | ((__float_as_uint(y) >> 24) & 0x80u);
}

template <int KIND, int D>
struct AppendPolicy;

// f32 input, f32 cache (x = 4) and bf16 input, bf16 cache (x = 8): copies.
template <int D>
struct AppendPolicy<KIND_F32, D> {
  using In = float;
  static constexpr int kX = 4;
  static constexpr int kElem = 4;
  __device__ static void k_chunk(const In* src, char* dst, float) {
    *reinterpret_cast<u32x4a*>(dst) = *reinterpret_cast<const u32x4a*>(src);
  }
  __device__ static void v_elem(const In* src, char* dst, float) { *reinterpret_cast<float*>(dst) = *src; }
};

template <int D>
struct AppendPolicy<KIND_BF16, D> {
  using In = unsigned short;
  static constexpr int kX = 8;
  static constexpr int kElem = 2;
  __device__ static void k_chunk(const In* src, char* dst, float) {
    *reinterpret_cast<u32x4a*>(dst) = *reinterpret_cast<const u32x4a*>(src);
  }
  __device__ static void v_elem(const In* src, char* dst, float) {
    *reinterpret_cast<unsigned short*>(dst) = *src;
  }
};

// fp8 cache (x = 16) from bf16 or f32 input.
template <typename InT>
struct QuantPolicy {
  using In = InT;
  static constexpr int kX = 16;
  static constexpr int kElem = 1;
  __device__ static float val(In v) {
    if constexpr (sizeof(In) == 4) return v;
    else return bf16_to_f32(v);
  }
  // src is 16-byte aligned: token rows are multiples of 128 bytes apart and
  // chunks 16 elements apart.
  __device__ static void k_chunk(const In* src, char* dst, float scale) {
    constexpr int kVec = 16 / sizeof(In);                 // elements per 16-byte load
    In v[16];
#pragma unroll
    for (int q = 0; q < 16 / kVec; ++q)
      *reinterpret_cast<u32x4a*>(v + q * kVec) = *reinterpret_cast<const u32x4a*>(src + q * kVec);
    u32x4a w = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) w[e >> 2] |= quant_e4m3(val(v[e]), scale) << (8 * (e & 3));
    *reinterpret_cast<u32x4a*>(dst) = w;
  }
  __device__ static void v_elem(const In* src, char* dst, float scale) {
    *reinterpret_cast<unsigned char*>(dst) = (unsigned char)quant_e4m3(val(*src), scale);
  }
};

// Orders this wave's LDS writes before its later LDS reads (each wave owns
// its own LDS tile, so no workgroup barrier is involved).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One workgroup = one wave per (sequence, kv head, physical block touched).
// The run's token rows are first staged through LDS with 16-byte loads along
// each row (consecutive lanes, consecutive bytes); the cache stores then read
// their elements from LDS. Reading the input directly in the stores' lane
// order (token fastest) would make every lane of a V store load from a
// different row.
template <typename Pol, int D>
__global__ void __launch_bounds__(64) pa_append_kernel(const AppendArgs a, int runs_per_pair) {
  using In = typename Pol::In;
  constexpr int kChunks = D / Pol::kX;
  constexpr int kRow = D * (int)sizeof(In);               // bytes of one token row
  constexpr int kPitch = kRow + 16;                       // LDS row pitch, spreads banks
  constexpr int kPieces = kRow / 16;
  __shared__ __align__(16) char ktile[32 * kPitch];       // one run: at most 32 tokens
  __shared__ __align__(16) char vtile[32 * kPitch];
  const int lane = threadIdx.x;
  const int64_t item = blockIdx.x;
  const int r = (int)(item % runs_per_pair);
  const int64_t sh = item / runs_per_pair;                // s * Hkv + h
  const int h = (int)(sh % a.num_kv_heads);
  const int s = (int)(sh / a.num_kv_heads);
  const int p0 = a.positions[s];
  if (p0 < 0) return;
  const int bs = a.block_size;                            // 16 or 32 tokens
  const int64_t blk = (int64_t)(p0 / bs) + r;             // logical block of this run
  const int64_t t_lo = blk * bs > p0 ? blk * bs : (int64_t)p0;
  const int64_t p_end = (int64_t)p0 + a.tokens_per_seq;
  const int64_t t_hi = (blk + 1) * bs < p_end ? (blk + 1) * bs : p_end;
  if (t_lo >= t_hi || blk >= a.max_blocks_per_seq) return;
  const int b = a.block_tables[(int64_t)s * a.max_blocks_per_seq + blk];
  if (b < 0 || b >= a.num_blocks) return;
  const int o0 = (int)(t_lo - blk * bs);                  // first slot
  const int n = (int)(t_hi - t_lo);                       // tokens in this run, 1..bs
  const int j0 = (int)(t_lo - p0);                        // their first index among the new tokens
  const int64_t tile_bytes = (int64_t)D * bs * Pol::kElem;
  const int64_t base = ((int64_t)b * a.num_kv_heads + h) * tile_bytes;
  const int64_t row_stride = (int64_t)a.num_kv_heads * kRow;   // bytes between consecutive tokens
  const int64_t row0 = ((int64_t)s * a.tokens_per_seq + j0) * row_stride + (int64_t)h * kRow;
  const char* krow = reinterpret_cast<const char*>(a.key) + row0;
  const char* vrow = reinterpret_cast<const char*>(a.value) + row0;
  const float ks = a.k_scale ? *a.k_scale : 1.f;
  const float vs = a.v_scale ? *a.v_scale : 1.f;
  char* kc = reinterpret_cast<char*>(a.key_cache) + base;
  char* vc = reinterpret_cast<char*>(a.value_cache) + base;
  // K and V rows of the run are loaded together (one round trip to memory).
  for (int i = lane; i < n * kPieces; i += 64) {
    const int t = i / kPieces, piece = i - t * kPieces;
    const int64_t src = t * row_stride + piece * 16;
    const int dst = t * kPitch + piece * 16;
    *reinterpret_cast<u32x4a*>(ktile + dst) = *reinterpret_cast<const u32x4a*>(krow + src);
    *reinterpret_cast<u32x4a*>(vtile + dst) = *reinterpret_cast<const u32x4a*>(vrow + src);
  }
  wave_sync();
  // K: item i = c * n + t -> chunk c of token t, 16 bytes at row o0 + t.
  for (int i = lane; i < kChunks * n; i += 64) {
    const int c = i / n, t = i - c * n;
    Pol::k_chunk(reinterpret_cast<const In*>(ktile + t * kPitch) + c * Pol::kX,
                 kc + ((int64_t)c * bs + o0 + t) * 16, ks);
  }
  // V: item i = d * n + t -> element d of token t at row d, slot o0 + t.
  for (int i = lane; i < D * n; i += 64) {
    const int d = i / n, t = i - d * n;
    Pol::v_elem(reinterpret_cast<const In*>(vtile + t * kPitch) + d, vc + ((int64_t)d * bs + o0 + t) * Pol::kElem,
                vs);
  }
}

template <typename Pol, int D>
hipError_t launch_append_t(const AppendArgs& a, hipStream_t stream) {
  // A run of T tokens starting anywhere in a block of B tokens touches at
  // most floor((B - 1 + T - 1) / B) + 1 blocks.
  const int bs = a.block_size;
  const int runs = (bs - 1 + a.tokens_per_seq - 1) / bs + 1;
  const int64_t items = (int64_t)a.num_seqs * a.num_kv_heads * runs;
  hipLaunchKernelGGL((pa_append_kernel<Pol, D>), dim3((unsigned)items), dim3(64), 0, stream, a, runs);
  return hipGetLastError();
}

// Latent rows (one compressed row [c_kv 512, k_rope 64] per token, bf16):
// one wave per (sequence, physical block touched). Chunk c (8 bf16 or 16
// fp8 codes, 16 bytes) of slot o sits at byte (B*c + o)*16 of a block of B
// tokens, so with the slot index fastest a run of n tokens is 72 (36)
// contiguous stores of 16*n bytes; the loads then take one chunk's elements
// of each row per lane, n rows side by side. The decode step (n = 1) reads
// its row contiguously and writes pieces 16 B bytes apart, which the layout
// fixes. fp8 codes are those of the K/V append (quant_e4m3).
template <bool FP8>
__global__ void __launch_bounds__(64) pa_latent_append_kernel(const LatentAppendArgs a, int runs_per_seq) {
  constexpr int kRow = 1152;
  constexpr int kChunks = FP8 ? 36 : 72;
  const int bs = a.block_size;                             // 16 or 32 tokens
  const int64_t block_bytes = (int64_t)kChunks * bs * 16;
  const int r = (int)(blockIdx.x % (unsigned)runs_per_seq);
  const int s = (int)(blockIdx.x / (unsigned)runs_per_seq);
  const int p0 = a.positions[s];
  if (p0 < 0) return;
  const int64_t blk = (int64_t)(p0 / bs) + r;
  const int64_t t_lo = blk * bs > p0 ? blk * bs : (int64_t)p0;
  const int64_t p_end = (int64_t)p0 + a.tokens_per_seq;
  const int64_t t_hi = (blk + 1) * bs < p_end ? (blk + 1) * bs : p_end;
  if (t_lo >= t_hi || blk >= a.max_blocks_per_seq) return;
  const int b = a.block_tables[(int64_t)s * a.max_blocks_per_seq + blk];
  if (b < 0 || b >= a.num_blocks) return;
  const int o0 = (int)(t_lo - blk * bs);
  const int n = (int)(t_hi - t_lo);
  const char* src = reinterpret_cast<const char*>(a.rows) + ((int64_t)s * a.tokens_per_seq + (t_lo - p0)) * kRow;
  char* dst = reinterpret_cast<char*>(a.latent_cache) + (int64_t)b * block_bytes + o0 * 16;
  const float vs = (FP8 && a.kv_scale) ? *a.kv_scale : 1.f;
  for (int i = threadIdx.x; i < kChunks * n; i += 64) {
    const int c = i / n, t = i - c * n;
    if constexpr (FP8) {
      QuantPolicy<unsigned short>::k_chunk(reinterpret_cast<const unsigned short*>(src + t * kRow + c * 32),
                                           dst + (c * bs + t) * 16, vs);
    } else {
      *reinterpret_cast<u32x4a*>(dst + (c * bs + t) * 16) =
          *reinterpret_cast<const u32x4a*>(src + t * kRow + c * 16);
    }
  }
}

// Copy-on-write support: pair blockIdx.x copies physical block src -> dst in
// both caches, 16 bytes per lane, workgroups along y splitting the block.
__global__ void __launch_bounds__(256) pa_copy_blocks_kernel(char* key_cache, char* value_cache,
                                                             const int32_t* src, const int32_t* dst,
                                                             int num_blocks, int64_t block_bytes) {
  const int32_t s = src[blockIdx.x], d = dst[blockIdx.x];
  if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) return;
  const int64_t so = (int64_t)s * block_bytes, dof = (int64_t)d * block_bytes;
  for (int64_t off = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 16; off < block_bytes;
       off += (int64_t)gridDim.y * 256 * 16) {
    *reinterpret_cast<u32x4a*>(key_cache + dof + off) = *reinterpret_cast<const u32x4a*>(key_cache + so + off);
    *reinterpret_cast<u32x4a*>(value_cache + dof + off) = *reinterpret_cast<const u32x4a*>(value_cache + so + off);
  }
}

}  // namespace

hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int32_t* src, const int32_t* dst,
                              int num_pairs, int num_blocks, size_t block_bytes, hipStream_t stream) {
  const int64_t per_wg = 256 * 16 * 4;                    // bytes per workgroup pass
  const int64_t gy64 = ((int64_t)block_bytes + per_wg - 1) / per_wg;
  const unsigned gy = (unsigned)(gy64 < 1024 ? gy64 : 1024);
  hipLaunchKernelGGL(pa_copy_blocks_kernel, dim3(num_pairs, gy), dim3(256), 0, stream,
                     static_cast<char*>(key_cache), static_cast<char*>(value_cache), src, dst, num_blocks,
                     (int64_t)block_bytes);
  return hipGetLastError();
}

hipError_t launch_latent_append(const LatentAppendArgs& a, hipStream_t stream) {
  // As for the K/V append: T tokens touch at most floor((B - 2 + T) / B) + 1
  // blocks of B tokens.
  const int bs = a.block_size;
  const int runs = (bs - 2 + a.tokens_per_seq) / bs + 1;
  const int64_t items = (int64_t)a.num_seqs * runs;
  if (a.fp8)
    hipLaunchKernelGGL((pa_latent_append_kernel<true>), dim3((unsigned)items), dim3(64), 0, stream, a, runs);
  else
    hipLaunchKernelGGL((pa_latent_append_kernel<false>), dim3((unsigned)items), dim3(64), 0, stream, a, runs);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, int in_kind, int cache_kind, hipStream_t stream) {
  const int key = (in_kind * 10 + cache_kind) * 1000 + a.head_size;
  switch (key) {
    case (KIND_F32 * 10 + KIND_F32) * 1000 + 32: return launch_append_t<AppendPolicy<KIND_F32, 32>, 32>(a, stream);
    case (KIND_F32 * 10 + KIND_F32) * 1000 + 64: return launch_append_t<AppendPolicy<KIND_F32, 64>, 64>(a, stream);
    case (KIND_F32 * 10 + KIND_F32) * 1000 + 128: return launch_append_t<AppendPolicy<KIND_F32, 128>, 128>(a, stream);
    case (KIND_BF16 * 10 + KIND_BF16) * 1000 + 32: return launch_append_t<AppendPolicy<KIND_BF16, 32>, 32>(a, stream);
    case (KIND_BF16 * 10 + KIND_BF16) * 1000 + 64: return launch_append_t<AppendPolicy<KIND_BF16, 64>, 64>(a, stream);
    case (KIND_BF16 * 10 + KIND_BF16) * 1000 + 128: return launch_append_t<AppendPolicy<KIND_BF16, 128>, 128>(a, stream);
    case (KIND_BF16 * 10 + KIND_FP8) * 1000 + 32: return launch_append_t<QuantPolicy<unsigned short>, 32>(a, stream);
    case (KIND_BF16 * 10 + KIND_FP8) * 1000 + 64: return launch_append_t<QuantPolicy<unsigned short>, 64>(a, stream);
    case (KIND_BF16 * 10 + KIND_FP8) * 1000 + 128: return launch_append_t<QuantPolicy<unsigned short>, 128>(a, stream);
    case (KIND_F32 * 10 + KIND_FP8) * 1000 + 32: return launch_append_t<QuantPolicy<float>, 32>(a, stream);
    case (KIND_F32 * 10 + KIND_FP8) * 1000 + 64: return launch_append_t<QuantPolicy<float>, 64>(a, stream);
    case (KIND_F32 * 10 + KIND_FP8) * 1000 + 128: return launch_append_t<QuantPolicy<float>, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
