// Internal interface between the C-ABI host code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Tuning knobs (compile-time): waves per workgroup, blocks per wave
// iteration for each cache type, stream-K waves per compute unit.
#ifndef PA_WAVES
#define PA_WAVES 4
#endif
#ifndef PA_NB_BF16
#define PA_NB_BF16 1
#endif
#ifndef PA_NB_FP8
#define PA_NB_FP8 1
#endif
#ifndef PA_NB_F32
#define PA_NB_F32 1
#endif
#ifndef PA_SK_WAVES_PER_CU_BF16
#define PA_SK_WAVES_PER_CU_BF16 4
#endif
#ifndef PA_SK_WAVES_PER_CU_FP8
#define PA_SK_WAVES_PER_CU_FP8 8
#endif
#ifndef PA_SK_WAVES_PER_CU_F32
#define PA_SK_WAVES_PER_CU_F32 4
#endif
#ifndef PA_PIPE
#define PA_PIPE 1
#endif
#ifndef PA_SK_WAVES_PER_CU_FP8MX
#define PA_SK_WAVES_PER_CU_FP8MX 8
#endif
#ifndef PA_SK_WAVES_PER_CU_BS32_FP8MX
#define PA_SK_WAVES_PER_CU_BS32_FP8MX 4
#endif
// 32-token blocks: stream-K waves per compute unit.
#ifndef PA_SK_WAVES_PER_CU_BS32_BF16
#define PA_SK_WAVES_PER_CU_BS32_BF16 3
#endif
#ifndef PA_SK_WAVES_PER_CU_BS32_FP8
#define PA_SK_WAVES_PER_CU_BS32_FP8 4
#endif
#ifndef PA_SK_WAVES_PER_CU_BS32_F32
#define PA_SK_WAVES_PER_CU_BS32_F32 PA_SK_WAVES_PER_CU_F32
#endif
// Upper bound on stream-K waves; sizes the segment workspace.
#define PA_SK_MAX_WAVES 4096
// MLA stream-K waves per compute unit (each wave needs more than 256
// registers per lane, so one per SIMD).
#ifndef PA_MLA_WAVES_PER_CU
#define PA_MLA_WAVES_PER_CU 4
#endif

namespace pa {

// KIND_FP8MX: fp8 cache with fp8 arithmetic (MX-scaled q, e4m3 P).
enum Kind { KIND_F32 = 0, KIND_BF16 = 1, KIND_FP8 = 2, KIND_FP8MX = 3 };

// Everything a launch needs, passed by value as the kernel argument.
struct DecodeArgs {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const float* alibi_slopes;   // nullable
  const float* k_scale;        // nullable (1.0)
  const float* v_scale;        // nullable (1.0)
  // split grid (streamk_workgroups == 0), num_splits > 1 only:
  float* tmp_out;              // [S][H][num_splits][D]
  float* max_logits;           // [S][H][num_splits]
  float* exp_sums;             // [S][H][num_splits]
  // stream-K (streamk_workgroups > 0); slots = S*Hkv + PA_SK_MAX_WAVES:
  float* seg_out;              // [slots][G][D]  normalised segment output (times v_scale)
  float* seg_max;              // [slots][G]     segment running max (log2 units)
  float* seg_sum;              // [slots][G]     segment exp2-sum relative to seg_max
  int32_t* seg_meta;           // [S*Hkv][2]     first and last wave of each (kv head, sequence) pair
  int64_t k_block_stride_bytes;
  int64_t k_head_stride_bytes;
  int64_t v_block_stride_bytes;
  int64_t v_head_stride_bytes;
  float scale;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int group;
  int head_size;
  int block_size;              // tokens per physical block: 16 or 32
  int num_blocks;
  int max_blocks_per_seq;
  int max_seq_len;
  int split_tokens;
  int num_splits;
  int streamk_workgroups;      // > 0 selects the stream-K scheduler
  // split grid only: per-sequence count of leading physical blocks handled
  // elsewhere (a shared prefix), clamped to [0, min(L / block_size,
  // max_first_block)]; nullable. When set, every split writes partials and no
  // reduce runs.
  const int32_t* first_block;
  int max_first_block;
};

// Shared-prefix decode (pa_shared.hip): the members of a group map their
// first prefix blocks to the same physical blocks; the prefix is read once
// per group (all members' query heads as MFMA columns), the rest per
// sequence through the split grid with first_block, and a merge combines the
// partials.
struct SharedArgs {
  DecodeArgs d;                        // split plan over the suffixes (tmp_out, max_logits, exp_sums)
  const int32_t* group_start;          // [num_groups + 1] offsets into group_seqs
  const int32_t* group_seqs;           // [num_members] member sequence ids
  int num_members;
  const int32_t* group_prefix_blocks;  // [num_groups] shared full physical blocks
  int num_groups;
  int max_chunks;                      // chunks of members per group in the grid
  int members_per_chunk;
  int prefix_split_blocks;             // prefix blocks per wave
  int max_prefix_splits;
  float* pre_out;                      // [S][H][max_prefix_splits][D]
  float* pre_max;                      // [S][H][max_prefix_splits] natural-log units
  float* pre_sum;                      // [S][H][max_prefix_splits]
};

// Most 16-column query tiles a prefix wave carries: four, except at
// head_size 128 with fp32 queries, or with a bf16 cache in 32-token blocks,
// whose operands would not fit in registers.
constexpr int max_column_tiles(int q_elem_bytes, int kv_elem_bytes, int head_size, int block_size) {
  return (head_size == 128 && (q_elem_bytes == 4 || (kv_elem_bytes == 2 && block_size == 32))) ? 2 : 4;
}

hipError_t launch_shared(const SharedArgs& a, int kind, int column_tiles, hipStream_t stream);

// Arguments of the KV-cache append kernel (pa_append.hip).
struct AppendArgs {
  void* key_cache;
  void* value_cache;
  const void* key;             // [num_seqs][tokens_per_seq][num_kv_heads][head_size]
  const void* value;
  const int32_t* block_tables; // [num_seqs][max_blocks_per_seq]
  const int32_t* positions;    // [num_seqs]
  const float* k_scale;        // nullable (1.0), fp8 cache only
  const float* v_scale;
  int num_seqs;
  int tokens_per_seq;
  int num_kv_heads;
  int head_size;
  int block_size;              // tokens per cache block: 16 or 32
  int num_blocks;
  int max_blocks_per_seq;
};

hipError_t launch_append(const AppendArgs& a, int in_kind, int cache_kind, hipStream_t stream);

// Arguments of the latent-row append kernel (pa_append.hip): bf16 rows of
// 576 elements into the latent cache [num_blocks][72][block_size][8], or as
// e4m3fn codes of row / *kv_scale into [num_blocks][36][block_size][16].
struct LatentAppendArgs {
  void* latent_cache;
  const void* rows;            // [num_seqs][tokens_per_seq][576]
  const int32_t* block_tables; // [num_seqs][max_blocks_per_seq]
  const int32_t* positions;    // [num_seqs]
  const float* kv_scale;       // fp8 only, nullable (1.0)
  int fp8;
  int num_seqs;
  int tokens_per_seq;
  int num_blocks;
  int max_blocks_per_seq;
  int block_size;              // 16 or 32 tokens
};

hipError_t launch_latent_append(const LatentAppendArgs& a, hipStream_t stream);

// Whole-block copies src[i] -> dst[i] in both caches (pa_append.hip).
hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int32_t* src, const int32_t* dst,
                              int num_pairs, int num_blocks, size_t block_bytes, hipStream_t stream);

// Optional callbacks around each launch (used for event timing).
struct LaunchHooks {
  void (*before_partition)(hipStream_t) = nullptr;
  void (*after_partition)(hipStream_t) = nullptr;
  void (*before_reduce)(hipStream_t) = nullptr;
  void (*after_reduce)(hipStream_t) = nullptr;
};

hipError_t launch_decode(const DecodeArgs& a, int kind, hipStream_t stream, const LaunchHooks& hooks);

// Latent-cache (MLA) decode (pa_mla.hip). d carries the batch: key_cache is
// the latent cache, head_size the row width, group 16 (heads per wave),
// num_kv_heads 1; seg_* as for stream-K with slots [S + shares][hpad], except
// that seg_out holds bf16 rows.
struct MlaArgs {
  DecodeArgs d;
  int head_groups;    // head groups: ceil(num_heads / 16), or ceil(num_heads / 32) for the wide kernel
  int waves_per_wg;   // head groups per workgroup
  int chunks;         // workgroups per share
  int shares;         // stream-K shares (a multiple of 8 when chunks > 1)
  int hpad;           // rows per slot in the segment partials (head groups x heads per group)
  int wide;           // 1: pa_mla_wide_kernel (32 heads per wave, one workgroup per share)
  int fp8;            // 1: e4m3fn latent cache [num_blocks][36][16][16], scale *d.k_scale (nullable: 1)
};

hipError_t launch_mla(const MlaArgs& a, hipStream_t stream, const LaunchHooks& hooks);
// The 32-heads-per-wave kernel alone (pa_mla_wide.hip).
hipError_t launch_mla_wide(const MlaArgs& a, hipStream_t stream);

// Streaming read of `bytes` (a multiple of 16) from `buf` by `workgroups`
// workgroups of 256 threads (pa_probe.hip).
hipError_t launch_read_probe(const void* buf, uint64_t bytes, int workgroups, unsigned* sink, hipStream_t stream);

// Whole-tile gathers of `tile_bytes` tiles listed in `ids` (pa_probe.hip).
hipError_t launch_gather_probe(const void* pool, uint64_t pool_bytes, int tile_bytes, const int32_t* ids,
                               int num_tiles, int depth, int workgroups, unsigned* sink, hipStream_t stream);

}  // namespace pa
