// Internal interface between the C-ABI host code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define PA_MAX_GROUP_DEV 16

namespace pa {

enum Kind { KIND_F32 = 0, KIND_BF16 = 1, KIND_FP8 = 2 };

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
  float* tmp_out;              // [S][H][num_splits][D]   (num_splits > 1 only)
  float* max_logits;           // [S][H][num_splits]
  float* exp_sums;             // [S][H][num_splits]
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
  int num_blocks;
  int max_blocks_per_seq;
  int max_seq_len;
  int split_tokens;
  int num_splits;
};

// Optional callbacks around each launch (used for event timing).
struct LaunchHooks {
  void (*before_partition)(hipStream_t) = nullptr;
  void (*after_partition)(hipStream_t) = nullptr;
  void (*before_reduce)(hipStream_t) = nullptr;
  void (*after_reduce)(hipStream_t) = nullptr;
};

hipError_t launch_decode(const DecodeArgs& a, int kind, hipStream_t stream, const LaunchHooks& hooks);

}  // namespace pa
