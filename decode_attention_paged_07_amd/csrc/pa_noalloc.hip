// Decode that allocates nothing: pa_paged_attention_decode_noalloc runs the
// decode call's default (stream-K) plan with its workspace in a static device
// array of this library instead of a caller buffer, for callers that cannot
// allocate device memory.
//
// The array's name is a host-side stand-in in host code, not a device
// address. Its address on a device comes from hipGetSymbolAddress, called
// once per device with that device current, and only that address is handed
// to the kernels. Every device that runs the library holds its own copy of
// the array until the process ends.

#include <hip/hip_runtime.h>

#include <mutex>

#include "pa_decode.h"

int pa_internal_fail(int code, const char* fmt, ...);
int pa_internal_decode(void* out, const void* query, const void* key_cache, const void* value_cache, int num_seqs,
                       int num_heads, int num_kv_heads, int head_size, int num_blocks, float scale,
                       const int32_t* block_tables, int max_blocks_per_seq, const int32_t* seq_lens, int block_size,
                       int max_seq_len, const float* alibi_slopes, int q_dtype, int kv_cache_dtype,
                       const float* k_scale, const float* v_scale, void* workspace, size_t workspace_bytes,
                       void* stream);
int pa_internal_decode_bytes(void* out, const void* query, const void* key_cache, const void* value_cache,
                             int num_seqs, int num_heads, int num_kv_heads, int head_size, int num_blocks, float scale,
                             const int32_t* block_tables, int max_blocks_per_seq, const int32_t* seq_lens,
                             int block_size, int max_seq_len, const float* alibi_slopes, int q_dtype,
                             int kv_cache_dtype, const float* k_scale, const float* v_scale, size_t* bytes);

// The workspace of every no-alloc call on a device. Nothing in it has to
// start at any value: the stream-K kernel writes every slot and pair record
// the merge reads in the same call.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch`, per device (null until looked up)

// Device address of the current device's copy of `scratch`.
int scratch_address(void** ptr) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return pa_internal_fail(PA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices) return pa_internal_fail(PA_ERR_HIP, "device %d is beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !p)
      return pa_internal_fail(PA_ERR_HIP, "hipGetSymbolAddress of the scratch array failed on device %d: %s", dev,
                              hipGetErrorString(err));
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return PA_OK;
}

}  // namespace

extern "C" int pa_paged_attention_decode_noalloc(void* out, const void* query, const void* key_cache,
                                                 const void* value_cache, int num_seqs, int num_heads,
                                                 int num_kv_heads, int head_size, int num_blocks, float scale,
                                                 const int32_t* block_tables, int max_blocks_per_seq,
                                                 const int32_t* seq_lens, int block_size, int max_seq_len,
                                                 const float* alibi_slopes, int q_dtype, int kv_cache_dtype,
                                                 const float* k_scale, const float* v_scale, void* stream) {
  size_t need = 0;
  int rc = pa_internal_decode_bytes(out, query, key_cache, value_cache, num_seqs, num_heads, num_kv_heads, head_size,
                                    num_blocks, scale, block_tables, max_blocks_per_seq, seq_lens, block_size,
                                    max_seq_len, alibi_slopes, q_dtype, kv_cache_dtype, k_scale, v_scale, &need);
  if (rc) return rc;
  if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES)
    return pa_internal_fail(PA_ERR_WORKSPACE,
                            "this call needs %zu bytes of workspace, more than the %zu of the no-alloc scratch; "
                            "call pa_paged_attention_decode with a workspace instead",
                            need, (size_t)PA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0 && (rc = scratch_address(&ws))) return rc;
  return pa_internal_decode(out, query, key_cache, value_cache, num_seqs, num_heads, num_kv_heads, head_size,
                            num_blocks, scale, block_tables, max_blocks_per_seq, seq_lens, block_size, max_seq_len,
                            alibi_slopes, q_dtype, kv_cache_dtype, k_scale, v_scale, ws,
                            need > 0 ? (size_t)PA_NOALLOC_SCRATCH_BYTES : 0, stream);
}
