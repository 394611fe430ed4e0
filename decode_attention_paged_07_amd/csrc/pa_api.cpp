// C-ABI of libpa_decode.so: validation, planning, workspace carving, launch.
// Every check happens on the host before any HIP call (see pa_decode.h).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "pa_decode.h"
#include "pa_kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return PA_OK;
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int elem_bytes_of(int q_dtype, int kv_cache_dtype) {
  if (kv_cache_dtype == PA_KV_FP8_E4M3) return 1;
  return q_dtype == PA_DTYPE_F32 ? 4 : 2;
}

int check_dtypes(int q_dtype, int kv_cache_dtype) {
  if (q_dtype != PA_DTYPE_F32 && q_dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_DTYPE, "q_dtype %d is not PA_DTYPE_F32 or PA_DTYPE_BF16", q_dtype);
  if (kv_cache_dtype != PA_KV_AUTO && kv_cache_dtype != PA_KV_FP8_E4M3)
    return fail(PA_ERR_DTYPE, "kv_cache_dtype %d is not PA_KV_AUTO or PA_KV_FP8_E4M3", kv_cache_dtype);
  if (kv_cache_dtype == PA_KV_FP8_E4M3 && q_dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_DTYPE, "the fp8 e4m3 cache requires bf16 queries");
  return PA_OK;
}

// Split size chosen by the library: the largest split (a power-of-two
// multiple of the 256-token partition, up to 8) that still leaves at least
// kTargetItems (sequence, kv head, split) work items, so that every one of the
// 256 compute units gets several workgroups.
constexpr int64_t kTargetItems = 2048;

int choose_split_tokens(int num_seqs, int num_kv_heads, int max_seq_len) {
  const int64_t parts = std::max<int64_t>(1, (max_seq_len + PA_PARTITION_SIZE - 1) / PA_PARTITION_SIZE);
  for (int k = 8; k > 1; k >>= 1) {
    const int64_t splits = (parts + k - 1) / k;
    if ((int64_t)num_seqs * num_kv_heads * splits >= kTargetItems) return k * PA_PARTITION_SIZE;
  }
  return PA_PARTITION_SIZE;
}

struct Plan {
  int split_tokens;
  int num_splits;
  size_t tmp_off, ml_off, es_off, bytes;
};

Plan make_plan(int num_seqs, int num_heads, int num_kv_heads, int head_size, int max_seq_len,
               int split_tokens) {
  Plan p{};
  p.split_tokens = split_tokens > 0 ? split_tokens : choose_split_tokens(num_seqs, num_kv_heads, max_seq_len);
  p.num_splits = std::max(1, (max_seq_len + p.split_tokens - 1) / p.split_tokens);
  if (p.num_splits > 1) {
    const size_t rows = (size_t)num_seqs * num_heads * p.num_splits;
    p.tmp_off = 0;
    p.ml_off = round_up(rows * head_size * sizeof(float), 256);
    p.es_off = p.ml_off + round_up(rows * sizeof(float), 256);
    p.bytes = p.es_off + round_up(rows * sizeof(float), 256);
  }
  return p;
}

int check_plan_args(int num_seqs, int num_heads, int num_kv_heads, int head_size, int max_seq_len,
                    int split_tokens) {
  if (num_seqs < 0) return fail(PA_ERR_SHAPE, "num_seqs %d < 0", num_seqs);
  if (num_heads <= 0 || num_kv_heads <= 0)
    return fail(PA_ERR_SHAPE, "num_heads %d and num_kv_heads %d must be positive", num_heads, num_kv_heads);
  if (num_heads % num_kv_heads)
    return fail(PA_ERR_SHAPE, "num_heads %d is not a multiple of num_kv_heads %d", num_heads, num_kv_heads);
  if (num_heads / num_kv_heads > PA_MAX_GROUP)
    return fail(PA_ERR_SHAPE, "query heads per kv head %d exceeds %d", num_heads / num_kv_heads, PA_MAX_GROUP);
  if (head_size != 64 && head_size != 128) return fail(PA_ERR_SHAPE, "head_size %d is not 64 or 128", head_size);
  if (max_seq_len < 0) return fail(PA_ERR_SHAPE, "max_seq_len %d < 0", max_seq_len);
  if (split_tokens < 0 || split_tokens % PA_PARTITION_SIZE)
    return fail(PA_ERR_SHAPE, "split_tokens %d is not 0 or a positive multiple of %d", split_tokens,
                PA_PARTITION_SIZE);
  // Index arithmetic inside the kernels: rows of the workspace and of q/out fit in int64,
  // per-dimension sizes fit in int32 (checked by the types above).
  return PA_OK;
}

// ---- event timing -----------------------------------------------------------------

struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;                 // free events
  std::vector<std::pair<hipEvent_t, hipEvent_t>> part, red;
  hipEvent_t pending = nullptr;
};
Timing g_timing;

hipEvent_t take_event() {
  if (!g_timing.pool.empty()) {
    hipEvent_t e = g_timing.pool.back();
    g_timing.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void record_begin(hipStream_t s) {
  hipEvent_t e = take_event();
  if (e) (void)hipEventRecord(e, s);
  g_timing.pending = e;
}
void record_end_into(std::vector<std::pair<hipEvent_t, hipEvent_t>>& v, hipStream_t s) {
  hipEvent_t e = take_event();
  if (e) (void)hipEventRecord(e, s);
  if (g_timing.pending && e) v.emplace_back(g_timing.pending, e);
  g_timing.pending = nullptr;
}
void hook_part_end(hipStream_t s) { record_end_into(g_timing.part, s); }
void hook_red_end(hipStream_t s) { record_end_into(g_timing.red, s); }

int decode_impl(void* out, const void* query, const void* key_cache, const void* value_cache,
                int num_seqs, int num_heads, int num_kv_heads, int head_size, int num_blocks,
                float scale, const int32_t* block_tables, int max_blocks_per_seq,
                const int32_t* seq_lens, int block_size, int max_seq_len,
                const float* alibi_slopes, int q_dtype, int kv_cache_dtype, const float* k_scale,
                const float* v_scale, void* workspace, size_t workspace_bytes, void* stream,
                int split_tokens) {
  int rc = check_plan_args(num_seqs, num_heads, num_kv_heads, head_size, max_seq_len, split_tokens);
  if (rc) return rc;
  if ((rc = check_dtypes(q_dtype, kv_cache_dtype))) return rc;
  if (block_size != PA_BLOCK_SIZE) return fail(PA_ERR_SHAPE, "block_size %d is not %d", block_size, PA_BLOCK_SIZE);
  if (num_seqs == 0) return ok();
  if (!out || !query || !key_cache || !value_cache || !block_tables || !seq_lens)
    return fail(PA_ERR_NULL, "out, query, key_cache, value_cache, block_tables and seq_lens must be non-NULL");
  if (num_blocks <= 0) return fail(PA_ERR_SHAPE, "num_blocks %d must be positive", num_blocks);
  if (max_blocks_per_seq <= 0) return fail(PA_ERR_SHAPE, "max_blocks_per_seq %d must be positive", max_blocks_per_seq);
  if ((int64_t)max_seq_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PA_ERR_SHAPE, "max_seq_len %d exceeds max_blocks_per_seq*block_size = %lld", max_seq_len,
                (long long)max_blocks_per_seq * block_size);
  if (!std::isfinite(scale)) return fail(PA_ERR_SHAPE, "scale is not finite");
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(key_cache, 16) || !aligned(value_cache, 16))
    return fail(PA_ERR_ALIGN, "out, query, key_cache and value_cache must be 16-byte aligned");
  if (!aligned(block_tables, 4) || !aligned(seq_lens, 4) || (alibi_slopes && !aligned(alibi_slopes, 4)) ||
      (k_scale && !aligned(k_scale, 4)) || (v_scale && !aligned(v_scale, 4)))
    return fail(PA_ERR_ALIGN, "block_tables, seq_lens, alibi_slopes and scales must be 4-byte aligned");
  const int ebq = q_dtype == PA_DTYPE_F32 ? 4 : 2;
  const size_t qo_bytes = (size_t)num_seqs * num_heads * head_size * ebq;
  const uintptr_t o0 = reinterpret_cast<uintptr_t>(out), q0 = reinterpret_cast<uintptr_t>(query);
  if (o0 < q0 + qo_bytes && q0 < o0 + qo_bytes) return fail(PA_ERR_SHAPE, "out overlaps query");

  const Plan plan = make_plan(num_seqs, num_heads, num_kv_heads, head_size, max_seq_len, split_tokens);
  if (plan.bytes) {
    if (!workspace) return fail(PA_ERR_WORKSPACE, "this plan needs a workspace of %zu bytes", plan.bytes);
    if (workspace_bytes < plan.bytes)
      return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu this plan needs",
                  workspace_bytes, plan.bytes);
    if (!aligned(workspace, 16)) return fail(PA_ERR_ALIGN, "workspace must be 16-byte aligned");
  }

  const int eb = elem_bytes_of(q_dtype, kv_cache_dtype);
  const int64_t tile = (int64_t)head_size * block_size * eb;   // one (block, kv head) tile
  pa::DecodeArgs a{};
  a.out = out;
  a.query = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.alibi_slopes = alibi_slopes;
  const bool fp8 = kv_cache_dtype == PA_KV_FP8_E4M3;
  a.k_scale = fp8 ? k_scale : nullptr;
  a.v_scale = fp8 ? v_scale : nullptr;
  char* ws = static_cast<char*>(workspace);
  a.tmp_out = plan.bytes ? reinterpret_cast<float*>(ws + plan.tmp_off) : nullptr;
  a.max_logits = plan.bytes ? reinterpret_cast<float*>(ws + plan.ml_off) : nullptr;
  a.exp_sums = plan.bytes ? reinterpret_cast<float*>(ws + plan.es_off) : nullptr;
  a.k_block_stride_bytes = tile * num_kv_heads;
  a.k_head_stride_bytes = tile;
  a.v_block_stride_bytes = tile * num_kv_heads;
  a.v_head_stride_bytes = tile;
  a.scale = scale;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_heads / num_kv_heads;
  a.head_size = head_size;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_seq_len = max_seq_len;
  a.split_tokens = plan.split_tokens;
  a.num_splits = plan.num_splits;
  const int kind = fp8 ? pa::KIND_FP8 : (q_dtype == PA_DTYPE_F32 ? pa::KIND_F32 : pa::KIND_BF16);

  pa::LaunchHooks hooks;
  std::unique_lock<std::mutex> lock(g_timing.mu, std::defer_lock);
  bool timed = false;
  {
    std::lock_guard<std::mutex> g(g_timing.mu);
    timed = g_timing.on;
  }
  if (timed) {
    lock.lock();
    hooks.before_partition = record_begin;
    hooks.after_partition = hook_part_end;
    hooks.before_reduce = record_begin;
    hooks.after_reduce = hook_red_end;
  }
  hipError_t err = pa::launch_decode(a, kind, static_cast<hipStream_t>(stream), hooks);
  if (err != hipSuccess) return fail(PA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return ok();
}

}  // namespace

extern "C" {

int pa_kv_layout(int num_kv_heads, int head_size, int block_size, int q_dtype, int kv_cache_dtype,
                 pa_layout_desc* desc) {
  if (!desc) return fail(PA_ERR_NULL, "desc is NULL");
  int rc = check_dtypes(q_dtype, kv_cache_dtype);
  if (rc) return rc;
  if (num_kv_heads <= 0) return fail(PA_ERR_SHAPE, "num_kv_heads %d must be positive", num_kv_heads);
  if (head_size != 64 && head_size != 128) return fail(PA_ERR_SHAPE, "head_size %d is not 64 or 128", head_size);
  if (block_size != PA_BLOCK_SIZE) return fail(PA_ERR_SHAPE, "block_size %d is not %d", block_size, PA_BLOCK_SIZE);
  const int eb = elem_bytes_of(q_dtype, kv_cache_dtype);
  const int64_t tile = (int64_t)head_size * block_size;
  desc->x = 16 / eb;
  desc->elem_bytes = eb;
  desc->k_block_stride = tile * num_kv_heads;
  desc->k_head_stride = tile;
  desc->v_block_stride = tile * num_kv_heads;
  desc->v_head_stride = tile;
  return ok();
}

int pa_decode_plan(int num_seqs, int num_heads, int num_kv_heads, int head_size, int max_seq_len,
                   int requested_split_tokens, int* split_tokens, int* num_splits,
                   size_t* workspace_bytes) {
  int rc = check_plan_args(num_seqs, num_heads, num_kv_heads, head_size, max_seq_len, requested_split_tokens);
  if (rc) return rc;
  const Plan p = make_plan(num_seqs, num_heads, num_kv_heads, head_size, max_seq_len, requested_split_tokens);
  if (split_tokens) *split_tokens = p.split_tokens;
  if (num_splits) *num_splits = p.num_splits;
  if (workspace_bytes) *workspace_bytes = p.bytes;
  return ok();
}

int pa_workspace_bytes(int num_seqs, int num_heads, int head_size, int max_seq_len, size_t* bytes) {
  if (!bytes) return fail(PA_ERR_NULL, "bytes is NULL");
  // The 256-token plan needs the most workspace; its size does not depend on num_kv_heads.
  int rc = check_plan_args(num_seqs, num_heads, num_heads, head_size, max_seq_len, PA_PARTITION_SIZE);
  if (rc) return rc;
  *bytes = make_plan(num_seqs, num_heads, num_heads, head_size, max_seq_len, PA_PARTITION_SIZE).bytes;
  return ok();
}

int pa_paged_attention_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                              int num_seqs, int num_heads, int num_kv_heads, int head_size, int num_blocks,
                              float scale, const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* seq_lens, int block_size, int max_seq_len,
                              const float* alibi_slopes, int q_dtype, int kv_cache_dtype,
                              const float* k_scale, const float* v_scale, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return decode_impl(out, query, key_cache, value_cache, num_seqs, num_heads, num_kv_heads, head_size,
                     num_blocks, scale, block_tables, max_blocks_per_seq, seq_lens, block_size, max_seq_len,
                     alibi_slopes, q_dtype, kv_cache_dtype, k_scale, v_scale, workspace, workspace_bytes,
                     stream, 0);
}

int pa_paged_attention_decode_split(void* out, const void* query, const void* key_cache,
                                    const void* value_cache, int num_seqs, int num_heads, int num_kv_heads,
                                    int head_size, int num_blocks, float scale, const int32_t* block_tables,
                                    int max_blocks_per_seq, const int32_t* seq_lens, int block_size,
                                    int max_seq_len, const float* alibi_slopes, int q_dtype,
                                    int kv_cache_dtype, const float* k_scale, const float* v_scale,
                                    void* workspace, size_t workspace_bytes, void* stream, int split_tokens) {
  return decode_impl(out, query, key_cache, value_cache, num_seqs, num_heads, num_kv_heads, head_size,
                     num_blocks, scale, block_tables, max_blocks_per_seq, seq_lens, block_size, max_seq_len,
                     alibi_slopes, q_dtype, kv_cache_dtype, k_scale, v_scale, workspace, workspace_bytes,
                     stream, split_tokens);
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

int pa_version(void) { return 100; }

int pa_timing_enable(int on) {
  std::lock_guard<std::mutex> g(g_timing.mu);
  g_timing.on = on != 0;
  return ok();
}

int pa_timing_read(double* partition_ms, int* partition_launches, double* reduce_ms, int* reduce_launches) {
  std::lock_guard<std::mutex> g(g_timing.mu);
  double tp = 0, tr = 0;
  int np = 0, nr = 0;
  hipError_t first_err = hipSuccess;
  auto drain = [&](std::vector<std::pair<hipEvent_t, hipEvent_t>>& v, double& t, int& n) {
    for (auto& pr : v) {
      float ms = 0.f;
      hipError_t e = hipEventSynchronize(pr.second);
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, pr.first, pr.second);
      if (e != hipSuccess && first_err == hipSuccess) first_err = e;
      t += ms;
      ++n;
      g_timing.pool.push_back(pr.first);
      g_timing.pool.push_back(pr.second);
    }
    v.clear();
  };
  drain(g_timing.part, tp, np);
  drain(g_timing.red, tr, nr);
  if (partition_ms) *partition_ms = tp;
  if (partition_launches) *partition_launches = np;
  if (reduce_ms) *reduce_ms = tr;
  if (reduce_launches) *reduce_launches = nr;
  if (first_err != hipSuccess) return fail(PA_ERR_HIP, "event timing failed: %s", hipGetErrorString(first_err));
  return ok();
}

}  // extern "C"
