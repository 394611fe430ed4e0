// C-ABI of libpa_decode.so: validation, planning, workspace carving, launch.
// Every check happens on the host before any HIP call (see pa_decode.h).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
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

bool is_fp8_cache(int kv_cache_dtype) {
  return kv_cache_dtype == PA_KV_FP8_E4M3 || kv_cache_dtype == PA_KV_FP8_E4M3_COMPUTE;
}

int elem_bytes_of(int q_dtype, int kv_cache_dtype) {
  if (is_fp8_cache(kv_cache_dtype)) return 1;
  return q_dtype == PA_DTYPE_F32 ? 4 : 2;
}

// Head sizes 32, 64 and 128 (the pages' kernel instantiations list these
// among others).
int check_head_size(int head_size) {
  if (head_size != 32 && head_size != 64 && head_size != 128)
    return fail(PA_ERR_SHAPE, "head_size %d is not 32, 64 or 128", head_size);
  return PA_OK;
}

// Cache blocks of 16 or 32 tokens.
int check_block_size(int block_size) {
  if (block_size != 16 && block_size != 32) return fail(PA_ERR_SHAPE, "block_size %d is not 16 or 32", block_size);
  return PA_OK;
}

int check_dtypes(int q_dtype, int kv_cache_dtype) {
  if (q_dtype != PA_DTYPE_F32 && q_dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_DTYPE, "q_dtype %d is not PA_DTYPE_F32 or PA_DTYPE_BF16", q_dtype);
  if (kv_cache_dtype != PA_KV_AUTO && !is_fp8_cache(kv_cache_dtype))
    return fail(PA_ERR_DTYPE, "kv_cache_dtype %d is not PA_KV_AUTO, PA_KV_FP8_E4M3 or PA_KV_FP8_E4M3_COMPUTE",
                kv_cache_dtype);
  if (is_fp8_cache(kv_cache_dtype) && q_dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_DTYPE, "the fp8 e4m3 cache requires bf16 queries");
  return PA_OK;
}

// Two schedulers (see pa_kernels.hip): an explicit split size selects the
// split grid, whose multi-split sequences keep per-split partials in the
// pages' partition format; split_tokens == 0 selects stream-K, where every
// wave gets an equal share of all (block, kv head) tiles. Workspace carving:
//   split:    tmp_out [S][H][P][D] | max_logits [S][H][P] | exp_sums [S][H][P]
//   stream-K: seg_out [slots][G][D] | seg_max [slots][G] | seg_sum [slots][G] | seg_meta [S*Hkv][2]
// with slots = S*Hkv + sk_waves (the persistent grid's waves); each array
// 256-byte aligned.
struct Plan {
  bool streamk;
  int split_tokens;
  int num_splits;
  size_t off[4];
  size_t bytes;
};

Plan make_plan(int num_seqs, int num_heads, int num_kv_heads, int head_size, int max_seq_len,
               int split_tokens, int sk_waves) {
  Plan p{};
  if (split_tokens > 0) {
    p.split_tokens = split_tokens;
    p.num_splits = std::max(1, (max_seq_len + split_tokens - 1) / split_tokens);
    if (p.num_splits > 1) {
      const size_t rows = (size_t)num_seqs * num_heads * p.num_splits;
      p.off[0] = 0;
      p.off[1] = round_up(rows * head_size * sizeof(float), 256);
      p.off[2] = p.off[1] + round_up(rows * sizeof(float), 256);
      p.bytes = p.off[2] + round_up(rows * sizeof(float), 256);
    }
    return p;
  }
  p.streamk = true;
  const size_t group = (size_t)(num_heads / num_kv_heads);
  const size_t pairs = (size_t)num_seqs * num_kv_heads;
  const size_t slots = pairs + (size_t)sk_waves;
  p.off[0] = 0;
  p.off[1] = round_up(slots * group * head_size * sizeof(float), 256);
  p.off[2] = p.off[1] + round_up(slots * group * sizeof(float), 256);
  p.off[3] = p.off[2] + round_up(slots * group * sizeof(float), 256);
  p.bytes = p.off[3] + round_up(pairs * 2 * sizeof(int32_t), 256);
  return p;
}

// Compute units of the current device (queried once per device).
int device_cus() {
  static std::atomic<int> cached[64];        // 0 = not yet queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Stream-K waves of the persistent grid for a kernel kind and block size.
// Waves per compute unit, measured per cache type and block size: each wave
// keeps one block's loads in flight, and throughput peaks at a total of about
// 8-12 MiB in flight (bf16, 16-token blocks: one wave per SIMD; fp8 needs
// more waves to overlap its conversions; 32-token blocks carry twice the bytes
// per wave). A fraction leaves some compute units without a workgroup, which
// measured faster than spreading them.
int streamk_waves(int kind, int block_size) {
  const bool b32 = block_size == 32;
  const double per_cu = kind == pa::KIND_FP8MX ? (b32 ? PA_SK_WAVES_PER_CU_BS32_FP8MX : PA_SK_WAVES_PER_CU_FP8MX)
                        : kind == pa::KIND_FP8 ? (b32 ? PA_SK_WAVES_PER_CU_BS32_FP8 : PA_SK_WAVES_PER_CU_FP8)
                        : kind == pa::KIND_F32 ? (b32 ? PA_SK_WAVES_PER_CU_BS32_F32 : PA_SK_WAVES_PER_CU_F32)
                                               : (b32 ? PA_SK_WAVES_PER_CU_BS32_BF16 : PA_SK_WAVES_PER_CU_BF16);
  const int waves = std::min(PA_SK_MAX_WAVES, (int)(device_cus() * per_cu));
  return std::max(1, waves / PA_WAVES) * PA_WAVES;
}

// The most stream-K waves any kind or block size launches on this device: the
// slot count pa_decode_plan and pa_workspace_bytes size the workspace for.
int streamk_waves_bound() {
  int w = 0;
  for (int kind : {pa::KIND_F32, pa::KIND_BF16, pa::KIND_FP8, pa::KIND_FP8MX})
    for (int bs : {16, 32}) w = std::max(w, streamk_waves(kind, bs));
  return w;
}

int check_plan_args(int num_seqs, int num_heads, int num_kv_heads, int head_size, int max_seq_len,
                    int split_tokens) {
  if (num_seqs < 0) return fail(PA_ERR_SHAPE, "num_seqs %d < 0", num_seqs);
  if (num_seqs > PA_MAX_SEQS) return fail(PA_ERR_SHAPE, "num_seqs %d exceeds %d", num_seqs, PA_MAX_SEQS);
  if (num_heads <= 0 || num_kv_heads <= 0)
    return fail(PA_ERR_SHAPE, "num_heads %d and num_kv_heads %d must be positive", num_heads, num_kv_heads);
  if (num_heads % num_kv_heads)
    return fail(PA_ERR_SHAPE, "num_heads %d is not a multiple of num_kv_heads %d", num_heads, num_kv_heads);
  if (num_heads / num_kv_heads > PA_MAX_GROUP)
    return fail(PA_ERR_SHAPE, "query heads per kv head %d exceeds %d", num_heads / num_kv_heads, PA_MAX_GROUP);
  int rc = check_head_size(head_size);
  if (rc) return rc;
  if (max_seq_len < 0) return fail(PA_ERR_SHAPE, "max_seq_len %d < 0", max_seq_len);
  if (split_tokens < 0 || split_tokens % PA_PARTITION_SIZE)
    return fail(PA_ERR_SHAPE, "split_tokens %d is not 0 or a positive multiple of %d", split_tokens,
                PA_PARTITION_SIZE);
  if (split_tokens > 0 && ((int64_t)max_seq_len + split_tokens - 1) / split_tokens > PA_MAX_SEQS)
    return fail(PA_ERR_SHAPE, "max_seq_len %d needs more than %d splits of %d tokens", max_seq_len, PA_MAX_SEQS,
                split_tokens);
  // Index arithmetic inside the kernels: rows of the workspace and of q/out fit in int64,
  // per-dimension sizes fit in int32 (checked by the types above).
  return PA_OK;
}

// ---- event timing -----------------------------------------------------------------

struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;                 // free events
  std::vector<std::pair<hipEvent_t, hipEvent_t>> part, red, app;
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

// Drains recorded (begin, end) event pairs into a total and a count; the
// caller holds g_timing.mu.
hipError_t drain_events(std::vector<std::pair<hipEvent_t, hipEvent_t>>& v, double& t, int& n) {
  hipError_t first_err = hipSuccess;
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
  return first_err;
}

// Host-side checks shared by the decode entry points; everything before the
// launch plan. Returns PA_OK, or an error code (nothing launched).
int check_decode_args(void* out, const void* query, const void* key_cache, const void* value_cache,
                      int num_seqs, int num_heads, int num_kv_heads, int head_size, int num_blocks,
                      float scale, const int32_t* block_tables, int max_blocks_per_seq,
                      const int32_t* seq_lens, int block_size, int max_seq_len,
                      const float* alibi_slopes, int q_dtype, int kv_cache_dtype, const float* k_scale,
                      const float* v_scale, int split_tokens) {
  int rc = check_plan_args(num_seqs, num_heads, num_kv_heads, head_size, max_seq_len, split_tokens);
  if (rc) return rc;
  if ((rc = check_dtypes(q_dtype, kv_cache_dtype))) return rc;
  if ((rc = check_block_size(block_size))) return rc;
  if (num_seqs == 0) return PA_OK;
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
  return PA_OK;
}

// The launch-independent fields of DecodeArgs; returns the kernel kind.
int fill_decode_args(pa::DecodeArgs& a, void* out, const void* query, const void* key_cache,
                     const void* value_cache, int num_seqs, int num_heads, int num_kv_heads, int head_size,
                     int num_blocks, float scale, const int32_t* block_tables, int max_blocks_per_seq,
                     const int32_t* seq_lens, int block_size, int max_seq_len, const float* alibi_slopes,
                     int q_dtype, int kv_cache_dtype, const float* k_scale, const float* v_scale) {
  const int eb = elem_bytes_of(q_dtype, kv_cache_dtype);
  const int64_t tile = (int64_t)head_size * block_size * eb;   // one (block, kv head) tile
  a = pa::DecodeArgs{};
  a.out = out;
  a.query = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.alibi_slopes = alibi_slopes;
  const bool fp8 = is_fp8_cache(kv_cache_dtype);
  a.k_scale = fp8 ? k_scale : nullptr;
  a.v_scale = fp8 ? v_scale : nullptr;
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
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_seq_len = max_seq_len;
  if (kv_cache_dtype == PA_KV_FP8_E4M3_COMPUTE) return pa::KIND_FP8MX;
  return fp8 ? pa::KIND_FP8 : (q_dtype == PA_DTYPE_F32 ? pa::KIND_F32 : pa::KIND_BF16);
}

int check_workspace(const void* workspace, size_t workspace_bytes, size_t need) {
  if (!need) return PA_OK;
  if (!workspace) return fail(PA_ERR_WORKSPACE, "this plan needs a workspace of %zu bytes", need);
  if (workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu this plan needs", workspace_bytes,
                need);
  if (!aligned(workspace, 16)) return fail(PA_ERR_ALIGN, "workspace must be 16-byte aligned");
  return PA_OK;
}

// ---- opt-in check of the device-resident metadata -----------------------------

// With PA_VALIDATE_DEVICE=1 in the environment, the decode calls copy
// seq_lens and the table entries each sequence uses (the first
// ceil(seq_len / block_size) of its row) to the host after the stream's
// earlier work, and reject values outside [0, max_seq_len] and
// [0, num_blocks) with PA_ERR_SHAPE before anything is launched. Without it
// the kernels clamp such values (a length into [0, max_seq_len], a block id
// into the pool), which keeps every access in bounds but gives meaningless
// output. The check synchronizes the stream and is slow: a debugging aid. It
// copies through a fixed buffer on the host stack (no allocation), and it is
// skipped while the stream is being captured into a graph.
bool validate_device_requested() {
  const char* v = std::getenv("PA_VALIDATE_DEVICE");
  return v && v[0] == '1' && v[1] == '\0';
}

int validate_device_metadata(const int32_t* seq_lens, const int32_t* block_tables, int num_seqs,
                             int max_blocks_per_seq, int block_size, int max_seq_len, int num_blocks,
                             hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess)
    return fail(PA_ERR_HIP, "PA_VALIDATE_DEVICE: hipStreamIsCapturing failed");
  if (cs != hipStreamCaptureStatusNone) return PA_OK;
  constexpr int kBuf = 2048;
  int32_t lens[kBuf], ent[kBuf];
  auto copy = [&](int32_t* dst, const int32_t* src, int64_t n) -> bool {
    if (hipMemcpyAsync(dst, src, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess) return false;
    return hipStreamSynchronize(stream) == hipSuccess;
  };
  for (int s0 = 0; s0 < num_seqs; s0 += kBuf) {
    const int n = std::min(kBuf, num_seqs - s0);
    if (!copy(lens, seq_lens + s0, n)) return fail(PA_ERR_HIP, "PA_VALIDATE_DEVICE: copy of seq_lens failed");
    for (int i = 0; i < n; ++i) {
      const int s = s0 + i, L = lens[i];
      if (L < 0 || L > max_seq_len)
        return fail(PA_ERR_SHAPE, "PA_VALIDATE_DEVICE: seq_lens[%d] = %d is outside [0, max_seq_len = %d]", s, L,
                    max_seq_len);
      const int used = (L + block_size - 1) / block_size;
      for (int b0 = 0; b0 < used; b0 += kBuf) {
        const int m = std::min(kBuf, used - b0);
        if (!copy(ent, block_tables + (int64_t)s * max_blocks_per_seq + b0, m))
          return fail(PA_ERR_HIP, "PA_VALIDATE_DEVICE: copy of block_tables failed");
        for (int j = 0; j < m; ++j)
          if (ent[j] < 0 || ent[j] >= num_blocks)
            return fail(PA_ERR_SHAPE, "PA_VALIDATE_DEVICE: block_tables[%d][%d] = %d is outside [0, num_blocks = %d)",
                        s, b0 + j, ent[j], num_blocks);
      }
    }
  }
  return PA_OK;
}

int maybe_validate_device(const int32_t* seq_lens, const int32_t* block_tables, int num_seqs,
                          int max_blocks_per_seq, int block_size, int max_seq_len, int num_blocks, void* stream) {
  if (!validate_device_requested()) return PA_OK;
  return validate_device_metadata(seq_lens, block_tables, num_seqs, max_blocks_per_seq, block_size, max_seq_len,
                                  num_blocks, static_cast<hipStream_t>(stream));
}

int decode_impl(void* out, const void* query, const void* key_cache, const void* value_cache,
                int num_seqs, int num_heads, int num_kv_heads, int head_size, int num_blocks,
                float scale, const int32_t* block_tables, int max_blocks_per_seq,
                const int32_t* seq_lens, int block_size, int max_seq_len,
                const float* alibi_slopes, int q_dtype, int kv_cache_dtype, const float* k_scale,
                const float* v_scale, void* workspace, size_t workspace_bytes, void* stream,
                int split_tokens) {
  int rc = check_decode_args(out, query, key_cache, value_cache, num_seqs, num_heads, num_kv_heads, head_size,
                             num_blocks, scale, block_tables, max_blocks_per_seq, seq_lens, block_size,
                             max_seq_len, alibi_slopes, q_dtype, kv_cache_dtype, k_scale, v_scale, split_tokens);
  if (rc) return rc;
  if (num_seqs == 0) return ok();
  pa::DecodeArgs a;
  const int kind = fill_decode_args(a, out, query, key_cache, value_cache, num_seqs, num_heads, num_kv_heads,
                                    head_size, num_blocks, scale, block_tables, max_blocks_per_seq, seq_lens,
                                    block_size, max_seq_len, alibi_slopes, q_dtype, kv_cache_dtype, k_scale,
                                    v_scale);
  const int sk_waves = split_tokens == 0 ? streamk_waves(kind, block_size) : 0;
  const Plan plan = make_plan(num_seqs, num_heads, num_kv_heads, head_size, max_seq_len, split_tokens, sk_waves);
  if ((rc = check_workspace(workspace, workspace_bytes, plan.bytes))) return rc;
  if ((rc = maybe_validate_device(seq_lens, block_tables, num_seqs, max_blocks_per_seq, block_size, max_seq_len,
                                  num_blocks, stream)))
    return rc;
  char* ws = static_cast<char*>(workspace);
  if (plan.bytes && !plan.streamk) {
    a.tmp_out = reinterpret_cast<float*>(ws + plan.off[0]);
    a.max_logits = reinterpret_cast<float*>(ws + plan.off[1]);
    a.exp_sums = reinterpret_cast<float*>(ws + plan.off[2]);
  }
  if (plan.streamk) {
    a.seg_out = reinterpret_cast<float*>(ws + plan.off[0]);
    a.seg_max = reinterpret_cast<float*>(ws + plan.off[1]);
    a.seg_sum = reinterpret_cast<float*>(ws + plan.off[2]);
    a.seg_meta = reinterpret_cast<int32_t*>(ws + plan.off[3]);
  }
  a.split_tokens = plan.split_tokens;
  a.num_splits = plan.num_splits;
  if (plan.streamk) a.streamk_workgroups = sk_waves / PA_WAVES;
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

// ---- shared-prefix decode -------------------------------------------------------

#ifndef PA_SHARED_SUFFIX_SPLIT
#define PA_SHARED_SUFFIX_SPLIT 512
#endif
#ifndef PA_SHARED_TARGET_WAVES
#define PA_SHARED_TARGET_WAVES 512
#endif
#ifndef PA_SHARED_MIN_SPLIT_TOKENS
#define PA_SHARED_MIN_SPLIT_TOKENS 512
#endif
#ifndef PA_SHARED_MAX_TILES
#define PA_SHARED_MAX_TILES 4
#endif
constexpr int kSharedSuffixSplit = PA_SHARED_SUFFIX_SPLIT;        // tokens per suffix split
constexpr int kSharedTargetWaves = PA_SHARED_TARGET_WAVES;        // prefix waves the split count aims for
constexpr int kSharedMinSplitTokens = PA_SHARED_MIN_SPLIT_TOKENS; // fewest prefix tokens per wave

struct SharedPlan {
  int column_tiles = 1;
  int members_per_chunk = 1;
  int max_chunks = 0;
  int prefix_split_blocks = 1;
  int max_prefix_splits = 0;
  int num_splits = 1;                       // suffix splits
  size_t off[6] = {0, 0, 0, 0, 0, 0};
  size_t bytes = 0;
};

int check_shared_plan_args(int num_seqs, int num_heads, int num_kv_heads, int head_size, int block_size,
                           int max_seq_len, int num_groups, int max_group_size, int max_prefix_blocks) {
  int rc = check_plan_args(num_seqs, num_heads, num_kv_heads, head_size, max_seq_len, 0);
  if (rc) return rc;
  if ((rc = check_block_size(block_size))) return rc;
  if (num_groups < 0) return fail(PA_ERR_SHAPE, "num_groups %d < 0", num_groups);
  if (num_groups > 0 && max_group_size < 1)
    return fail(PA_ERR_SHAPE, "max_group_size %d must be positive with groups", max_group_size);
  if (max_prefix_blocks < 0) return fail(PA_ERR_SHAPE, "max_prefix_blocks %d < 0", max_prefix_blocks);
  if ((int64_t)max_prefix_blocks * block_size > max_seq_len)
    return fail(PA_ERR_SHAPE, "max_prefix_blocks %d exceeds max_seq_len %d / %d", max_prefix_blocks, max_seq_len,
                block_size);
  return PA_OK;
}

// max_tiles: the kernel kind's column-tile limit (pa::max_column_tiles); the
// workspace for 4 bounds that of every smaller limit (fewer tiles, more
// member chunks, fewer prefix splits). Prefix splits count cache blocks.
SharedPlan make_shared_plan(int num_seqs, int num_heads, int num_kv_heads, int head_size, int block_size,
                            int max_seq_len, int num_groups, int max_group_size, int max_prefix_blocks,
                            int max_tiles = 4) {
  SharedPlan p;
  const int min_split_blocks = kSharedMinSplitTokens / block_size;
  const int group = num_heads / num_kv_heads;
  const int64_t cols = (int64_t)std::max(1, max_group_size) * group;
  p.column_tiles = std::min(max_tiles, cols <= 16 ? 1 : (cols <= 32 ? 2 : 4));
  p.members_per_chunk = std::max(1, 16 * p.column_tiles / group);
  p.max_chunks = num_groups > 0 ? (std::max(1, max_group_size) + p.members_per_chunk - 1) / p.members_per_chunk : 0;
  if (num_groups > 0 && max_prefix_blocks > 0) {
    const int64_t base = (int64_t)num_groups * p.max_chunks * num_kv_heads;
    int64_t splits = std::max<int64_t>(1, (kSharedTargetWaves + base - 1) / base);
    splits = std::min<int64_t>(splits, std::max(1, (max_prefix_blocks + min_split_blocks - 1) / min_split_blocks));
    p.prefix_split_blocks = (int)((max_prefix_blocks + splits - 1) / splits);
    p.max_prefix_splits = (max_prefix_blocks + p.prefix_split_blocks - 1) / p.prefix_split_blocks;
  }
  p.num_splits = std::max(1, (max_seq_len + kSharedSuffixSplit - 1) / kSharedSuffixSplit);
  const size_t rows_s = (size_t)num_seqs * num_heads * p.num_splits;
  const size_t rows_p = (size_t)num_seqs * num_heads * p.max_prefix_splits;
  size_t o = 0;
  p.off[0] = o; o += round_up(rows_s * head_size * sizeof(float), 256);
  p.off[1] = o; o += round_up(rows_s * sizeof(float), 256);
  p.off[2] = o; o += round_up(rows_s * sizeof(float), 256);
  p.off[3] = o; o += round_up(rows_p * head_size * sizeof(float), 256);
  p.off[4] = o; o += round_up(rows_p * sizeof(float), 256);
  p.off[5] = o; o += round_up(rows_p * sizeof(float), 256);
  p.bytes = o;
  return p;
}

// ---- latent-cache (MLA) decode --------------------------------------------------

// MLA stream-K workgroups (one wave each) per compute unit with a single
// 16-head group. With more groups the 16-heads-per-wave kernel fills all four
// SIMDs (PA_MLA_WAVES_PER_CU); with one group it is bound by its reads, which
// two waves per compute unit sustain as well as four, with half the shares
// and so half the partial outputs the merge reads.
#ifndef PA_MLA_WAVES_PER_CU_ONE_GROUP
#define PA_MLA_WAVES_PER_CU_ONE_GROUP 2
#endif
// The same for an fp8 latent cache: each wave has one 9 KiB tile in flight
// instead of 18 KiB, so more waves keep as many bytes in flight.
#ifndef PA_MLA_FP8_WAVES_PER_CU_ONE_GROUP
#define PA_MLA_FP8_WAVES_PER_CU_ONE_GROUP 4
#endif
// Head counts from which the 32-heads-per-wave kernel (pa_mla_wide.hip) runs:
// three or four of its waves fill a compute unit's SIMDs (its 88 KiB of LDS,
// 124 KiB with an fp8 cache, admit one workgroup per compute unit); fewer
// heads fit the 16-heads-per-wave kernel's single workgroup per share.
#ifndef PA_MLA_WIDE_MIN_HEADS
#define PA_MLA_WIDE_MIN_HEADS 65
#endif
static_assert(PA_MLA_WIDE_MIN_HEADS > 64, "the 32-heads-per-wave kernel is built for three or four waves");

// Stream-K plan of the MLA kernels.
//  * 16 heads per wave (pa_mla.hip; fewer than PA_MLA_WIDE_MIN_HEADS heads):
//    one wave per 16-head group and share (each needs more than 256 registers
//    per lane, so one per SIMD), up to four groups in a workgroup that shares
//    one pair of 18 KiB LDS tile buffers, more groups in `chunks` workgroups
//    per share.
//  * 32 heads per wave (pa_mla_wide.hip): one workgroup of ceil(H / 32) waves
//    (one per SIMD) per share and compute unit.
// Workspace: seg_out [slots][hpad][512] bf16 | seg_max [slots][hpad] |
// seg_sum [slots][hpad] | seg_meta [S][2], slots = S + shares.
struct MlaPlan {
  bool wide;
  int head_groups, waves_per_wg, chunks, shares, hpad;
  size_t off[4];
  size_t bytes;
};

MlaPlan make_mla_plan(int num_seqs, int num_heads, bool fp8) {
  MlaPlan p{};
  p.wide = num_heads >= PA_MLA_WIDE_MIN_HEADS;
  const int cus = device_cus();
  if (p.wide) {
    p.head_groups = (num_heads + 31) / 32;
    p.waves_per_wg = p.head_groups;
    p.chunks = 1;
    p.shares = cus;
    p.hpad = 32 * p.head_groups;
  } else {
    p.head_groups = (num_heads + 15) / 16;
    p.waves_per_wg = std::min(p.head_groups, 4);
    p.chunks = (p.head_groups + p.waves_per_wg - 1) / p.waves_per_wg;
    // Shares: the waves per compute unit of the knobs in all, a multiple of 8
    // so that the head groups of a share land on one XCD.
    const int one = fp8 ? PA_MLA_FP8_WAVES_PER_CU_ONE_GROUP : PA_MLA_WAVES_PER_CU_ONE_GROUP;
    const int waves = cus * (p.head_groups == 1 ? one : PA_MLA_WAVES_PER_CU);
    const int shares = std::max(8, waves / (p.waves_per_wg * p.chunks) / 8 * 8);
    p.shares = std::min(shares, PA_MLA_MAX_WAVES / (p.waves_per_wg * p.chunks));
    p.hpad = 16 * p.head_groups;
  }
  const size_t hpad = (size_t)p.hpad;
  const size_t slots = (size_t)num_seqs + p.shares;
  p.off[0] = 0;
  p.off[1] = round_up(slots * hpad * PA_MLA_LATENT_DIM * 2, 256);   // bf16 rows
  p.off[2] = p.off[1] + round_up(slots * hpad * sizeof(float), 256);
  p.off[3] = p.off[2] + round_up(slots * hpad * sizeof(float), 256);
  p.bytes = p.off[3] + round_up((size_t)num_seqs * 2 * sizeof(int32_t), 256);
  return p;
}

int check_mla_plan_args(int num_seqs, int num_heads) {
  if (num_seqs < 0) return fail(PA_ERR_SHAPE, "num_seqs %d < 0", num_seqs);
  if (num_seqs > PA_MAX_SEQS) return fail(PA_ERR_SHAPE, "num_seqs %d exceeds %d", num_seqs, PA_MAX_SEQS);
  if (num_heads <= 0 || num_heads > PA_MLA_MAX_HEADS)
    return fail(PA_ERR_SHAPE, "num_heads %d is not in [1, %d]", num_heads, PA_MLA_MAX_HEADS);
  return PA_OK;
}

}  // namespace

// Error helpers for the other host translation units (pa_blocks.cpp).
__attribute__((visibility("hidden"))) int pa_internal_fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}
__attribute__((visibility("hidden"))) int pa_internal_ok() { return ok(); }

// The decode call for the other host translation units (pa_noalloc.hip).
__attribute__((visibility("hidden"))) int pa_internal_decode(
    void* out, const void* query, const void* key_cache, const void* value_cache, int num_seqs, int num_heads,
    int num_kv_heads, int head_size, int num_blocks, float scale, const int32_t* block_tables,
    int max_blocks_per_seq, const int32_t* seq_lens, int block_size, int max_seq_len, const float* alibi_slopes,
    int q_dtype, int kv_cache_dtype, const float* k_scale, const float* v_scale, void* workspace,
    size_t workspace_bytes, void* stream) {
  return decode_impl(out, query, key_cache, value_cache, num_seqs, num_heads, num_kv_heads, head_size, num_blocks,
                     scale, block_tables, max_blocks_per_seq, seq_lens, block_size, max_seq_len, alibi_slopes,
                     q_dtype, kv_cache_dtype, k_scale, v_scale, workspace, workspace_bytes, stream, 0);
}

// Validates the decode arguments as the decode call does and returns, in
// *bytes, the workspace its default (stream-K) plan needs on the current
// device; no launch.
__attribute__((visibility("hidden"))) int pa_internal_decode_bytes(
    void* out, const void* query, const void* key_cache, const void* value_cache, int num_seqs, int num_heads,
    int num_kv_heads, int head_size, int num_blocks, float scale, const int32_t* block_tables,
    int max_blocks_per_seq, const int32_t* seq_lens, int block_size, int max_seq_len, const float* alibi_slopes,
    int q_dtype, int kv_cache_dtype, const float* k_scale, const float* v_scale, size_t* bytes) {
  *bytes = 0;
  int rc = check_decode_args(out, query, key_cache, value_cache, num_seqs, num_heads, num_kv_heads, head_size,
                             num_blocks, scale, block_tables, max_blocks_per_seq, seq_lens, block_size,
                             max_seq_len, alibi_slopes, q_dtype, kv_cache_dtype, k_scale, v_scale, 0);
  if (rc) return rc;
  if (num_seqs == 0) return ok();
  pa::DecodeArgs a;
  const int kind = fill_decode_args(a, out, query, key_cache, value_cache, num_seqs, num_heads, num_kv_heads,
                                    head_size, num_blocks, scale, block_tables, max_blocks_per_seq, seq_lens,
                                    block_size, max_seq_len, alibi_slopes, q_dtype, kv_cache_dtype, k_scale,
                                    v_scale);
  *bytes = make_plan(num_seqs, num_heads, num_kv_heads, head_size, max_seq_len, 0,
                     streamk_waves(kind, block_size))
               .bytes;
  return ok();
}

extern "C" {

int pa_kv_layout(int num_kv_heads, int head_size, int block_size, int q_dtype, int kv_cache_dtype,
                 pa_layout_desc* desc) {
  if (!desc) return fail(PA_ERR_NULL, "desc is NULL");
  int rc = check_dtypes(q_dtype, kv_cache_dtype);
  if (rc) return rc;
  if (num_kv_heads <= 0) return fail(PA_ERR_SHAPE, "num_kv_heads %d must be positive", num_kv_heads);
  if ((rc = check_head_size(head_size))) return rc;
  if ((rc = check_block_size(block_size))) return rc;
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
  const Plan p = make_plan(num_seqs, num_heads, num_kv_heads, head_size, max_seq_len, requested_split_tokens,
                           requested_split_tokens == 0 ? streamk_waves_bound() : 0);
  if (split_tokens) *split_tokens = p.split_tokens;   // 0 for the stream-K plan
  if (num_splits) *num_splits = p.num_splits;         // 0 for the stream-K plan
  if (workspace_bytes) *workspace_bytes = p.bytes;
  return ok();
}

int pa_workspace_bytes(int num_seqs, int num_heads, int head_size, int max_seq_len, size_t* bytes) {
  if (!bytes) return fail(PA_ERR_NULL, "bytes is NULL");
  // The larger of the 256-token split plan and the stream-K plan over every
  // valid num_kv_heads (stream-K grows with the group size G = H / Hkv).
  int rc = check_plan_args(num_seqs, num_heads, num_heads, head_size, max_seq_len, PA_PARTITION_SIZE);
  if (rc) return rc;
  size_t best = make_plan(num_seqs, num_heads, num_heads, head_size, max_seq_len, PA_PARTITION_SIZE, 0).bytes;
  const int waves = streamk_waves_bound();
  for (int g = 1; g <= PA_MAX_GROUP && g <= num_heads; ++g)
    if (num_heads % g == 0)
      best = std::max(best, make_plan(num_seqs, num_heads, num_heads / g, head_size, max_seq_len, 0, waves).bytes);
  *bytes = best;
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

int pa_shared_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads, int head_size, int block_size,
                              int max_seq_len, int num_groups, int max_group_size, int max_prefix_blocks,
                              size_t* bytes) {
  if (!bytes) return fail(PA_ERR_NULL, "bytes is NULL");
  int rc = check_shared_plan_args(num_seqs, num_heads, num_kv_heads, head_size, block_size, max_seq_len,
                                  num_groups, max_group_size, max_prefix_blocks);
  if (rc) return rc;
  *bytes = make_shared_plan(num_seqs, num_heads, num_kv_heads, head_size, block_size, max_seq_len, num_groups,
                            max_group_size, max_prefix_blocks)
               .bytes;
  return ok();
}

int pa_paged_attention_decode_shared(void* out, const void* query, const void* key_cache,
                                     const void* value_cache, int num_seqs, int num_heads, int num_kv_heads,
                                     int head_size, int num_blocks, float scale, const int32_t* block_tables,
                                     int max_blocks_per_seq, const int32_t* seq_lens, int block_size,
                                     int max_seq_len, const float* alibi_slopes, int q_dtype,
                                     int kv_cache_dtype, const float* k_scale, const float* v_scale,
                                     int num_groups, const int32_t* group_start, const int32_t* group_seqs,
                                     int num_members, const int32_t* group_prefix_blocks,
                                     const int32_t* seq_prefix_blocks, int max_group_size,
                                     int max_prefix_blocks, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  int rc = check_decode_args(out, query, key_cache, value_cache, num_seqs, num_heads, num_kv_heads, head_size,
                             num_blocks, scale, block_tables, max_blocks_per_seq, seq_lens, block_size,
                             max_seq_len, alibi_slopes, q_dtype, kv_cache_dtype, k_scale, v_scale, 0);
  if (rc) return rc;
  if ((rc = check_shared_plan_args(num_seqs, num_heads, num_kv_heads, head_size, block_size, max_seq_len,
                                   num_groups, max_group_size, max_prefix_blocks)))
    return rc;
  if (num_seqs == 0) return ok();
  if (!seq_prefix_blocks) return fail(PA_ERR_NULL, "seq_prefix_blocks must be non-NULL");
  if (num_groups > 0 && (!group_start || !group_prefix_blocks || (num_members > 0 && !group_seqs)))
    return fail(PA_ERR_NULL, "group_start, group_seqs and group_prefix_blocks must be non-NULL with groups");
  if (num_members < 0) return fail(PA_ERR_SHAPE, "num_members %d < 0", num_members);
  if (!aligned(seq_prefix_blocks, 4) || (group_start && !aligned(group_start, 4)) ||
      (group_seqs && !aligned(group_seqs, 4)) || (group_prefix_blocks && !aligned(group_prefix_blocks, 4)))
    return fail(PA_ERR_ALIGN, "group arrays must be 4-byte aligned");
  const int max_tiles = std::min(PA_SHARED_MAX_TILES,
                                 pa::max_column_tiles(q_dtype == PA_DTYPE_F32 ? 4 : 2,
                                                      elem_bytes_of(q_dtype, kv_cache_dtype), head_size, block_size));
  const SharedPlan plan = make_shared_plan(num_seqs, num_heads, num_kv_heads, head_size, block_size, max_seq_len,
                                           num_groups, max_group_size, max_prefix_blocks, max_tiles);
  if (plan.max_prefix_splits > 65535) return fail(PA_ERR_SHAPE, "too many prefix splits");
  if ((rc = check_workspace(workspace, workspace_bytes, plan.bytes))) return rc;
  if ((rc = maybe_validate_device(seq_lens, block_tables, num_seqs, max_blocks_per_seq, block_size, max_seq_len,
                                  num_blocks, stream)))
    return rc;

  pa::SharedArgs sa{};
  const int kind = fill_decode_args(sa.d, out, query, key_cache, value_cache, num_seqs, num_heads, num_kv_heads,
                                    head_size, num_blocks, scale, block_tables, max_blocks_per_seq, seq_lens,
                                    block_size, max_seq_len, alibi_slopes, q_dtype, kv_cache_dtype, k_scale,
                                    v_scale);
  char* ws = static_cast<char*>(workspace);
  sa.d.tmp_out = reinterpret_cast<float*>(ws + plan.off[0]);
  sa.d.max_logits = reinterpret_cast<float*>(ws + plan.off[1]);
  sa.d.exp_sums = reinterpret_cast<float*>(ws + plan.off[2]);
  sa.d.split_tokens = kSharedSuffixSplit;
  sa.d.num_splits = plan.num_splits;
  sa.d.first_block = seq_prefix_blocks;
  sa.d.max_first_block = plan.max_prefix_splits * plan.prefix_split_blocks;
  sa.group_start = group_start;
  sa.group_seqs = group_seqs;
  sa.num_members = num_members;
  sa.group_prefix_blocks = group_prefix_blocks;
  sa.num_groups = num_groups;
  sa.max_chunks = plan.max_chunks;
  sa.members_per_chunk = plan.members_per_chunk;
  sa.prefix_split_blocks = plan.prefix_split_blocks;
  sa.max_prefix_splits = plan.max_prefix_splits;
  sa.pre_out = reinterpret_cast<float*>(ws + plan.off[3]);
  sa.pre_max = reinterpret_cast<float*>(ws + plan.off[4]);
  sa.pre_sum = reinterpret_cast<float*>(ws + plan.off[5]);
  hipError_t err = pa::launch_shared(sa, kind, plan.column_tiles, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(PA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return ok();
}

int pa_hbm_read_probe(const void* buf, size_t bytes, int workgroups, unsigned* sink, void* stream) {
  if (!buf || !sink) return fail(PA_ERR_NULL, "buf and sink must be non-NULL");
  if (bytes == 0 || bytes % 16) return fail(PA_ERR_SHAPE, "bytes %zu is not a positive multiple of 16", bytes);
  if (workgroups < 1 || workgroups > (1 << 20))
    return fail(PA_ERR_SHAPE, "workgroups %d is outside [1, 1<<20]", workgroups);
  if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(PA_ERR_ALIGN, "buf must be 16-B and sink 4-B aligned");
  hipError_t err = pa::launch_read_probe(buf, bytes, workgroups, sink, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(PA_ERR_HIP, "probe launch failed: %s", hipGetErrorString(err));
  return ok();
}

int pa_hbm_gather_probe(const void* pool, size_t pool_bytes, int tile_bytes, const int32_t* ids, int num_tiles,
                        int depth, int workgroups, unsigned* sink, void* stream) {
  if (!pool || !ids || !sink) return fail(PA_ERR_NULL, "pool, ids and sink must be non-NULL");
  if (tile_bytes != 1024 && tile_bytes != 2048 && tile_bytes != 4096 && tile_bytes != 8192 && tile_bytes != 18432)
    return fail(PA_ERR_SHAPE, "tile_bytes %d is not 1024, 2048, 4096, 8192 or 18432", tile_bytes);
  if (pool_bytes < (size_t)tile_bytes) return fail(PA_ERR_SHAPE, "pool of %zu bytes holds no tile", pool_bytes);
  if (num_tiles < 1 || num_tiles > (1 << 28))
    return fail(PA_ERR_SHAPE, "num_tiles %d is outside [1, 1<<28]", num_tiles);
  if (depth != 1 && depth != 2) return fail(PA_ERR_SHAPE, "depth %d is not 1 or 2", depth);
  if (workgroups < 1 || workgroups > (1 << 20))
    return fail(PA_ERR_SHAPE, "workgroups %d is outside [1, 1<<20]", workgroups);
  if (!aligned(pool, 16) || !aligned(ids, 4) || !aligned(sink, 4))
    return fail(PA_ERR_ALIGN, "pool must be 16-B aligned, ids and sink 4-B aligned");
  hipError_t err = pa::launch_gather_probe(pool, pool_bytes, tile_bytes, ids, num_tiles, depth, workgroups, sink,
                                           static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(PA_ERR_HIP, "probe launch failed: %s", hipGetErrorString(err));
  return ok();
}

int pa_kv_cache_append(void* key_cache, void* value_cache, const void* key, const void* value, int num_seqs,
                       int tokens_per_seq, int num_kv_heads, int head_size, int num_blocks,
                       const int32_t* block_tables, int max_blocks_per_seq, const int32_t* positions,
                       int block_size, int in_dtype, int kv_cache_dtype, const float* k_scale,
                       const float* v_scale, void* stream) {
  if (in_dtype != PA_DTYPE_F32 && in_dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_DTYPE, "in_dtype %d is not PA_DTYPE_F32 or PA_DTYPE_BF16", in_dtype);
  if (kv_cache_dtype != PA_KV_AUTO && !is_fp8_cache(kv_cache_dtype))
    return fail(PA_ERR_DTYPE, "kv_cache_dtype %d is not PA_KV_AUTO, PA_KV_FP8_E4M3 or PA_KV_FP8_E4M3_COMPUTE",
                kv_cache_dtype);
  if (num_seqs < 0) return fail(PA_ERR_SHAPE, "num_seqs %d < 0", num_seqs);
  if (tokens_per_seq < 1) return fail(PA_ERR_SHAPE, "tokens_per_seq %d must be positive", tokens_per_seq);
  if (num_kv_heads <= 0) return fail(PA_ERR_SHAPE, "num_kv_heads %d must be positive", num_kv_heads);
  int rc = check_head_size(head_size);
  if (rc) return rc;
  if ((rc = check_block_size(block_size))) return rc;
  if (num_blocks <= 0) return fail(PA_ERR_SHAPE, "num_blocks %d must be positive", num_blocks);
  if (max_blocks_per_seq <= 0) return fail(PA_ERR_SHAPE, "max_blocks_per_seq %d must be positive", max_blocks_per_seq);
  if ((int64_t)num_seqs * tokens_per_seq * num_kv_heads >= ((int64_t)1 << 31))
    return fail(PA_ERR_SHAPE, "num_seqs * tokens_per_seq * num_kv_heads must be below 2^31");
  if (num_seqs == 0) return ok();
  if (!key_cache || !value_cache || !key || !value || !block_tables || !positions)
    return fail(PA_ERR_NULL, "key_cache, value_cache, key, value, block_tables and positions must be non-NULL");
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16) || !aligned(key, 16) || !aligned(value, 16))
    return fail(PA_ERR_ALIGN, "key_cache, value_cache, key and value must be 16-byte aligned");
  if (!aligned(block_tables, 4) || !aligned(positions, 4) || (k_scale && !aligned(k_scale, 4)) ||
      (v_scale && !aligned(v_scale, 4)))
    return fail(PA_ERR_ALIGN, "block_tables, positions and scales must be 4-byte aligned");
  pa::AppendArgs a{};
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.key = key;
  a.value = value;
  a.block_tables = block_tables;
  a.positions = positions;
  const bool fp8 = is_fp8_cache(kv_cache_dtype);
  a.k_scale = fp8 ? k_scale : nullptr;
  a.v_scale = fp8 ? v_scale : nullptr;
  a.num_seqs = num_seqs;
  a.tokens_per_seq = tokens_per_seq;
  a.num_kv_heads = num_kv_heads;
  a.head_size = head_size;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  const int in_kind = in_dtype == PA_DTYPE_F32 ? pa::KIND_F32 : pa::KIND_BF16;
  const int cache_kind = fp8 ? pa::KIND_FP8 : in_kind;
  hipStream_t st = static_cast<hipStream_t>(stream);
  std::unique_lock<std::mutex> lock(g_timing.mu);
  const bool timed = g_timing.on;
  if (!timed) lock.unlock();
  if (timed) record_begin(st);
  hipError_t err = pa::launch_append(a, in_kind, cache_kind, st);
  if (timed) record_end_into(g_timing.app, st);
  if (err != hipSuccess) return fail(PA_ERR_HIP, "append launch failed: %s", hipGetErrorString(err));
  return ok();
}

namespace {

int mla_cache_append(void* latent_cache, const void* rows, int num_seqs, int tokens_per_seq, int num_blocks,
                     const int32_t* block_tables, int max_blocks_per_seq, const int32_t* positions, int block_size,
                     bool fp8, const float* kv_scale, void* stream) {
  if (num_seqs < 0) return fail(PA_ERR_SHAPE, "num_seqs %d < 0", num_seqs);
  if (tokens_per_seq < 1) return fail(PA_ERR_SHAPE, "tokens_per_seq %d must be positive", tokens_per_seq);
  if (block_size != 16 && block_size != 32) return fail(PA_ERR_SHAPE, "block_size %d is not 16 or 32", block_size);
  if (num_blocks <= 0) return fail(PA_ERR_SHAPE, "num_blocks %d must be positive", num_blocks);
  if (max_blocks_per_seq <= 0) return fail(PA_ERR_SHAPE, "max_blocks_per_seq %d must be positive", max_blocks_per_seq);
  if ((int64_t)num_seqs * tokens_per_seq >= ((int64_t)1 << 31))
    return fail(PA_ERR_SHAPE, "num_seqs * tokens_per_seq must be below 2^31");
  if (num_seqs == 0) return ok();
  if (!latent_cache || !rows || !block_tables || !positions)
    return fail(PA_ERR_NULL, "latent_cache, rows, block_tables and positions must be non-NULL");
  if (!aligned(latent_cache, 16) || !aligned(rows, 16))
    return fail(PA_ERR_ALIGN, "latent_cache and rows must be 16-byte aligned");
  if (!aligned(block_tables, 4) || !aligned(positions, 4) || (kv_scale && !aligned(kv_scale, 4)))
    return fail(PA_ERR_ALIGN, "block_tables, positions and kv_scale must be 4-byte aligned");
  const uint64_t width = PA_MLA_LATENT_DIM + PA_MLA_ROPE_DIM;
  const uint64_t cache_bytes = (uint64_t)num_blocks * width * block_size * (fp8 ? 1 : 2);
  const uint64_t rows_bytes = (uint64_t)num_seqs * tokens_per_seq * width * 2;
  const uintptr_t c0 = reinterpret_cast<uintptr_t>(latent_cache), r0 = reinterpret_cast<uintptr_t>(rows);
  if (c0 < r0 + rows_bytes && r0 < c0 + cache_bytes) return fail(PA_ERR_SHAPE, "rows overlap latent_cache");
  pa::LatentAppendArgs a{};
  a.latent_cache = latent_cache;
  a.rows = rows;
  a.block_tables = block_tables;
  a.positions = positions;
  a.num_seqs = num_seqs;
  a.tokens_per_seq = tokens_per_seq;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.block_size = block_size;
  a.kv_scale = fp8 ? kv_scale : nullptr;
  a.fp8 = fp8 ? 1 : 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  std::unique_lock<std::mutex> lock(g_timing.mu);
  const bool timed = g_timing.on;
  if (!timed) lock.unlock();
  if (timed) record_begin(st);
  hipError_t err = pa::launch_latent_append(a, st);
  if (timed) record_end_into(g_timing.app, st);
  if (err != hipSuccess) return fail(PA_ERR_HIP, "latent append launch failed: %s", hipGetErrorString(err));
  return ok();
}

}  // namespace

int pa_mla_cache_append(void* latent_cache, const void* rows, int num_seqs, int tokens_per_seq, int num_blocks,
                        const int32_t* block_tables, int max_blocks_per_seq, const int32_t* positions,
                        int block_size, void* stream) {
  return mla_cache_append(latent_cache, rows, num_seqs, tokens_per_seq, num_blocks, block_tables,
                          max_blocks_per_seq, positions, block_size, false, nullptr, stream);
}

int pa_mla_cache_append_fp8(void* latent_cache, const void* rows, int num_seqs, int tokens_per_seq,
                            int num_blocks, const int32_t* block_tables, int max_blocks_per_seq,
                            const int32_t* positions, int block_size, const float* kv_scale, void* stream) {
  return mla_cache_append(latent_cache, rows, num_seqs, tokens_per_seq, num_blocks, block_tables,
                          max_blocks_per_seq, positions, block_size, true, kv_scale, stream);
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

int pa_version(void) { return 100; }

int pa_mla_workspace_bytes(int num_seqs, int num_heads, size_t* bytes) {
  if (!bytes) return fail(PA_ERR_NULL, "bytes is NULL");
  const int rc = check_mla_plan_args(num_seqs, num_heads);
  if (rc) return rc;
  // One size serves both cache types.
  *bytes = num_seqs == 0 ? 0
                         : std::max(make_mla_plan(num_seqs, num_heads, false).bytes,
                                    make_mla_plan(num_seqs, num_heads, true).bytes);
  return ok();
}

namespace {

int mla_decode(void* out, const void* query, const void* latent_cache, int num_seqs, int num_heads, int num_blocks,
               float scale, const int32_t* block_tables, int max_blocks_per_seq, const int32_t* seq_lens,
               int block_size, int max_seq_len, bool fp8, const float* kv_scale, void* workspace,
               size_t workspace_bytes, void* stream) {
  int rc = check_mla_plan_args(num_seqs, num_heads);
  if (rc) return rc;
  if (block_size != 16 && block_size != 32) return fail(PA_ERR_SHAPE, "block_size %d is not 16 or 32", block_size);
  if (max_seq_len < 0) return fail(PA_ERR_SHAPE, "max_seq_len %d < 0", max_seq_len);
  if (num_seqs == 0) return ok();
  if (!out || !query || !latent_cache || !block_tables || !seq_lens)
    return fail(PA_ERR_NULL, "out, query, latent_cache, block_tables and seq_lens must be non-NULL");
  if (num_blocks <= 0) return fail(PA_ERR_SHAPE, "num_blocks %d must be positive", num_blocks);
  if (max_blocks_per_seq <= 0) return fail(PA_ERR_SHAPE, "max_blocks_per_seq %d must be positive", max_blocks_per_seq);
  if ((int64_t)max_seq_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PA_ERR_SHAPE, "max_seq_len %d exceeds max_blocks_per_seq*block_size = %lld", max_seq_len,
                (long long)max_blocks_per_seq * block_size);
  if (!std::isfinite(scale)) return fail(PA_ERR_SHAPE, "scale is not finite");
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(latent_cache, 16))
    return fail(PA_ERR_ALIGN, "out, query and latent_cache must be 16-byte aligned");
  if (!aligned(block_tables, 4) || !aligned(seq_lens, 4) || (kv_scale && !aligned(kv_scale, 4)))
    return fail(PA_ERR_ALIGN, "block_tables, seq_lens and kv_scale must be 4-byte aligned");
  const size_t q_bytes = (size_t)num_seqs * num_heads * (PA_MLA_LATENT_DIM + PA_MLA_ROPE_DIM) * 2;
  const size_t o_bytes = (size_t)num_seqs * num_heads * PA_MLA_LATENT_DIM * 2;
  const uintptr_t o0 = reinterpret_cast<uintptr_t>(out), q0 = reinterpret_cast<uintptr_t>(query);
  if (o0 < q0 + q_bytes && q0 < o0 + o_bytes) return fail(PA_ERR_SHAPE, "out overlaps query");
  const MlaPlan plan = make_mla_plan(num_seqs, num_heads, fp8);
  if ((rc = check_workspace(workspace, workspace_bytes, plan.bytes))) return rc;
  if ((rc = maybe_validate_device(seq_lens, block_tables, num_seqs, max_blocks_per_seq, block_size, max_seq_len,
                                  num_blocks, stream)))
    return rc;

  pa::MlaArgs a{};
  pa::DecodeArgs& d = a.d;
  d.out = out;
  d.query = query;
  d.key_cache = latent_cache;
  d.value_cache = latent_cache;
  d.block_tables = block_tables;
  d.seq_lens = seq_lens;
  char* ws = static_cast<char*>(workspace);
  d.seg_out = reinterpret_cast<float*>(ws + plan.off[0]);
  d.seg_max = reinterpret_cast<float*>(ws + plan.off[1]);
  d.seg_sum = reinterpret_cast<float*>(ws + plan.off[2]);
  d.seg_meta = reinterpret_cast<int32_t*>(ws + plan.off[3]);
  d.k_block_stride_bytes = (int64_t)(PA_MLA_LATENT_DIM + PA_MLA_ROPE_DIM) * block_size * (fp8 ? 1 : 2);
  d.v_block_stride_bytes = d.k_block_stride_bytes;
  d.k_scale = fp8 ? kv_scale : nullptr;
  d.v_scale = d.k_scale;
  d.scale = scale;
  d.num_seqs = num_seqs;
  d.num_heads = num_heads;
  d.num_kv_heads = 1;
  d.group = 16;
  d.head_size = PA_MLA_LATENT_DIM + PA_MLA_ROPE_DIM;
  d.block_size = block_size;
  d.num_blocks = num_blocks;
  d.max_blocks_per_seq = max_blocks_per_seq;
  d.max_seq_len = max_seq_len;
  a.head_groups = plan.head_groups;
  a.waves_per_wg = plan.waves_per_wg;
  a.chunks = plan.chunks;
  a.shares = plan.shares;
  a.hpad = plan.hpad;
  a.wide = plan.wide ? 1 : 0;
  a.fp8 = fp8 ? 1 : 0;
  d.streamk_workgroups = a.shares * a.chunks;

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
  hipError_t err = pa::launch_mla(a, static_cast<hipStream_t>(stream), hooks);
  if (err != hipSuccess) return fail(PA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return ok();
}

}  // namespace

int pa_mla_decode(void* out, const void* query, const void* latent_cache, int num_seqs, int num_heads,
                  int num_blocks, float scale, const int32_t* block_tables, int max_blocks_per_seq,
                  const int32_t* seq_lens, int block_size, int max_seq_len, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return mla_decode(out, query, latent_cache, num_seqs, num_heads, num_blocks, scale, block_tables,
                    max_blocks_per_seq, seq_lens, block_size, max_seq_len, false, nullptr, workspace,
                    workspace_bytes, stream);
}

int pa_mla_decode_fp8(void* out, const void* query, const void* latent_cache, int num_seqs, int num_heads,
                      int num_blocks, float scale, const int32_t* block_tables, int max_blocks_per_seq,
                      const int32_t* seq_lens, int block_size, int max_seq_len, const float* kv_scale,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return mla_decode(out, query, latent_cache, num_seqs, num_heads, num_blocks, scale, block_tables,
                    max_blocks_per_seq, seq_lens, block_size, max_seq_len, true, kv_scale, workspace,
                    workspace_bytes, stream);
}

int pa_timing_enable(int on) {
  std::lock_guard<std::mutex> g(g_timing.mu);
  g_timing.on = on != 0;
  return ok();
}

int pa_timing_read(double* partition_ms, int* partition_launches, double* reduce_ms, int* reduce_launches) {
  std::lock_guard<std::mutex> g(g_timing.mu);
  double tp = 0, tr = 0;
  int np = 0, nr = 0;
  hipError_t e1 = drain_events(g_timing.part, tp, np);
  hipError_t e2 = drain_events(g_timing.red, tr, nr);
  if (partition_ms) *partition_ms = tp;
  if (partition_launches) *partition_launches = np;
  if (reduce_ms) *reduce_ms = tr;
  if (reduce_launches) *reduce_launches = nr;
  const hipError_t err = e1 != hipSuccess ? e1 : e2;
  if (err != hipSuccess) return fail(PA_ERR_HIP, "event timing failed: %s", hipGetErrorString(err));
  return ok();
}

int pa_timing_read_append(double* append_ms, int* append_launches) {
  std::lock_guard<std::mutex> g(g_timing.mu);
  double t = 0;
  int n = 0;
  hipError_t err = drain_events(g_timing.app, t, n);
  if (append_ms) *append_ms = t;
  if (append_launches) *append_launches = n;
  if (err != hipSuccess) return fail(PA_ERR_HIP, "event timing failed: %s", hipGetErrorString(err));
  return ok();
}

}  // extern "C"
