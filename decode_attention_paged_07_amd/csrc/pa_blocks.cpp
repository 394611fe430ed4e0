// Host block pool (include/pa_blocks.h): reference counts, a free list
// handed out lowest id first, on-demand growth and copy-on-write of a shared
// partially filled block.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <functional>
#include <mutex>
#include <queue>
#include <string>
#include <vector>

#include "pa_blocks.h"
#include "pa_kernels.h"

// Shared with pa_api.cpp: sets the thread's last-error text, returns code.
__attribute__((visibility("hidden"))) int pa_internal_fail(int code, const char* fmt, ...);
__attribute__((visibility("hidden"))) int pa_internal_ok();

struct pa_block_pool {
  int num_blocks = 0;
  int block_size = 0;
  std::vector<int> refs;                                             // per block, 0 = free
  std::priority_queue<int, std::vector<int>, std::greater<int>> free_ids;
  mutable std::mutex mu;
};

namespace {

int blocks_for(int tokens, int bs) { return tokens <= 0 ? 0 : (tokens + bs - 1) / bs; }

// Checks that row[0..n) names live blocks of the pool.
int check_row(const pa_block_pool* p, const int32_t* row, int n) {
  for (int i = 0; i < n; ++i) {
    const int32_t b = row[i];
    if (b < 0 || b >= p->num_blocks)
      return pa_internal_fail(PA_ERR_SHAPE, "table entry %d = %d is outside the pool of %d blocks", i, b,
                              p->num_blocks);
    if (p->refs[b] <= 0) return pa_internal_fail(PA_ERR_SHAPE, "table entry %d names free block %d", i, b);
  }
  return PA_OK;
}

int take(pa_block_pool* p) {
  const int b = p->free_ids.top();
  p->free_ids.pop();
  p->refs[b] = 1;
  return b;
}

void drop(pa_block_pool* p, int b) {
  if (--p->refs[b] == 0) p->free_ids.push(b);
}

}  // namespace

extern "C" {

int pa_pool_create(int num_blocks, int block_size, pa_block_pool** pool) {
  if (!pool) return pa_internal_fail(PA_ERR_NULL, "pool is NULL");
  if (num_blocks <= 0 || block_size <= 0)
    return pa_internal_fail(PA_ERR_SHAPE, "num_blocks %d and block_size %d must be positive", num_blocks,
                            block_size);
  auto* p = new pa_block_pool;
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->refs.assign(num_blocks, 0);
  for (int b = 0; b < num_blocks; ++b) p->free_ids.push(b);
  *pool = p;
  return pa_internal_ok();
}

void pa_pool_destroy(pa_block_pool* pool) { delete pool; }

int pa_pool_num_free(const pa_block_pool* pool, int* num_free) {
  if (!pool || !num_free) return pa_internal_fail(PA_ERR_NULL, "pool and num_free must be non-NULL");
  std::lock_guard<std::mutex> g(pool->mu);
  *num_free = (int)pool->free_ids.size();
  return pa_internal_ok();
}

int pa_pool_refcount(const pa_block_pool* pool, int32_t block, int* refcount) {
  if (!pool || !refcount) return pa_internal_fail(PA_ERR_NULL, "pool and refcount must be non-NULL");
  std::lock_guard<std::mutex> g(pool->mu);
  if (block < 0 || block >= pool->num_blocks)
    return pa_internal_fail(PA_ERR_SHAPE, "block %d is outside the pool of %d blocks", block, pool->num_blocks);
  *refcount = pool->refs[block];
  return pa_internal_ok();
}

int pa_pool_append(pa_block_pool* pool, int32_t* table_row, int max_blocks, int seq_len, int num_new,
                   int32_t* cow_src, int32_t* cow_dst, int* num_cow) {
  if (!pool || !table_row || !cow_src || !cow_dst || !num_cow)
    return pa_internal_fail(PA_ERR_NULL, "pool, table_row, cow_src, cow_dst and num_cow must be non-NULL");
  if (seq_len < 0 || num_new < 1 || max_blocks < 0)
    return pa_internal_fail(PA_ERR_SHAPE, "seq_len %d must be >= 0, num_new %d >= 1, max_blocks %d >= 0",
                            seq_len, num_new, max_blocks);
  std::lock_guard<std::mutex> g(pool->mu);
  const int bs = pool->block_size;
  const int have = blocks_for(seq_len, bs);
  if ((int64_t)seq_len + num_new > (int64_t)max_blocks * bs)
    return pa_internal_fail(PA_ERR_SHAPE, "%d + %d tokens do not fit in %d blocks of %d", seq_len, num_new,
                            max_blocks, bs);
  if (have > max_blocks) return pa_internal_fail(PA_ERR_SHAPE, "seq_len %d exceeds the row", seq_len);
  int rc = check_row(pool, table_row, have);
  if (rc) return rc;
  const int need = blocks_for(seq_len + num_new, bs);
  const bool cow = (seq_len % bs) != 0 && pool->refs[table_row[have - 1]] > 1;
  const int fresh = need - have + (cow ? 1 : 0);
  if ((int)pool->free_ids.size() < fresh)
    return pa_internal_fail(PA_ERR_NOMEM, "need %d free blocks, the pool has %d", fresh,
                            (int)pool->free_ids.size());
  *num_cow = 0;
  if (cow) {
    const int old = table_row[have - 1];
    const int nb = take(pool);
    drop(pool, old);
    table_row[have - 1] = nb;
    *cow_src = old;
    *cow_dst = nb;
    *num_cow = 1;
  }
  for (int i = have; i < need; ++i) table_row[i] = take(pool);
  return pa_internal_ok();
}

int pa_pool_fork(pa_block_pool* pool, const int32_t* src_row, int seq_len, int32_t* dst_row, int max_blocks) {
  if (!pool || !src_row || !dst_row) return pa_internal_fail(PA_ERR_NULL, "pool, src_row and dst_row must be non-NULL");
  if (seq_len < 0) return pa_internal_fail(PA_ERR_SHAPE, "seq_len %d < 0", seq_len);
  std::lock_guard<std::mutex> g(pool->mu);
  const int n = blocks_for(seq_len, pool->block_size);
  if (n > max_blocks) return pa_internal_fail(PA_ERR_SHAPE, "%d blocks do not fit in a row of %d", n, max_blocks);
  int rc = check_row(pool, src_row, n);
  if (rc) return rc;
  for (int i = 0; i < n; ++i) {
    ++pool->refs[src_row[i]];
    dst_row[i] = src_row[i];
  }
  return pa_internal_ok();
}

int pa_pool_release(pa_block_pool* pool, const int32_t* table_row, int seq_len) {
  if (!pool || (!table_row && seq_len > 0)) return pa_internal_fail(PA_ERR_NULL, "pool and table_row must be non-NULL");
  if (seq_len < 0) return pa_internal_fail(PA_ERR_SHAPE, "seq_len %d < 0", seq_len);
  std::lock_guard<std::mutex> g(pool->mu);
  const int n = blocks_for(seq_len, pool->block_size);
  int rc = check_row(pool, table_row, n);
  if (rc) return rc;
  // A row may name a block twice only if that block holds enough references.
  std::vector<int32_t> ids(table_row, table_row + n);
  std::sort(ids.begin(), ids.end());
  for (int i = 0; i < n;) {
    int j = i;
    while (j < n && ids[j] == ids[i]) ++j;
    if (pool->refs[ids[i]] < j - i)
      return pa_internal_fail(PA_ERR_SHAPE, "block %d is named %d times but holds %d references", ids[i], j - i,
                              pool->refs[ids[i]]);
    i = j;
  }
  for (int i = 0; i < n; ++i) drop(pool, table_row[i]);
  return pa_internal_ok();
}

int pa_copy_blocks(void* key_cache, void* value_cache, const int32_t* src, const int32_t* dst, int num_pairs,
                   int num_blocks, size_t block_bytes, void* stream) {
  if (num_pairs < 0) return pa_internal_fail(PA_ERR_SHAPE, "num_pairs %d < 0", num_pairs);
  if (num_pairs == 0) return pa_internal_ok();
  if (!key_cache || !value_cache || !src || !dst)
    return pa_internal_fail(PA_ERR_NULL, "key_cache, value_cache, src and dst must be non-NULL");
  if (num_blocks <= 0) return pa_internal_fail(PA_ERR_SHAPE, "num_blocks %d must be positive", num_blocks);
  if (block_bytes == 0 || block_bytes % 16)
    return pa_internal_fail(PA_ERR_SHAPE, "block_bytes %zu is not a positive multiple of 16", block_bytes);
  if ((reinterpret_cast<uintptr_t>(key_cache) | reinterpret_cast<uintptr_t>(value_cache)) % 16 ||
      (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 4)
    return pa_internal_fail(PA_ERR_ALIGN, "caches must be 16-B aligned, src and dst 4-B aligned");
  hipError_t err = pa::launch_copy_blocks(key_cache, value_cache, src, dst, num_pairs, num_blocks, block_bytes,
                                          static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return pa_internal_fail(PA_ERR_HIP, "copy launch failed: %s", hipGetErrorString(err));
  return pa_internal_ok();
}

}  // extern "C"
