/*
 * pa_blocks.h — host block pool for the paged KV cache (libpa_decode.so).
 *
 * The cache is a pool of fixed-size physical blocks; each sequence owns a
 * row of the int32 block table that maps its logical blocks to physical ones
 * (10100.com retirement article, §1). Blocks are taken on demand as a
 * sequence grows, and several sequences may map logical blocks to the same
 * physical block — parallel sampling, beam search, a shared prompt — with a
 * block copied only when a sequence writes into a block others still read
 * (copy-on-write) ("vLLM 0.25.0 解读：PagedAttention 退场，MRv2 接管", §1:
 * on-demand allocation, sharing, copy-on-write).
 *
 * The pool keeps a reference count per physical block and a free list. It is
 * host-only bookkeeping (no HIP call); the caller applies the copies it asks
 * for with pa_copy_blocks and keeps the device copy of the table in sync.
 * Every entry point validates its arguments, returns PA_OK or a negative
 * PA_ERR_* code (pa_decode.h; PA_ERR_NOMEM when the pool is exhausted) and
 * leaves the pool unchanged on failure. A pool is internally locked, so
 * calls from several host threads are serialised.
 */
#ifndef PA_BLOCKS_H
#define PA_BLOCKS_H

#include <stddef.h>
#include <stdint.h>

#include "pa_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ERR_NOMEM (-7)  /* not enough free blocks in the pool */

typedef struct pa_block_pool pa_block_pool;

/* A pool of num_blocks (> 0) physical blocks of block_size (> 0) tokens,
 * all free. Free blocks are handed out lowest id first. *pool receives the
 * handle (owned by the caller; release with pa_pool_destroy). */
int pa_pool_create(int num_blocks, int block_size, pa_block_pool** pool);
void pa_pool_destroy(pa_block_pool* pool);

/* Number of free blocks, and the reference count of one block (0 = free). */
int pa_pool_num_free(const pa_block_pool* pool, int* num_free);
int pa_pool_refcount(const pa_block_pool* pool, int32_t block, int* refcount);

/*
 * Make room for num_new (>= 1) tokens appended to a sequence that holds
 * seq_len (>= 0) tokens in table_row[0 .. ceil(seq_len / block_size)).
 * table_row: host int32 [max_blocks], updated in place. Blocks for the new
 * positions seq_len .. seq_len+num_new-1 that the row does not yet hold are
 * taken from the free list (refcount 1). If the block that receives the first
 * new token already holds tokens and is shared (refcount > 1), it is replaced
 * in table_row by a fresh block (copy-on-write): *cow_src / *cow_dst receive
 * the (shared, fresh) pair, the shared block's count drops by one, and
 * *num_cow is 1; otherwise *num_cow is 0. The caller must copy cow_src to
 * cow_dst on the device (pa_copy_blocks) before writing the new tokens.
 * Errors: PA_ERR_SHAPE if the new tokens do not fit in max_blocks blocks,
 * PA_ERR_NOMEM if the pool cannot supply the blocks (nothing changes).
 */
int pa_pool_append(pa_block_pool* pool, int32_t* table_row, int max_blocks, int seq_len, int num_new,
                   int32_t* cow_src, int32_t* cow_dst, int* num_cow);

/* Share a sequence: dst_row[i] = src_row[i] for the ceil(seq_len /
 * block_size) blocks of the source, each of which gains one reference.
 * dst_row must have room for them (max_blocks). */
int pa_pool_fork(pa_block_pool* pool, const int32_t* src_row, int seq_len, int32_t* dst_row,
                 int max_blocks);

/* Drop a sequence: each of its ceil(seq_len / block_size) blocks loses one
 * reference and returns to the free list at zero. */
int pa_pool_release(pa_block_pool* pool, const int32_t* table_row, int seq_len);

/*
 * Device copy of whole physical blocks, both caches: for each i < num_pairs,
 * block dst[i] of key_cache and of value_cache becomes a copy of block
 * src[i] (all kv heads). src, dst: device int32 [num_pairs]; pairs with an id
 * outside [0, num_blocks) are skipped; a dst that is also some src, or that
 * repeats, gives unspecified contents. block_bytes: bytes of one physical
 * block of one cache (num_kv_heads * head_size * block_size * element size,
 * a positive multiple of 16). Caches 16-B aligned. Asynchronous on stream.
 */
int pa_copy_blocks(void* key_cache, void* value_cache, const int32_t* src, const int32_t* dst,
                   int num_pairs, int num_blocks, size_t block_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKS_H */
