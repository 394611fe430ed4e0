/*
 * pa_decode.h — C ABI of the paged decode-attention library (libpa_decode.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * What it computes. One decode step of PagedAttention: for every sequence s
 * and query head h, the single query row q[s,h,:] attends over the sequence's
 * first seq_lens[s] cached tokens,
 *
 *     out[s,h,:] = sum_t softmax_t( scale * q[s,h,:].K[t,:] + alibi ) * V[t,:]
 *
 * where token t of sequence s lives in physical block
 * block_tables[s, t / block_size] at slot t % block_size (the block-table
 * indirection of the 10100.com retirement article, §1, and of the vLLM 0.25.0
 * notes on jokeuncle.github.io, §1). The attention formula itself was lost in
 * the extraction of that article (§2); this is the standard decode-attention
 * definition the rest of the pages support. The argument list follows the
 * ROCm call kept in the PR #47361 report (prhub.com.cn, "关键源码片段",
 * benchmark and _custom_ops.py snippets), with its three partial-result
 * buffers folded into one caller-provided workspace.
 *
 * Conventions for every entry point:
 *  - Pointers named "device" are HIP device addresses; all others are host.
 *    The caller owns every buffer; the library allocates nothing, keeps no
 *    per-call state, writes only the buffers each call documents as outputs
 *    (`out` and `workspace` for the decode calls, the caches for append and
 *    block copies), and never blocks the host: kernels are queued on `stream` (a hipStream_t; NULL = the null
 *    stream). No host synchronisation and no allocation happen inside a call,
 *    so it can be captured into a HIP graph.
 *  - Every argument is validated on the host before any HIP call; on failure
 *    nothing is launched, a negative PA_ERR_* code is returned and
 *    pa_last_error() describes the problem (thread-local text).
 *  - Values that live in device memory (seq_lens, block-table entries) are the
 *    caller's contract: seq_lens[s] in [0, max_seq_len], entries for the
 *    blocks a sequence uses in [0, num_blocks). The kernels clamp both into
 *    range, so a violation gives unspecified output values but never an
 *    out-of-bounds access.
 *  - Debugging aid: with the environment variable PA_VALIDATE_DEVICE=1, the
 *    decode calls (pa_paged_attention_decode and its _split, _noalloc and
 *    _shared forms, pa_mla_decode and pa_mla_decode_fp8) first copy seq_lens
 *    and the table entries each sequence uses to the host, after the
 *    stream's earlier work, and return PA_ERR_SHAPE, launching nothing, for
 *    a value outside the ranges above. This synchronises the stream (an
 *    exception to "never blocks the host"; no allocation: the copies go
 *    through a fixed buffer), is slow, and is skipped while the stream is
 *    being captured into a graph.
 *  - Results are deterministic for given inputs and launch plan (no atomics).
 */
#ifndef PA_DECODE_H
#define PA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define PA_OK             0
#define PA_ERR_NULL      (-1)  /* a required pointer is NULL                     */
#define PA_ERR_SHAPE     (-2)  /* sizes out of the supported set / inconsistent  */
#define PA_ERR_DTYPE     (-3)  /* unsupported dtype combination                   */
#define PA_ERR_WORKSPACE (-4)  /* workspace missing or smaller than required      */
#define PA_ERR_ALIGN     (-5)  /* pointer not aligned as documented               */
#define PA_ERR_HIP       (-6)  /* the HIP runtime reported an error on launch     */

/* Element types of query/out (q_dtype). */
#define PA_DTYPE_F32   0
#define PA_DTYPE_BF16  1

/* Cache element type (kv_cache_dtype). AUTO = same as q_dtype. FP8_E4M3 =
 * OCP E4M3FN codes (uint8; max 448, no infinities), each decoded value
 * multiplied by *k_scale (K) or *v_scale (V), the scaled conversion of the
 * 10100.com retirement article, §4. FP8 requires q_dtype = BF16. */
#define PA_KV_AUTO      0
#define PA_KV_FP8_E4M3  1
/* The same E4M3FN cache with the attention arithmetic itself in fp8 (the
 * variant of the 10100.com article, §4, that computes in fp8 and converts
 * once at the output): q is quantised to MX fp8 (32 consecutive head dims
 * share a power-of-two scale 2^X, X = floor(log2 max|q|) - 8, elements the
 * nearest e4m3 of q / 2^X, saturating at 448); S = K q^T and O = V^T P run
 * on fp8 operands with fp32 accumulation; each cache block's probabilities
 * are quantised to e4m3 as p = 2^(z - ceil(max z)) (z the log2-domain
 * logits of that block), and out = v_scale * sum_b 2^ceil_b sum_t p_t V_t /
 * sum_b 2^ceil_b sum_t p_t. Requires bf16 queries. */
#define PA_KV_FP8_E4M3_COMPUTE  2

/* Sizes: the default tokens per cache block (16; 32 is also accepted), and
 * the partition granularity of the split-KV path (the 256-token partitions
 * of the PR #47361 report). */
#define PA_BLOCK_SIZE      16
#define PA_PARTITION_SIZE  256
#define PA_MAX_GROUP       16   /* num_heads / num_kv_heads */
#define PA_MAX_SEQS        65535 /* num_seqs, and num_splits of a split plan: a grid dimension */

/*
 * Cache layouts (the pages' layouts, 10100.com retirement article, §2), with
 * x = 16 bytes / element size (4 for f32, 8 for bf16, 16 for fp8):
 *   key_cache   [num_blocks][num_kv_heads][head_size/x][block_size][x]
 *   value_cache [num_blocks][num_kv_heads][head_size][block_size]
 * so one (block, kv head) K tile and V tile are each one contiguous run of
 * head_size*block_size elements. All strides below are in elements.
 */
typedef struct pa_layout_desc {
  int x;                    /* innermost K width                                 */
  int elem_bytes;           /* bytes per cache element                           */
  int64_t k_block_stride;   /* elements between consecutive physical K blocks    */
  int64_t k_head_stride;    /* elements between kv heads inside a K block        */
  int64_t v_block_stride;
  int64_t v_head_stride;
} pa_layout_desc;

/* Describe the cache layout for (num_kv_heads, head_size, block_size, dtypes).
 * Host only; no HIP call. Returns PA_OK or PA_ERR_SHAPE / PA_ERR_DTYPE / PA_ERR_NULL. */
int pa_kv_layout(int num_kv_heads, int head_size, int block_size, int q_dtype,
                 int kv_cache_dtype, pa_layout_desc* desc);

/*
 * Launch plan. requested_split_tokens == 0 selects the default stream-K plan:
 * a persistent grid whose waves take equal, contiguous shares of all
 * (kv head, sequence, block) tiles; a (sequence, kv head) pair cut by a share
 * boundary leaves segment partials in the workspace and a small merge kernel
 * combines them (log-sum-exp merge). Its outputs are split_tokens = 0,
 * num_splits = 0 and its workspace size (layout private to the library).
 *
 * A positive multiple of PA_PARTITION_SIZE selects the split grid: each
 * sequence is divided into splits of split_tokens tokens; one wave handles
 * one (sequence, kv head, split) and the query heads that share that kv head.
 * Sequences longer than one split write per-split partial results into the
 * workspace and a reduce kernel merges them. Outputs (any may be NULL): the
 * split_tokens, num_splits = ceil(max_seq_len / split_tokens) (>= 1), and the
 * workspace bytes this plan needs (0 when num_splits == 1). For the stream-K
 * plan that is the size for the most waves any cache type launches on the
 * current device (its compute-unit count is queried once; 256 is assumed
 * where none can be queried); the decode call itself requires only the size
 * for the grid it launches. No kernel launch.
 *
 * Workspace layout for num_splits = P > 1, all fp32, each array starting at a
 * 256-byte-aligned offset from the workspace base, in this order:
 *   tmp_out    [num_seqs][num_heads][P][head_size]  normalised partial outputs
 *                                                   (already multiplied by *v_scale)
 *   max_logits [num_seqs][num_heads][P]             max of scale*q.k + alibi (natural units)
 *   exp_sums   [num_seqs][num_heads][P]             sum of exp(logit - max_logit)
 * Entries of splits that start at or after a sequence's length are not written.
 */
int pa_decode_plan(int num_seqs, int num_heads, int num_kv_heads, int head_size,
                   int max_seq_len, int requested_split_tokens,
                   int* split_tokens, int* num_splits, size_t* workspace_bytes);

/* Workspace bytes sufficient for every plan of this problem: the 256-token
 * split plan and the stream-K plan of every valid num_kv_heads. No kernel
 * launch (the device's compute-unit count is queried as for pa_decode_plan). */
int pa_workspace_bytes(int num_seqs, int num_heads, int head_size, int max_seq_len,
                       size_t* bytes);

/*
 * The decode step. Arguments:
 *   out          device, [num_seqs][num_heads][head_size], q_dtype, contiguous,
 *                16-byte aligned, must not overlap `query`.
 *   query        device, [num_seqs][num_heads][head_size], q_dtype, contiguous, 16-B aligned.
 *   key_cache    device, layout above, 16-B aligned.  value_cache  likewise.
 *   num_seqs     0 .. PA_MAX_SEQS (0 is a no-op). num_heads, num_kv_heads: > 0,
 *                num_heads % num_kv_heads == 0, group <= PA_MAX_GROUP; query
 *                head h uses kv head h / (num_heads / num_kv_heads).
 *   head_size    32, 64 or 128 (64 and 128 are the PR #47361 report's test sizes;
 *                32 is among the 10100.com article's kernel instantiations, §5).
 *   num_blocks   physical blocks in each cache (> 0).
 *   scale        finite; multiplies q.k (not the ALiBi term).
 *   block_tables device int32 [num_seqs][max_blocks_per_seq], 4-B aligned.
 *   seq_lens     device int32 [num_seqs].
 *   block_size   tokens per cache block: 16 or 32.
 *   max_seq_len  >= every seq_lens[s], <= max_blocks_per_seq * block_size.
 *   alibi_slopes device fp32 [num_heads] or NULL; adds
 *                slope[h] * (t - (seq_len - 1)) to the logit of token t.
 *   q_dtype, kv_cache_dtype: see above.
 *   k_scale, v_scale: device fp32 scalars or NULL (= 1.0); used only with
 *                the fp8 cache (PA_KV_FP8_E4M3 or PA_KV_FP8_E4M3_COMPUTE).
 *   workspace    device, >= the plan's workspace bytes (may be NULL when the
 *                plan needs none), 16-B aligned.
 *   stream       hipStream_t or NULL.
 * A sequence with seq_lens[s] == 0 gets an all-zero output row.
 */
int pa_paged_attention_decode(void* out, const void* query, const void* key_cache,
                              const void* value_cache, int num_seqs, int num_heads,
                              int num_kv_heads, int head_size, int num_blocks, float scale,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* seq_lens, int block_size, int max_seq_len,
                              const float* alibi_slopes, int q_dtype, int kv_cache_dtype,
                              const float* k_scale, const float* v_scale, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Same as pa_paged_attention_decode with an explicit split size (see
 * pa_decode_plan; 0 = library's choice). */
int pa_paged_attention_decode_split(void* out, const void* query, const void* key_cache,
                                    const void* value_cache, int num_seqs, int num_heads,
                                    int num_kv_heads, int head_size, int num_blocks,
                                    float scale, const int32_t* block_tables,
                                    int max_blocks_per_seq, const int32_t* seq_lens,
                                    int block_size, int max_seq_len,
                                    const float* alibi_slopes, int q_dtype,
                                    int kv_cache_dtype, const float* k_scale,
                                    const float* v_scale, void* workspace,
                                    size_t workspace_bytes, void* stream,
                                    int split_tokens);

/*
 * Decode that allocates nothing, for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. The same computation, plan
 * (stream-K) and kernels as pa_paged_attention_decode, with the workspace in
 * a static device array of PA_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends. Arguments, validation and
 * errors as for pa_paged_attention_decode, without the workspace arguments;
 * in addition PA_ERR_WORKSPACE when the call needs more workspace than
 * PA_NOALLOC_SCRATCH_BYTES (the need grows with num_seqs * num_kv_heads,
 * the group size and head_size; nothing is launched then), and PA_ERR_HIP
 * when the array's device address cannot be looked up (done once per device,
 * on the first call with that device current). The call itself allocates
 * nothing: no hipMalloc, no hipFree.
 * Every call on a GPU uses that GPU's one array: calls whose executions may
 * overlap (on different streams without ordering between them, or from
 * several host threads) race on it and give wrong results. Calls ordered on
 * one stream are safe. The array keeps the last call's contents; no call
 * depends on them.
 */
#define PA_NOALLOC_SCRATCH_BYTES (32u << 20)
int pa_paged_attention_decode_noalloc(void* out, const void* query, const void* key_cache,
                                      const void* value_cache, int num_seqs, int num_heads,
                                      int num_kv_heads, int head_size, int num_blocks, float scale,
                                      const int32_t* block_tables, int max_blocks_per_seq,
                                      const int32_t* seq_lens, int block_size, int max_seq_len,
                                      const float* alibi_slopes, int q_dtype, int kv_cache_dtype,
                                      const float* k_scale, const float* v_scale, void* stream);

/*
 * HBM read-bandwidth probe (measurement aid, not part of the decode path):
 * reads every byte of `buf` once with the decode kernels' load form
 * (16-byte non-temporal loads, 1 KiB contiguous per wave instruction) using
 * `workgroups` workgroups of 256 threads, on `stream`. Timing the call gives
 * the read bandwidth a pure streaming kernel reaches on the device, the
 * practical ceiling for the decode kernels. buf: device, 16-B aligned,
 * bytes a positive multiple of 16. sink: device, 4 bytes, written only in the
 * (practically impossible) case that the XOR of all words read equals
 * 0x9E3779B9. workgroups in [1, 1<<20]. Errors as for the decode call.
 */
int pa_hbm_read_probe(const void* buf, size_t bytes, int workgroups, unsigned* sink, void* stream);

/*
 * HBM gather probe (measurement aid, not part of the decode path): reads the
 * whole tiles ids[0..num_tiles) of `pool`, tile t being bytes
 * [t*tile_bytes, (t+1)*tile_bytes), the way the decode kernels read one
 * (block, kv head) K or V tile. Wave w of the grid reads tiles w, w+W, ...
 * (W = 4*workgroups waves of 64 lanes), `depth` tiles in flight before any
 * is consumed. pool: device, 16-B aligned, pool_bytes >= tile_bytes.
 * tile_bytes: 1024, 2048, 4096, 8192 or 18432 (one 16-token block of the
 * latent cache). ids: device int32 [num_tiles];
 * entries outside the pool are clamped into it; num_tiles in [1, 1<<28].
 * depth: 1 or 2.
 * workgroups in [1, 1<<20]; sink as for pa_hbm_read_probe.
 */
int pa_hbm_gather_probe(const void* pool, size_t pool_bytes, int tile_bytes, const int32_t* ids,
                        int num_tiles, int depth, int workgroups, unsigned* sink, void* stream);

/*
 * KV-cache append: store the K and V rows of new tokens in the paged cache,
 * the step before attention in every decode iteration (the cache grows one
 * token per step; "vLLM 0.25.0 解读" §1). Token j (0 <= j < tokens_per_seq)
 * of sequence s goes to logical position p = positions[s] + j, i.e. physical
 * block block_tables[s, p / block_size], slot p % block_size (10100.com
 * retirement article, §1), written in the cache layouts described by
 * pa_kv_layout.
 *   key_cache, value_cache  device, the caches (16-B aligned); written only at
 *                the slots named by the positions.
 *   key, value   device, [num_seqs][tokens_per_seq][num_kv_heads][head_size],
 *                element type in_dtype, contiguous, 16-B aligned.
 *   num_seqs >= 0 (0 is a no-op); tokens_per_seq >= 1; num_kv_heads > 0;
 *   head_size 32, 64 or 128; num_blocks > 0; max_blocks_per_seq > 0 (table
 *   stride); block_size 16 or 32;
 *   num_seqs * tokens_per_seq * num_kv_heads < 2^31.
 *   block_tables device int32 [num_seqs][max_blocks_per_seq]; positions device
 *   int32 [num_seqs]. A negative position skips the sequence; positions past
 *   max_blocks_per_seq*block_size and table entries outside [0, num_blocks) are not
 *   written.
 *   in_dtype: PA_DTYPE_F32 or PA_DTYPE_BF16. kv_cache_dtype: PA_KV_AUTO (the
 *   cache holds in_dtype and the rows are copied unchanged) or
 *   PA_KV_FP8_E4M3: each element is stored as the E4M3FN code nearest to
 *   value / scale (float32 quotient, ties to even, magnitude saturated at
 *   448, NaN -> 0x7F, sign kept), scale = *k_scale for K and *v_scale for V
 *   (device fp32 scalars; NULL = 1.0), the inverse of the decode call's
 *   dequantisation (10100.com article, §4). PA_KV_FP8_E4M3_COMPUTE stores
 *   the same codes.
 * Two tokens naming the same slot leave either one. Asynchronous on `stream`;
 * no allocation; host-side validation as for the decode call.
 */
int pa_kv_cache_append(void* key_cache, void* value_cache, const void* key, const void* value,
                       int num_seqs, int tokens_per_seq, int num_kv_heads, int head_size,
                       int num_blocks, const int32_t* block_tables, int max_blocks_per_seq,
                       const int32_t* positions, int block_size, int in_dtype,
                       int kv_cache_dtype, const float* k_scale, const float* v_scale,
                       void* stream);

/*
 * Shared-prefix decode: the same result as pa_paged_attention_decode, for a
 * batch in which groups of sequences map their first blocks to the same
 * physical blocks (a forked prompt: parallel sampling, beam search, a shared
 * system prompt; "vLLM 0.25.0 解读" §1 on sharing). Each shared K/V tile is
 * read once per group: the query heads of up to 16*T/G members (T = 4 tiles
 * of 16 MFMA columns; 2 for fp32 queries at head_size 128) are multiplied
 * against it together. Each sequence's remaining blocks are processed on
 * their own and a log-sum-exp merge combines the two parts.
 * Arguments as for pa_paged_attention_decode, plus (device int32 arrays):
 *   num_groups >= 0; group_start [num_groups + 1]: members of group g are
 *   group_seqs[group_start[g] .. group_start[g+1]) (num_members entries in
 *   all; each sequence in at most one group); group_prefix_blocks
 *   [num_groups]: P_g, the number of leading logical blocks all members map
 *   to the same physical blocks, each member holding at least
 *   P_g * block_size tokens; seq_prefix_blocks [num_seqs]: P_g of the sequence's group, 0 if
 *   it is in none. max_group_size >= the largest group (host), and
 *   max_prefix_blocks >= every P_g (host; P_g beyond it are cut to it).
 *   Sequences in no group are computed as by the plain call.
 *   workspace: >= pa_shared_workspace_bytes(...) bytes.
 * Device values that break this contract give unspecified output but no
 * access outside the arrays (ids and offsets are clamped).
 */
int pa_shared_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads, int head_size,
                              int block_size, int max_seq_len, int num_groups,
                              int max_group_size, int max_prefix_blocks, size_t* bytes);

int pa_paged_attention_decode_shared(void* out, const void* query, const void* key_cache,
                                     const void* value_cache, int num_seqs, int num_heads,
                                     int num_kv_heads, int head_size, int num_blocks, float scale,
                                     const int32_t* block_tables, int max_blocks_per_seq,
                                     const int32_t* seq_lens, int block_size, int max_seq_len,
                                     const float* alibi_slopes, int q_dtype, int kv_cache_dtype,
                                     const float* k_scale, const float* v_scale, int num_groups,
                                     const int32_t* group_start, const int32_t* group_seqs,
                                     int num_members, const int32_t* group_prefix_blocks,
                                     const int32_t* seq_prefix_blocks, int max_group_size,
                                     int max_prefix_blocks, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * Latent-cache (MLA) decode. Multi-head latent attention, as the 10100.com
 * retirement article (§2) describes it: each token stores one compressed row
 * [c_kv, k_rope] instead of separate K and V. The call computes the absorbed
 * decode step, for every sequence s and query head h:
 *
 *     out[s,h,:] = sum_t softmax_t( scale * q[s,h,:] . row_t ) * row_t[0:512]
 *
 * over the first seq_lens[s] tokens, where row_t = [c_kv_t (512), k_rope_t
 * (64)] (DeepSeek-V2's widths; the article's figures for them did not survive
 * extraction). q[s,h,:] is the absorbed query [q_nope_h W_UK_h, q_rope_h]
 * (576 wide); out is the latent output (512 wide) before the up-projection
 * W_UV_h, which is outside this call.
 *
 *   query        device, bf16 [num_seqs][num_heads][576], 16-byte aligned
 *   latent_cache device, bf16 [num_blocks][576/8][block_size][8] (the pages'
 *                K layout, §2, with one kv head and x = 8), 16-byte aligned
 *   out          device, bf16 [num_seqs][num_heads][512], 16-byte aligned,
 *                not overlapping query
 *   block_tables, seq_lens, max_seq_len: as for pa_paged_attention_decode
 *   block_size   16 or 32; num_heads in [1, PA_MLA_MAX_HEADS]
 *   workspace    device, at least pa_mla_workspace_bytes(num_seqs,
 *                num_heads) bytes, 16-byte aligned (NULL allowed when that
 *                size is 0); contents on entry do not matter, and on return
 *                they are unspecified
 *
 * The schedule is stream-K: every workgroup of a persistent grid takes an
 * equal share of the batch's tiles, and a sequence cut by a share boundary
 * is finished by a merge kernel. Up to 64 heads, a wave holds 16 heads and a
 * tile is one block; from 65 heads, a wave holds 32 heads, one workgroup holds
 * them all, and a tile is two blocks. The workspace size depends on the head
 * count and on the compute units of the current device (queried once; 256
 * where none can be queried). Errors, threading, ownership and device-value
 * contracts as for pa_paged_attention_decode. Timed by pa_timing_* like the
 * decode calls.
 */
#define PA_MLA_LATENT_DIM 512
#define PA_MLA_ROPE_DIM   64
#define PA_MLA_MAX_HEADS  128
#define PA_MLA_MAX_WAVES  4096   /* bound on the 16-heads-per-wave persistent grid */
int pa_mla_workspace_bytes(int num_seqs, int num_heads, size_t* bytes);
int pa_mla_decode(void* out, const void* query, const void* latent_cache, int num_seqs, int num_heads,
                  int num_blocks, float scale, const int32_t* block_tables, int max_blocks_per_seq,
                  const int32_t* seq_lens, int block_size, int max_seq_len, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * pa_mla_decode over an fp8 latent cache: the pages' scaled fp8 storage
 * (10100.com retirement article, §4) applied to the latent row, with one
 * per-tensor scale because the row is both key and value. Element e of a
 * token's row stands for e4m3fn(code) * *kv_scale, and the call computes
 * pa_mla_decode's formula over those values.
 *   latent_cache device, uint8 E4M3FN codes [num_blocks][576/16][block_size][16]
 *                (the pages' K layout with one kv head and x = 16), 16-B
 *                aligned.
 *   kv_scale     device fp32 scalar (NULL = 1.0), 4-B aligned.
 * Every other argument, the workspace size (pa_mla_workspace_bytes serves
 * both calls), the kernels by head count and the errors as for
 * pa_mla_decode; the kernels convert the codes to bf16 exactly (in registers
 * up to 64 heads, into the LDS tile from 65) and then run the bf16
 * arithmetic.
 */
int pa_mla_decode_fp8(void* out, const void* query, const void* latent_cache, int num_seqs, int num_heads,
                      int num_blocks, float scale, const int32_t* block_tables, int max_blocks_per_seq,
                      const int32_t* seq_lens, int block_size, int max_seq_len, const float* kv_scale,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Latent-cache append: store the latent rows [c_kv, k_rope] of new tokens in
 * the paged latent cache, the step before pa_mla_decode in every decode
 * iteration (the cache grows one token per step; "vLLM 0.25.0 解读" §1; one
 * compressed row per token, 10100.com retirement article, §2). Token j
 * (0 <= j < tokens_per_seq) of sequence s goes to logical position
 * p = positions[s] + j, i.e. physical block block_tables[s, p / block_size],
 * slot p % block_size (same article, §1): element e of its row is stored at
 * latent_cache[b][e / 8][p % block_size][e % 8].
 *   latent_cache device, bf16 [num_blocks][576/8][block_size][8] as for
 *                pa_mla_decode, 16-B aligned; written only at the slots
 *                named by the positions, the rows copied unchanged.
 *   rows         device, bf16 [num_seqs][tokens_per_seq][576], contiguous,
 *                16-B aligned, not overlapping latent_cache.
 *   num_seqs >= 0 (0 is a no-op); tokens_per_seq >= 1; num_blocks > 0;
 *   max_blocks_per_seq > 0 (table stride); block_size 16 or 32;
 *   num_seqs * tokens_per_seq < 2^31.
 *   block_tables device int32 [num_seqs][max_blocks_per_seq]; positions device
 *   int32 [num_seqs]. A negative position skips the sequence; positions past
 *   max_blocks_per_seq*block_size and table entries outside [0, num_blocks)
 *   are not written.
 * Two tokens naming the same slot leave either one. Asynchronous on `stream`;
 * no allocation; host-side validation and errors as for pa_kv_cache_append;
 * timed with it by pa_timing_read_append.
 */
int pa_mla_cache_append(void* latent_cache, const void* rows, int num_seqs, int tokens_per_seq, int num_blocks,
                        const int32_t* block_tables, int max_blocks_per_seq, const int32_t* positions,
                        int block_size, void* stream);

/*
 * pa_mla_cache_append into an fp8 latent cache (pa_mla_decode_fp8's layout,
 * uint8 [num_blocks][36][block_size][16]): each element of the bf16 rows is stored
 * as the E4M3FN code nearest to value / *kv_scale (float32 quotient, ties to
 * even, magnitude saturated at 448, NaN -> 0x7F, sign kept), the inverse of
 * the decode's dequantisation (10100.com article, §4). kv_scale: device fp32
 * scalar, NULL = 1.0, 4-B aligned. Everything else as for
 * pa_mla_cache_append.
 */
int pa_mla_cache_append_fp8(void* latent_cache, const void* rows, int num_seqs, int tokens_per_seq,
                            int num_blocks, const int32_t* block_tables, int max_blocks_per_seq,
                            const int32_t* positions, int block_size, const float* kv_scale, void* stream);

/* Text describing the last error returned on the calling thread ("" if none). */
const char* pa_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int pa_version(void);

/*
 * Kernel timing. While enabled, each decode call records HIP events on its
 * stream around the partition kernel and around the reduce kernel, and each
 * append call around its kernel (creating events on first use, outside any
 * graph capture). pa_timing_read waits for
 * the recorded events, returns the summed milliseconds and launch counts since
 * the last read, and clears them. Meant for benchmarks; off by default.
 */
int pa_timing_enable(int on);
int pa_timing_read(double* partition_ms, int* partition_launches, double* reduce_ms,
                   int* reduce_launches);
/* The same for the append kernels launched by pa_kv_cache_append and
 * pa_mla_cache_append (one sum over both). */
int pa_timing_read_append(double* append_ms, int* append_launches);

#ifdef __cplusplus
}
#endif

#endif /* PA_DECODE_H */
