/*
 * Lightning-indexer score and top-k for AMD Instinct MI355X (gfx950).
 *
 * For every query row t and pooled key s the library computes
 *
 *     score[t][s] = sum_h  w[h] * max(q[t][h][:] . k[s][:], 0)  +  mask[t][s]
 *
 * (llama.cpp release b11372 notes, "qwen4exp: halve the indexer score
 * memory": each head's product is rectified and summed in place into one
 * [n_pool, n_tokens] score; "qwen4exp: compute the indexer score with the
 * lightning indexer": per-head weights carry any 1/sqrt(head_dim) scale, the
 * keys are shared by all heads and read once, the pool mask is f16), and then
 * selects, per row, the k_top keys with the largest score (vLLM PR #45743,
 * index_topk module).  No per-head score tensor is ever stored.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers owned by the caller.  The library never
 *    allocates, frees or retains them; all work is enqueued asynchronously on
 *    `stream` (a hipStream_t; NULL = the null stream) and the call returns
 *    before the GPU finishes.
 *  - Strides are in ELEMENTS of the pointed-to type.  The last dimension of
 *    q and k (head_dim) is contiguous.
 *  - Types: q, k and mask are IEEE binary16; w and scores are binary32;
 *    indices, lengths and block ids are int32.
 *  - Arguments are checked on the host before anything is enqueued; on any
 *    error nothing is enqueued and a status other than INDEXER_OK is returned
 *    (indexer_last_error() then describes it for the calling thread).  Values
 *    stored in device memory (block ids, lengths) are trusted, not checked.
 *  - Visibility: an entry is invisible when its mask value is -inf or its key
 *    lies past the row's visible length; invisible entries score -inf.
 *    Finite mask values are additive biases, added once after the head sum.
 *  - Top-k order: score descending, equal scores by lower key index first;
 *    -inf and NaN are never selected and -0 ties with +0.  Rows with fewer
 *    than k_top selectable keys are padded with index -1 and value -inf.
 *  - Supported shapes (others return INDEXER_ENOTSUP, as a backend's
 *    supports_op check would): 1 <= n_heads <= 1024; head_dim a multiple of
 *    8 in [8, 256]; 1 <= k_top <= INDEXER_MAX_K_TOP.  Kernels are compiled
 *    for 4, 8, 16, 32 and 64 heads and head dimensions 64, 128 and 256:
 *      - other head counts run as the next compiled one with the last head
 *        tile zero-filled (the b11372 notes' Metal kernel does the same): the
 *        extra heads read a real head's q and weigh exactly zero;
 *      - other head dimensions run zero-padded to the next compiled one (the
 *        padded q and key elements are 0, so every dot product is unchanged);
 *      - more than 64 heads (32 at head dimensions above 128) run as passes
 *        over head groups, each adding its rectified, weighted head sum into
 *        the same score rows in place; the mask is added once, by the last.
 *    No byte past q's or w's n_heads heads or a row's head_dim is read.
 *  - Alignment: q, k (or k_cache) and every q/k row must be 16-byte aligned
 *    (strides multiples of 8 elements); score and w 4-byte aligned.
 *  - Thread safety: every entry point may be called from any host thread;
 *    calls on one stream execute in order, calls on different streams that
 *    write the same buffers race.
 */
#ifndef LIGHTNING_INDEXER_H
#define LIGHTNING_INDEXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define INDEXER_ABI_VERSION 1
#define INDEXER_MAX_K_TOP 2048

typedef enum {
    INDEXER_OK = 0,
    INDEXER_EINVAL = 1,      /* null required pointer, bad size, stride or alignment */
    INDEXER_ENOTSUP = 2,     /* n_heads, head_dim, k_top outside the supported set */
    INDEXER_EWORKSPACE = 3,  /* workspace missing or smaller than required */
    INDEXER_EHIP = 4         /* the HIP runtime rejected a launch */
} indexer_status;

/* Operation codes for indexer_workspace_bytes. */
typedef enum {
    INDEXER_OP_TOPK = 0,
    INDEXER_OP_FUSED_PREFILL = 1,
    INDEXER_OP_FUSED_DECODE = 2,
    INDEXER_OP_STREAM_PREFILL = 3
} indexer_op;

/* ABI version of the loaded library (INDEXER_ABI_VERSION at build time). */
int indexer_abi_version(void);

/* Static, human-readable name of a status code. */
const char *indexer_status_string(int status);

/* Description of the last error returned on the calling host thread
 * ("" if none).  The pointer stays valid until the thread's next call. */
const char *indexer_last_error(void);

/*
 * indexer_score_prefill -- contiguous keys (prefill, chunked prefill).
 *
 * The score of the b11372 notes for n_tokens query rows against n_pool
 * pooled keys stored contiguously.
 *
 *   q        f16 [n_tokens][n_heads][head_dim], strides (q_stride_t, q_stride_h, 1)
 *   k        f16 [n_pool][head_dim], row stride k_stride_s
 *   w        f32 [n_heads] per-head weights (any sign; scale folded in)
 *   mask     f16 [n_tokens][n_pool], row stride mask_stride_t, 0 / bias / -inf;
 *            NULL = no mask (all keys visible, bias 0)
 *   vis_len  i32 [n_tokens]: key s is visible to row t only if s < vis_len[t];
 *            NULL = every s < n_pool.  Optional; lets fully invisible key
 *            ranges be skipped without reading the mask.
 *   score    f32 [n_tokens][n_pool] output, row stride score_stride_t; every
 *            entry is written (invisible entries -inf)
 *
 * n_tokens >= 0, n_pool >= 0 (either 0: nothing is enqueued).
 */
indexer_status indexer_score_prefill(
    const void *q, int64_t q_stride_t, int64_t q_stride_h,
    const void *k, int64_t k_stride_s,
    const float *w,
    const void *mask, int64_t mask_stride_t,
    const int32_t *vis_len,
    int32_t n_tokens, int32_t n_pool, int32_t n_heads, int32_t head_dim,
    float *score, int64_t score_stride_t,
    void *stream);

/*
 * indexer_score_decode -- paged keys, decode and speculative decode.
 *
 * One program per request batches that request's query_len query tokens
 * (vLLM PR #45743: query j of request r is row r*query_len + j; keys are
 * read through the block table; no implicit scale).  Query j sees the keys
 * s < seq_lens[r] - query_len + 1 + j (query_len = 1: every s < seq_len).
 *
 *   q            f16 [n_requests*query_len][n_heads][head_dim], strides
 *                (q_stride_t, q_stride_h, 1)
 *   k_cache      f16 paged keys: logical key s of request r is at
 *                k_cache + ((int64)block_table[r*bt_stride + s/block_size]
 *                           * block_size + s % block_size) * k_stride_s
 *   block_table  i32 [n_requests][bt_stride]; only entries of keys
 *                s < min(seq_lens[r], max_seq_len) are used, but any entry
 *                of the first ceil(max_seq_len / block_size) columns may be
 *                loaded (to warm the cache), so all of them must be readable
 *   seq_lens     i32 [n_requests] keys per request (device memory)
 *   max_seq_len  width of the score rows; keys at or past it are ignored
 *   mask         f16 [n_requests*query_len][max_seq_len] (stride
 *                mask_stride_t) or NULL
 *   score        f32 [n_requests*query_len][max_seq_len] output, row stride
 *                score_stride_t; columns past a row's visible length are -inf
 *
 * Indices everywhere are LOGICAL key positions, never physical slots.
 * bt_stride >= ceil(max_seq_len / block_size) and block_size >= 1.
 */
indexer_status indexer_score_decode(
    const void *q, int64_t q_stride_t, int64_t q_stride_h,
    const void *k_cache, int32_t block_size, int64_t k_stride_s,
    const int32_t *block_table, int64_t bt_stride,
    const int32_t *seq_lens,
    int32_t n_requests, int32_t query_len, int32_t max_seq_len,
    const float *w,
    const void *mask, int64_t mask_stride_t,
    int32_t n_heads, int32_t head_dim,
    float *score, int64_t score_stride_t,
    void *stream);

/*
 * indexer_topk -- per-row top-k of f32 score rows (vLLM PR #45743,
 * index_topk: score, then select the top keys per token).
 *
 *   score     f32 [n_rows][n_cols], row stride score_stride_t
 *   row_len   i32 [n_rows]: only columns s < row_len[t] are candidates;
 *             NULL = all n_cols
 *   idx       i32 [n_rows][k_top] output (row stride out_stride)
 *   val       f32 [n_rows][k_top] output (row stride out_stride), or NULL;
 *             holds score[t][idx] as stored (-inf for padding)
 *   workspace device scratch of at least
 *             indexer_workspace_bytes(INDEXER_OP_TOPK, n_rows, n_cols, k_top)
 *             bytes (may be NULL when that is 0)
 */
indexer_status indexer_topk(
    const float *score, int64_t score_stride_t, int32_t n_rows, int32_t n_cols,
    const int32_t *row_len,
    int32_t k_top, int32_t *idx, float *val, int64_t out_stride,
    void *workspace, size_t workspace_bytes,
    void *stream);

/*
 * indexer_topk_blocks -- indexer_topk with block ranking (vLLM PR #45743,
 * "Key source snippets": the decode index-score kernel takes init_blocks and
 * local_blocks, and "decode only needs block ordering": each pooled key
 * stands for a block of the cache, and the selection is an ordering of
 * blocks).  The pages do not spell the two arguments out; the reading here:
 * of each row's candidates (s < row_len[t], or every column), the first
 * init_blocks and the last local_blocks are always selected, when selectable
 * (a -inf or NaN score is never selected), ahead of every other key and
 * among themselves by key index; the remaining k_top slots go to the other
 * candidates by score descending, ties to the lower index.  If more keys are
 * forced than k_top, the lowest-indexed are kept.  val holds the stored
 * scores of the selected keys.  init_blocks = local_blocks = 0 is
 * indexer_topk.  EINVAL for a negative init_blocks or local_blocks; other
 * arguments and errors as in indexer_topk.
 */
indexer_status indexer_topk_blocks(
    const float *score, int64_t score_stride_t, int32_t n_rows, int32_t n_cols,
    const int32_t *row_len, int32_t init_blocks, int32_t local_blocks,
    int32_t k_top, int32_t *idx, float *val, int64_t out_stride,
    void *workspace, size_t workspace_bytes,
    void *stream);

/*
 * indexer_score_topk_fused_prefill -- indexer_score_prefill followed by
 * indexer_topk, with the score rows kept in the caller's workspace instead of
 * a caller-visible buffer.  Arguments as in the two calls; vis_len (when
 * given) also serves as the top-k's row_len, since keys at or past
 * vis_len[t] score -inf by definition (the result is the same).  workspace
 * must hold indexer_workspace_bytes(INDEXER_OP_FUSED_PREFILL, n_tokens,
 * n_pool, k_top) bytes, 256-byte aligned.
 */
indexer_status indexer_score_topk_fused_prefill(
    const void *q, int64_t q_stride_t, int64_t q_stride_h,
    const void *k, int64_t k_stride_s,
    const float *w,
    const void *mask, int64_t mask_stride_t,
    const int32_t *vis_len,
    int32_t n_tokens, int32_t n_pool, int32_t n_heads, int32_t head_dim,
    int32_t k_top, int32_t *idx, float *val, int64_t out_stride,
    void *workspace, size_t workspace_bytes,
    void *stream);

/*
 * indexer_score_topk_stream_prefill -- the result of
 * indexer_score_topk_fused_prefill (bit for bit: the same scores, selected
 * in the same order) without any [n_tokens][n_pool] score buffer, for long
 * rows.  The b11372 notes cut the indexer's score memory from per-head
 * tensors to one [n_pool, n_tokens] score; this keeps per row only candidate
 * lists: the workgroup scoring a row group against a chunk of keys keeps,
 * per row, the keys whose score can still be among the row's top k_top in
 * that chunk (a bound raised by compacting the list when it fills), and a
 * second kernel merges a row's chunk lists into its ordered top-k.
 * Arguments as in indexer_score_topk_fused_prefill; the workspace
 * (indexer_workspace_bytes(INDEXER_OP_STREAM_PREFILL, n_tokens, n_pool,
 * k_top) bytes, 256-byte aligned) is
 *   n_tokens * min(4, ceil(n_pool / 32768)) * (k_top + 2048, rounded up to
 *   256) * 8 bytes (+ list lengths),
 * about 128 KiB per row at k_top = 2048 however long the rows are.  The
 * heads must fit one pass of the kernels (n_heads <= 64, or <= 32 at a
 * head_dim above 128), else INDEXER_ENOTSUP.  A score of -0 is reported as
 * +0 (the kernels' scores are never -0 for finite inputs).
 */
indexer_status indexer_score_topk_stream_prefill(
    const void *q, int64_t q_stride_t, int64_t q_stride_h,
    const void *k, int64_t k_stride_s,
    const float *w,
    const void *mask, int64_t mask_stride_t,
    const int32_t *vis_len,
    int32_t n_tokens, int32_t n_pool, int32_t n_heads, int32_t head_dim,
    int32_t k_top, int32_t *idx, float *val, int64_t out_stride,
    void *workspace, size_t workspace_bytes,
    void *stream);

/*
 * indexer_score_topk_fused_decode -- indexer_score_decode followed by
 * indexer_topk over its [n_requests*query_len][max_seq_len] rows, scores
 * kept in the workspace (indexer_workspace_bytes(INDEXER_OP_FUSED_DECODE,
 * n_requests*query_len, max_seq_len, k_top) bytes, 256-byte aligned).
 */
indexer_status indexer_score_topk_fused_decode(
    const void *q, int64_t q_stride_t, int64_t q_stride_h,
    const void *k_cache, int32_t block_size, int64_t k_stride_s,
    const int32_t *block_table, int64_t bt_stride,
    const int32_t *seq_lens,
    int32_t n_requests, int32_t query_len, int32_t max_seq_len,
    const float *w,
    const void *mask, int64_t mask_stride_t,
    int32_t n_heads, int32_t head_dim,
    int32_t k_top, int32_t *idx, float *val, int64_t out_stride,
    void *workspace, size_t workspace_bytes,
    void *stream);

/*
 * indexer_score_topk_fused_decode_blocks -- indexer_score_topk_fused_decode
 * with block ranking (the decode index-score kernel of vLLM PR #45743 with its
 * init_blocks and local_blocks arguments): the selection of
 * indexer_topk_blocks over each row's visible keys (query j of request r sees
 * s < seq_lens[r] - query_len + 1 + j), so a row's last local_blocks visible
 * keys and its first init_blocks keys are always selected (when not masked).
 * Same workspace as indexer_score_topk_fused_decode; EINVAL for a negative
 * init_blocks or local_blocks.
 */
indexer_status indexer_score_topk_fused_decode_blocks(
    const void *q, int64_t q_stride_t, int64_t q_stride_h,
    const void *k_cache, int32_t block_size, int64_t k_stride_s,
    const int32_t *block_table, int64_t bt_stride,
    const int32_t *seq_lens,
    int32_t n_requests, int32_t query_len, int32_t max_seq_len,
    const float *w,
    const void *mask, int64_t mask_stride_t,
    int32_t n_heads, int32_t head_dim,
    int32_t init_blocks, int32_t local_blocks,
    int32_t k_top, int32_t *idx, float *val, int64_t out_stride,
    void *workspace, size_t workspace_bytes,
    void *stream);

/*
 * indexer_score_topk_fused_decode_noalloc -- for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): indexer_score_topk_fused_decode with the
 * score rows kept in a static device array of INDEXER_NOALLOC_SCRATCH_BYTES
 * inside the library (one per GPU, held until the process ends) instead of a
 * caller workspace.  The call allocates and frees nothing.  Arguments,
 * results and errors as in indexer_score_topk_fused_decode, except that
 * INDEXER_EWORKSPACE is returned (before anything is enqueued) when the rows
 * need more than that:
 *   indexer_workspace_bytes(INDEXER_OP_FUSED_DECODE, n_requests*query_len,
 *                           max_seq_len, k_top) > INDEXER_NOALLOC_SCRATCH_BYTES
 * (16 MiB: for example 128 rows of 16384 keys, or 512 rows of 8192).  Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (different streams, or different host threads without ordering) race and
 * give undefined results; calls ordered on one stream are safe.  The first
 * call on a device looks up the array's address there (hipGetSymbolAddress,
 * with that device current).
 */
#define INDEXER_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
indexer_status indexer_score_topk_fused_decode_noalloc(
    const void *q, int64_t q_stride_t, int64_t q_stride_h,
    const void *k_cache, int32_t block_size, int64_t k_stride_s,
    const int32_t *block_table, int64_t bt_stride,
    const int32_t *seq_lens,
    int32_t n_requests, int32_t query_len, int32_t max_seq_len,
    const float *w,
    const void *mask, int64_t mask_stride_t,
    int32_t n_heads, int32_t head_dim,
    int32_t k_top, int32_t *idx, float *val, int64_t out_stride,
    void *stream);

/*
 * indexer_pool_keys -- the pooled keys the indexer scores (llama.cpp b11372
 * notes, "qwen4exp: compute the indexer score with the lightning indexer":
 * the lightning indexer runs on the pooled keys).  The pages do not define
 * the pooling; the reading here is mean pooling over consecutive windows:
 *
 *   k_pool[p][i] = mean of k[s][i] over s in [p*pool_size,
 *                  min((p+1)*pool_size, n_keys)),  p < ceil(n_keys / pool_size)
 *
 * (a short last window averages the keys it holds).  The sum is formed
 * exactly (f64), divided once by the window's key count (f64, correctly
 * rounded) and rounded to the nearest f16, ties to even, so the result does
 * not depend on the order of the sum.
 *
 *   k       f16 [n_keys][head_dim], row stride k_stride_s (16-byte aligned)
 *   k_pool  f16 [ceil(n_keys/pool_size)][head_dim] output, row stride
 *           pool_stride_s (16-byte aligned); may not overlap k
 *
 * head_dim a multiple of 8 in [8, 1024] and pool_size in [1, 8192] (above
 * that an f64 sum of f16 values may round), else INDEXER_ENOTSUP (a
 * pool_size below 1 is INDEXER_EINVAL).  n_keys = 0 enqueues nothing.
 */
indexer_status indexer_pool_keys(
    const void *k, int64_t k_stride_s, int32_t n_keys, int32_t head_dim,
    int32_t pool_size, void *k_pool, int64_t pool_stride_s,
    void *stream);

/*
 * Bytes of device workspace an operation needs (0 if none).  For the fused
 * operations n_rows/n_cols are the score rows and columns (n_tokens x n_pool,
 * or n_requests*query_len x max_seq_len).  Returns (size_t)-1 for negative
 * sizes or an unknown op.
 */
size_t indexer_workspace_bytes(int op, int32_t n_rows, int32_t n_cols, int32_t k_top);

#ifdef __cplusplus
}
#endif

#endif /* LIGHTNING_INDEXER_H */
