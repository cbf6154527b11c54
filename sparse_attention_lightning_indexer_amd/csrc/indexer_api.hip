// C-ABI of the lightning-indexer library (declared in include/indexer.h).
//
// Every entry point validates its arguments on the host before it enqueues
// anything; the checks touch no device memory and make no HIP call, so the
// error paths run without a GPU.  Kernels are enqueued on the caller's
// stream; the library allocates nothing.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "../../include/indexer.h"
#include "internal.h"

namespace {

thread_local char g_last_error[512] = "";

indexer_status fail(indexer_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

indexer_status ok() {
    g_last_error[0] = '\0';
    return INDEXER_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

indexer_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(INDEXER_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int log2_exact(int v) {
    if (v <= 0 || (v & (v - 1))) return -1;
    int s = 0;
    while ((1 << s) < v) ++s;
    return s;
}

size_t round_up(size_t v, size_t m) { return (v + m - 1) / m * m; }

// Checks shared by the prefill and decode score entry points.
indexer_status check_q_w(const void *q, int64_t q_stride_t, int64_t q_stride_h, const float *w,
                         int32_t n_heads, int32_t head_dim) {
    if (!lidx::score_shape_supported(n_heads, head_dim))
        return fail(INDEXER_ENOTSUP,
                    "n_heads=%d head_dim=%d not supported (n_heads in 1..%d, head_dim a multiple of 8 in 8..256)",
                    n_heads, head_dim, lidx::kMaxHeads);
    if (!q) return fail(INDEXER_EINVAL, "q is NULL");
    if (!w) return fail(INDEXER_EINVAL, "w is NULL");
    if (!aligned(q, 16)) return fail(INDEXER_EINVAL, "q must be 16-byte aligned");
    if (!aligned(w, 4)) return fail(INDEXER_EINVAL, "w must be 4-byte aligned");
    if (q_stride_h < head_dim || q_stride_h % 8)
        return fail(INDEXER_EINVAL, "q_stride_h=%lld must be >= head_dim and a multiple of 8", (long long)q_stride_h);
    if (q_stride_t < head_dim || q_stride_t % 8)
        return fail(INDEXER_EINVAL, "q_stride_t=%lld must be >= head_dim and a multiple of 8", (long long)q_stride_t);
    return INDEXER_OK;
}

indexer_status check_prefill(const void *q, int64_t q_stride_t, int64_t q_stride_h, const void *k,
                             int64_t k_stride_s, const float *w, const void *mask, int64_t mask_stride_t,
                             const int32_t *vis_len, int32_t n_tokens, int32_t n_pool, int32_t n_heads,
                             int32_t head_dim) {
    if (n_tokens < 0 || n_pool < 0)
        return fail(INDEXER_EINVAL, "n_tokens=%d n_pool=%d must be >= 0", n_tokens, n_pool);
    indexer_status st = check_q_w(q, q_stride_t, q_stride_h, w, n_heads, head_dim);
    if (st != INDEXER_OK) return st;
    if (!k) return fail(INDEXER_EINVAL, "k is NULL");
    if (!aligned(k, 16)) return fail(INDEXER_EINVAL, "k must be 16-byte aligned");
    if (k_stride_s < head_dim || k_stride_s % 8)
        return fail(INDEXER_EINVAL, "k_stride_s=%lld must be >= head_dim and a multiple of 8", (long long)k_stride_s);
    if (mask) {
        if (!aligned(mask, 2)) return fail(INDEXER_EINVAL, "mask must be 2-byte aligned");
        if (mask_stride_t < n_pool)
            return fail(INDEXER_EINVAL, "mask_stride_t=%lld < n_pool=%d", (long long)mask_stride_t, n_pool);
    }
    if (vis_len && !aligned(vis_len, 4)) return fail(INDEXER_EINVAL, "vis_len must be 4-byte aligned");
    return INDEXER_OK;
}

indexer_status check_decode(const void *q, int64_t q_stride_t, int64_t q_stride_h, const void *k_cache,
                            int32_t block_size, int64_t k_stride_s, const int32_t *block_table,
                            int64_t bt_stride, const int32_t *seq_lens, int32_t n_requests,
                            int32_t query_len, int32_t max_seq_len, const float *w, const void *mask,
                            int64_t mask_stride_t, int32_t n_heads, int32_t head_dim) {
    if (n_requests < 0 || max_seq_len < 0)
        return fail(INDEXER_EINVAL, "n_requests=%d max_seq_len=%d must be >= 0", n_requests, max_seq_len);
    if (query_len < 1) return fail(INDEXER_EINVAL, "query_len=%d must be >= 1", query_len);
    if ((int64_t)n_requests * query_len > INT32_MAX)
        return fail(INDEXER_EINVAL, "n_requests*query_len exceeds the int32 row range");
    indexer_status st = check_q_w(q, q_stride_t, q_stride_h, w, n_heads, head_dim);
    if (st != INDEXER_OK) return st;
    if (!k_cache) return fail(INDEXER_EINVAL, "k_cache is NULL");
    if (!block_table) return fail(INDEXER_EINVAL, "block_table is NULL");
    if (!seq_lens) return fail(INDEXER_EINVAL, "seq_lens is NULL");
    if (!aligned(k_cache, 16)) return fail(INDEXER_EINVAL, "k_cache must be 16-byte aligned");
    if (!aligned(block_table, 4) || !aligned(seq_lens, 4))
        return fail(INDEXER_EINVAL, "block_table and seq_lens must be 4-byte aligned");
    if (block_size < 1) return fail(INDEXER_EINVAL, "block_size=%d must be >= 1", block_size);
    if (k_stride_s < head_dim || k_stride_s % 8)
        return fail(INDEXER_EINVAL, "k_stride_s=%lld must be >= head_dim and a multiple of 8", (long long)k_stride_s);
    const int64_t need_blocks = ((int64_t)max_seq_len + block_size - 1) / block_size;
    if (bt_stride < need_blocks)
        return fail(INDEXER_EINVAL, "bt_stride=%lld < ceil(max_seq_len/block_size)=%lld", (long long)bt_stride,
                    (long long)need_blocks);
    if (mask) {
        if (!aligned(mask, 2)) return fail(INDEXER_EINVAL, "mask must be 2-byte aligned");
        if (mask_stride_t < max_seq_len)
            return fail(INDEXER_EINVAL, "mask_stride_t=%lld < max_seq_len=%d", (long long)mask_stride_t, max_seq_len);
    }
    return INDEXER_OK;
}

indexer_status check_score_out(const float *score, int64_t score_stride_t, int32_t n_cols) {
    if (!score) return fail(INDEXER_EINVAL, "score is NULL");
    if (!aligned(score, 4)) return fail(INDEXER_EINVAL, "score must be 4-byte aligned");
    if (score_stride_t < n_cols)
        return fail(INDEXER_EINVAL, "score_stride_t=%lld < row width %d", (long long)score_stride_t, n_cols);
    return INDEXER_OK;
}

indexer_status check_topk_out(int32_t k_top, const int32_t *idx, const float *val, int64_t out_stride) {
    if (k_top < 1) return fail(INDEXER_EINVAL, "k_top=%d must be >= 1", k_top);
    if (k_top > INDEXER_MAX_K_TOP)
        return fail(INDEXER_ENOTSUP, "k_top=%d exceeds INDEXER_MAX_K_TOP=%d", k_top, INDEXER_MAX_K_TOP);
    if (!idx) return fail(INDEXER_EINVAL, "idx is NULL");
    if (!aligned(idx, 4) || (val && !aligned(val, 4)))
        return fail(INDEXER_EINVAL, "idx and val must be 4-byte aligned");
    if (out_stride < k_top)
        return fail(INDEXER_EINVAL, "out_stride=%lld < k_top=%d", (long long)out_stride, k_top);
    return INDEXER_OK;
}

size_t fused_bytes(int32_t n_rows, int32_t n_cols, int32_t k_top) {
    const size_t row = round_up((size_t)n_cols, 4) * 4;
    return round_up(row * (size_t)n_rows, 256) + round_up(lidx::topk_workspace_bytes(n_rows, n_cols, k_top), 256);
}

lidx::ScoreArgs prefill_args(const void *q, int64_t q_stride_t, int64_t q_stride_h, const void *k,
                             int64_t k_stride_s, const float *w, const void *mask, int64_t mask_stride_t,
                             const int32_t *vis_len, int32_t n_tokens, int32_t n_pool, float *score,
                             int64_t score_stride_t) {
    lidx::ScoreArgs a{};
    a.q = (const _Float16 *)q;
    a.q_st = q_stride_t;
    a.q_sh = q_stride_h;
    a.k = (const _Float16 *)k;
    a.k_ss = k_stride_s;
    a.block_size = 1;
    a.bs_shift = 0;
    a.w = w;
    a.mask = (const _Float16 *)mask;
    a.mask_st = mask_stride_t;
    a.vis_len = vis_len;
    a.score = score;
    a.score_st = score_stride_t;
    a.n_rows = n_tokens;
    a.n_cols = n_pool;
    a.q_per_req = n_tokens;
    a.mask_vec = mask && aligned(mask, 16) && mask_stride_t % 8 == 0;
    a.score_vec = aligned(score, 16) && score_stride_t % 4 == 0;
    return a;
}

lidx::ScoreArgs decode_args(const void *q, int64_t q_stride_t, int64_t q_stride_h, const void *k_cache,
                            int32_t block_size, int64_t k_stride_s, const int32_t *block_table,
                            int64_t bt_stride, const int32_t *seq_lens, int32_t n_requests, int32_t query_len,
                            int32_t max_seq_len, const float *w, const void *mask, int64_t mask_stride_t,
                            float *score, int64_t score_stride_t) {
    lidx::ScoreArgs a{};
    a.q = (const _Float16 *)q;
    a.q_st = q_stride_t;
    a.q_sh = q_stride_h;
    a.k = (const _Float16 *)k_cache;
    a.k_ss = k_stride_s;
    a.block_table = block_table;
    a.bt_stride = bt_stride;
    a.block_size = block_size;
    a.bs_shift = log2_exact(block_size);
    a.seq_lens = seq_lens;
    a.w = w;
    a.mask = (const _Float16 *)mask;
    a.mask_st = mask_stride_t;
    a.score = score;
    a.score_st = score_stride_t;
    a.n_rows = n_requests * query_len;
    a.n_cols = max_seq_len;
    a.q_per_req = query_len;
    a.mask_vec = mask && aligned(mask, 16) && mask_stride_t % 8 == 0;
    a.score_vec = aligned(score, 16) && score_stride_t % 4 == 0;
    return a;
}

// The score kernels hold up to 64 heads (32 at head dimension 256) of one
// row's q in registers.  More heads run as passes over head groups: each
// pass adds its groups' rectified, weighted head sum into the same score
// rows (the b11372 notes' in-place sum over heads, a group at a time), and
// the last pass adds the mask.  A head dimension other than 64, 128 or 256
// runs zero-padded to the next of them.
indexer_status run_score(const lidx::ScoreArgs &base, int n_heads_real, int head_dim, bool paged, int n_requests,
                         hipStream_t stream) {
    const int dpad = lidx::compiled_dim(head_dim);
    const int per_pass = lidx::pass_heads(dpad);
    for (int lo = 0; lo < n_heads_real; lo += per_pass) {
        lidx::ScoreArgs a = base;
        const int cnt = n_heads_real - lo < per_pass ? n_heads_real - lo : per_pass;
        a.q = base.q + (int64_t)lo * base.q_sh;
        a.w = base.w + lo;
        a.n_heads = cnt;  // the kernels run the next compiled head count; the extra heads weigh 0
        a.head_dim = head_dim;
        a.accumulate = lo > 0;
        a.add_mask = lo + cnt >= n_heads_real;
        const int n_heads = lidx::compiled_heads(cnt);
        lidx::ScorePlan p = paged ? lidx::plan_decode(a, n_heads, dpad, n_requests)
                                  : lidx::plan_score(a, n_heads, dpad);
        if ((int64_t)a.n_row_groups * a.n_chunks > INT32_MAX)
            return fail(INDEXER_EINVAL, "problem too large for one launch");
        hipError_t e = paged ? lidx::launch_decode(a, p, n_heads, dpad, stream)
                             : lidx::launch_score(a, p, n_heads, dpad, stream);
        indexer_status st = hip_status(e, "score kernel launch");
        if (st != INDEXER_OK) return st;
    }
    return ok();
}

// Top-k over score rows.  Candidates: s < row_len[t] when given, else the
// visible keys of paged decode rows when seq_lens is given (keys past them
// score -inf by definition, so reading only the visible prefix gives the
// same result), else every column.  The first init_blocks and last
// local_blocks candidates are always selected when selectable.
indexer_status run_topk(const float *score, int64_t score_stride_t, int32_t n_rows, int32_t n_cols,
                        const int32_t *row_len, int32_t k_top, int32_t *idx, float *val, int64_t out_stride,
                        void *workspace, hipStream_t stream, const int32_t *seq_lens = nullptr,
                        int32_t q_per_req = 1, int32_t init_blocks = 0, int32_t local_blocks = 0) {
    lidx::TopkArgs t{};
    t.score = score;
    t.score_st = score_stride_t;
    t.n_rows = n_rows;
    t.n_cols = n_cols;
    t.row_len = row_len;
    t.seq_lens = seq_lens;
    t.q_per_req = q_per_req;
    t.init_blocks = init_blocks;
    t.local_blocks = local_blocks;
    t.k_top = k_top;
    t.idx = idx;
    t.val = val;
    t.out_st = out_stride;
    return hip_status(lidx::launch_topk(t, workspace, stream), "top-k kernel launch");
}

// Score decode into `workspace` (fused_bytes(...) bytes, 256-byte aligned),
// then the top-k of its rows; arguments already checked.
indexer_status fused_decode(const void *q, int64_t q_stride_t, int64_t q_stride_h, const void *k_cache,
                            int32_t block_size, int64_t k_stride_s, const int32_t *block_table, int64_t bt_stride,
                            const int32_t *seq_lens, int32_t n_requests, int32_t query_len, int32_t max_seq_len,
                            const float *w, const void *mask, int64_t mask_stride_t, int32_t n_heads,
                            int32_t head_dim, int32_t k_top, int32_t *idx, float *val, int64_t out_stride,
                            void *workspace, hipStream_t s, int32_t init_blocks = 0, int32_t local_blocks = 0) {
    const int32_t n_rows = n_requests * query_len;
    const int64_t row = (int64_t)round_up((size_t)max_seq_len, 4);
    float *scores = (float *)workspace;
    void *topk_ws = (char *)workspace + round_up((size_t)row * 4 * n_rows, 256);
    if (max_seq_len > 0) {
        lidx::ScoreArgs a = decode_args(q, q_stride_t, q_stride_h, k_cache, block_size, k_stride_s, block_table,
                                        bt_stride, seq_lens, n_requests, query_len, max_seq_len, w, mask,
                                        mask_stride_t, scores, row);
        indexer_status st = run_score(a, n_heads, head_dim, true, n_requests, s);
        if (st != INDEXER_OK) return st;
    }
    // each row's candidates are its visible keys (the rest score -inf)
    return run_topk(scores, row, n_rows, max_seq_len, nullptr, k_top, idx, val, out_stride, topk_ws, s, seq_lens,
                    query_len, init_blocks, local_blocks);
}

indexer_status check_blocks(int32_t init_blocks, int32_t local_blocks) {
    if (init_blocks < 0 || local_blocks < 0)
        return fail(INDEXER_EINVAL, "init_blocks=%d local_blocks=%d must be >= 0", init_blocks, local_blocks);
    return INDEXER_OK;
}

// Scratch of the no-allocation fused decode: a static device array, one copy
// per GPU, held until the process ends.  In host code its name is only a
// stand-in for the device copies, so the device address is looked up once per
// device (with that device current) and kept; only that address is ever
// passed to a kernel.  Every entry the top-k reads is written by the score
// kernel first, so nothing in it needs clearing between calls.
static __device__ __attribute__((aligned(256))) unsigned char scratch[INDEXER_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

indexer_status scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(INDEXER_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(INDEXER_EHIP, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(INDEXER_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return INDEXER_OK;
}

}  // namespace

namespace lidx {

int device_cu_count() {
    static std::mutex mu;
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cached[dev] = v;
    }
    return cached[dev];
}

}  // namespace lidx

extern "C" {

int indexer_abi_version(void) { return INDEXER_ABI_VERSION; }

const char *indexer_status_string(int status) {
    switch (status) {
        case INDEXER_OK: return "INDEXER_OK";
        case INDEXER_EINVAL: return "INDEXER_EINVAL: invalid argument";
        case INDEXER_ENOTSUP: return "INDEXER_ENOTSUP: unsupported shape";
        case INDEXER_EWORKSPACE: return "INDEXER_EWORKSPACE: workspace too small";
        case INDEXER_EHIP: return "INDEXER_EHIP: HIP runtime error";
        default: return "unknown indexer status";
    }
}

const char *indexer_last_error(void) { return g_last_error; }

indexer_status indexer_pool_keys(const void *k, int64_t k_stride_s, int32_t n_keys, int32_t head_dim,
                                 int32_t pool_size, void *k_pool, int64_t pool_stride_s, void *stream) {
    if (n_keys < 0) return fail(INDEXER_EINVAL, "n_keys=%d must be >= 0", n_keys);
    if (head_dim < 8 || head_dim > 1024 || head_dim % 8)
        return fail(INDEXER_ENOTSUP, "head_dim=%d not supported (a multiple of 8 in 8..1024)", head_dim);
    if (pool_size < 1 || pool_size > lidx::kMaxPool)
        return fail(pool_size < 1 ? INDEXER_EINVAL : INDEXER_ENOTSUP, "pool_size=%d must be in 1..%d", pool_size,
                    lidx::kMaxPool);
    if (!k || !k_pool) return fail(INDEXER_EINVAL, "k and k_pool must not be NULL");
    if (!aligned(k, 16) || !aligned(k_pool, 16)) return fail(INDEXER_EINVAL, "k and k_pool must be 16-byte aligned");
    if (k_stride_s < head_dim || k_stride_s % 8)
        return fail(INDEXER_EINVAL, "k_stride_s=%lld must be >= head_dim and a multiple of 8", (long long)k_stride_s);
    if (pool_stride_s < head_dim || pool_stride_s % 8)
        return fail(INDEXER_EINVAL, "pool_stride_s=%lld must be >= head_dim and a multiple of 8",
                    (long long)pool_stride_s);
    if (n_keys == 0) return ok();
    return hip_status(lidx::launch_pool((const _Float16 *)k, k_stride_s, n_keys, head_dim, pool_size,
                                        (_Float16 *)k_pool, pool_stride_s, (hipStream_t)stream),
                      "pool kernel launch");
}

size_t indexer_workspace_bytes(int op, int32_t n_rows, int32_t n_cols, int32_t k_top) {
    if (n_rows < 0 || n_cols < 0 || k_top < 0) return (size_t)-1;
    switch (op) {
        case INDEXER_OP_TOPK: return lidx::topk_workspace_bytes(n_rows, n_cols, k_top);
        case INDEXER_OP_FUSED_PREFILL:
        case INDEXER_OP_FUSED_DECODE: return fused_bytes(n_rows, n_cols, k_top);
        case INDEXER_OP_STREAM_PREFILL:
            return k_top > INDEXER_MAX_K_TOP ? (size_t)-1 : lidx::stream_workspace_bytes(n_rows, n_cols, k_top);
        default: return (size_t)-1;
    }
}

indexer_status indexer_score_prefill(const void *q, int64_t q_stride_t, int64_t q_stride_h, const void *k,
                                     int64_t k_stride_s, const float *w, const void *mask, int64_t mask_stride_t,
                                     const int32_t *vis_len, int32_t n_tokens, int32_t n_pool, int32_t n_heads,
                                     int32_t head_dim, float *score, int64_t score_stride_t, void *stream) {
    indexer_status st = check_prefill(q, q_stride_t, q_stride_h, k, k_stride_s, w, mask, mask_stride_t, vis_len,
                                      n_tokens, n_pool, n_heads, head_dim);
    if (st != INDEXER_OK) return st;
    if ((st = check_score_out(score, score_stride_t, n_pool)) != INDEXER_OK) return st;
    if (n_tokens == 0 || n_pool == 0) return ok();
    lidx::ScoreArgs a = prefill_args(q, q_stride_t, q_stride_h, k, k_stride_s, w, mask, mask_stride_t, vis_len,
                                     n_tokens, n_pool, score, score_stride_t);
    return run_score(a, n_heads, head_dim, false, 1, (hipStream_t)stream);
}

indexer_status indexer_score_decode(const void *q, int64_t q_stride_t, int64_t q_stride_h, const void *k_cache,
                                    int32_t block_size, int64_t k_stride_s, const int32_t *block_table,
                                    int64_t bt_stride, const int32_t *seq_lens, int32_t n_requests,
                                    int32_t query_len, int32_t max_seq_len, const float *w, const void *mask,
                                    int64_t mask_stride_t, int32_t n_heads, int32_t head_dim, float *score,
                                    int64_t score_stride_t, void *stream) {
    indexer_status st = check_decode(q, q_stride_t, q_stride_h, k_cache, block_size, k_stride_s, block_table,
                                     bt_stride, seq_lens, n_requests, query_len, max_seq_len, w, mask,
                                     mask_stride_t, n_heads, head_dim);
    if (st != INDEXER_OK) return st;
    if ((st = check_score_out(score, score_stride_t, max_seq_len)) != INDEXER_OK) return st;
    if (n_requests == 0 || max_seq_len == 0) return ok();
    lidx::ScoreArgs a = decode_args(q, q_stride_t, q_stride_h, k_cache, block_size, k_stride_s, block_table,
                                    bt_stride, seq_lens, n_requests, query_len, max_seq_len, w, mask,
                                    mask_stride_t, score, score_stride_t);
    return run_score(a, n_heads, head_dim, true, n_requests, (hipStream_t)stream);
}

indexer_status indexer_topk(const float *score, int64_t score_stride_t, int32_t n_rows, int32_t n_cols,
                            const int32_t *row_len, int32_t k_top, int32_t *idx, float *val, int64_t out_stride,
                            void *workspace, size_t workspace_bytes, void *stream) {
    if (n_rows < 0 || n_cols < 0) return fail(INDEXER_EINVAL, "n_rows=%d n_cols=%d must be >= 0", n_rows, n_cols);
    indexer_status st = check_topk_out(k_top, idx, val, out_stride);
    if (st != INDEXER_OK) return st;
    if (n_rows > 0 && n_cols > 0 && (st = check_score_out(score, score_stride_t, n_cols)) != INDEXER_OK) return st;
    if (row_len && !aligned(row_len, 4)) return fail(INDEXER_EINVAL, "row_len must be 4-byte aligned");
    const size_t need = lidx::topk_workspace_bytes(n_rows, n_cols, k_top);
    if (need && (!workspace || workspace_bytes < need))
        return fail(INDEXER_EWORKSPACE, "top-k needs %zu workspace bytes, got %zu", need, workspace_bytes);
    if (n_rows == 0) return ok();
    return run_topk(score, score_stride_t, n_rows, n_cols, row_len, k_top, idx, val, out_stride, workspace,
                    (hipStream_t)stream);
}

indexer_status indexer_topk_blocks(const float *score, int64_t score_stride_t, int32_t n_rows, int32_t n_cols,
                                   const int32_t *row_len, int32_t init_blocks, int32_t local_blocks, int32_t k_top,
                                   int32_t *idx, float *val, int64_t out_stride, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    if (n_rows < 0 || n_cols < 0) return fail(INDEXER_EINVAL, "n_rows=%d n_cols=%d must be >= 0", n_rows, n_cols);
    indexer_status st = check_blocks(init_blocks, local_blocks);
    if (st != INDEXER_OK) return st;
    if ((st = check_topk_out(k_top, idx, val, out_stride)) != INDEXER_OK) return st;
    if (n_rows > 0 && n_cols > 0 && (st = check_score_out(score, score_stride_t, n_cols)) != INDEXER_OK) return st;
    if (row_len && !aligned(row_len, 4)) return fail(INDEXER_EINVAL, "row_len must be 4-byte aligned");
    const size_t need = lidx::topk_workspace_bytes(n_rows, n_cols, k_top);
    if (need && (!workspace || workspace_bytes < need))
        return fail(INDEXER_EWORKSPACE, "top-k needs %zu workspace bytes, got %zu", need, workspace_bytes);
    if (n_rows == 0) return ok();
    return run_topk(score, score_stride_t, n_rows, n_cols, row_len, k_top, idx, val, out_stride, workspace,
                    (hipStream_t)stream, nullptr, 1, init_blocks, local_blocks);
}

indexer_status indexer_score_topk_fused_decode_blocks(
    const void *q, int64_t q_stride_t, int64_t q_stride_h, const void *k_cache, int32_t block_size,
    int64_t k_stride_s, const int32_t *block_table, int64_t bt_stride, const int32_t *seq_lens, int32_t n_requests,
    int32_t query_len, int32_t max_seq_len, const float *w, const void *mask, int64_t mask_stride_t,
    int32_t n_heads, int32_t head_dim, int32_t init_blocks, int32_t local_blocks, int32_t k_top, int32_t *idx,
    float *val, int64_t out_stride, void *workspace, size_t workspace_bytes, void *stream) {
    indexer_status st = check_decode(q, q_stride_t, q_stride_h, k_cache, block_size, k_stride_s, block_table,
                                     bt_stride, seq_lens, n_requests, query_len, max_seq_len, w, mask,
                                     mask_stride_t, n_heads, head_dim);
    if (st != INDEXER_OK) return st;
    if ((st = check_blocks(init_blocks, local_blocks)) != INDEXER_OK) return st;
    if ((st = check_topk_out(k_top, idx, val, out_stride)) != INDEXER_OK) return st;
    const int32_t n_rows = n_requests * query_len;
    const size_t need = fused_bytes(n_rows, max_seq_len, k_top);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(INDEXER_EWORKSPACE, "fused decode needs %zu bytes of 256-byte aligned workspace, got %zu", need,
                    workspace ? workspace_bytes : 0);
    if (n_rows == 0) return ok();
    return fused_decode(q, q_stride_t, q_stride_h, k_cache, block_size, k_stride_s, block_table, bt_stride,
                        seq_lens, n_requests, query_len, max_seq_len, w, mask, mask_stride_t, n_heads, head_dim,
                        k_top, idx, val, out_stride, workspace, (hipStream_t)stream, init_blocks, local_blocks);
}

indexer_status indexer_score_topk_stream_prefill(const void *q, int64_t q_stride_t, int64_t q_stride_h,
                                                 const void *k, int64_t k_stride_s, const float *w,
                                                 const void *mask, int64_t mask_stride_t, const int32_t *vis_len,
                                                 int32_t n_tokens, int32_t n_pool, int32_t n_heads,
                                                 int32_t head_dim, int32_t k_top, int32_t *idx, float *val,
                                                 int64_t out_stride, void *workspace, size_t workspace_bytes,
                                                 void *stream) {
    indexer_status st = check_prefill(q, q_stride_t, q_stride_h, k, k_stride_s, w, mask, mask_stride_t, vis_len,
                                      n_tokens, n_pool, n_heads, head_dim);
    if (st != INDEXER_OK) return st;
    if ((st = check_topk_out(k_top, idx, val, out_stride)) != INDEXER_OK) return st;
    if (n_heads > lidx::pass_heads(lidx::compiled_dim(head_dim)))
        return fail(INDEXER_ENOTSUP, "streaming score + top-k runs one pass over the heads: n_heads=%d exceeds %d at "
                    "head_dim=%d", n_heads, lidx::pass_heads(lidx::compiled_dim(head_dim)), head_dim);
    const size_t need = lidx::stream_workspace_bytes(n_tokens, n_pool, k_top);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(INDEXER_EWORKSPACE, "streaming prefill needs %zu bytes of 256-byte aligned workspace, got %zu",
                    need, workspace ? workspace_bytes : 0);
    if (n_tokens == 0) return ok();
    hipStream_t s = (hipStream_t)stream;
    lidx::ScoreArgs a = prefill_args(q, q_stride_t, q_stride_h, k, k_stride_s, w, mask, mask_stride_t, vis_len,
                                     n_tokens, n_pool, nullptr, 0);
    const int nc = lidx::stream_chunks(n_pool);
    a.cand = (unsigned long long *)workspace;
    a.cand_count = (int32_t *)((char *)workspace +
                               round_up((size_t)n_tokens * nc * lidx::stream_cap(k_top) * 8, 256));
    a.cand_cap = lidx::stream_cap(k_top);
    a.k_top = k_top;
    a.n_heads = n_heads;
    a.head_dim = head_dim;
    a.accumulate = 0;
    a.add_mask = 1;
    if (n_pool > 0) {
        const int dpad = lidx::compiled_dim(head_dim);
        const int hc = lidx::compiled_heads(n_heads);
        lidx::ScorePlan p = lidx::plan_score_stream(a, hc, dpad);
        if (a.n_chunks > nc) return fail(INDEXER_EINVAL, "internal: %d key chunks for %d lists", a.n_chunks, nc);
        if ((int64_t)a.n_row_groups * a.n_chunks > INT32_MAX)
            return fail(INDEXER_EINVAL, "problem too large for one launch");
        if ((st = hip_status(lidx::launch_score_stream(a, p, hc, dpad, s), "streaming score launch")) != INDEXER_OK)
            return st;
    } else {
        a.n_chunks = 0;  // no candidates: every row is padding
    }
    a.n_rows = n_tokens;
    return hip_status(lidx::launch_stream_merge(a, idx, val, out_stride, s), "streaming merge launch");
}

indexer_status indexer_score_topk_fused_prefill(const void *q, int64_t q_stride_t, int64_t q_stride_h,
                                                const void *k, int64_t k_stride_s, const float *w,
                                                const void *mask, int64_t mask_stride_t, const int32_t *vis_len,
                                                int32_t n_tokens, int32_t n_pool, int32_t n_heads,
                                                int32_t head_dim, int32_t k_top, int32_t *idx, float *val,
                                                int64_t out_stride, void *workspace, size_t workspace_bytes,
                                                void *stream) {
    indexer_status st = check_prefill(q, q_stride_t, q_stride_h, k, k_stride_s, w, mask, mask_stride_t, vis_len,
                                      n_tokens, n_pool, n_heads, head_dim);
    if (st != INDEXER_OK) return st;
    if ((st = check_topk_out(k_top, idx, val, out_stride)) != INDEXER_OK) return st;
    const size_t need = fused_bytes(n_tokens, n_pool, k_top);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(INDEXER_EWORKSPACE, "fused prefill needs %zu bytes of 256-byte aligned workspace, got %zu", need,
                    workspace ? workspace_bytes : 0);
    if (n_tokens == 0) return ok();
    const int64_t row = (int64_t)round_up((size_t)n_pool, 4);
    float *scores = (float *)workspace;
    void *topk_ws = (char *)workspace + round_up((size_t)row * 4 * n_tokens, 256);
    hipStream_t s = (hipStream_t)stream;
    if (n_pool > 0) {
        lidx::ScoreArgs a = prefill_args(q, q_stride_t, q_stride_h, k, k_stride_s, w, mask, mask_stride_t, vis_len,
                                         n_tokens, n_pool, scores, row);
        a.fill_to_vis = 1;  // the top-k below reads s < vis_len[t] only
        if ((st = run_score(a, n_heads, head_dim, false, 1, s)) != INDEXER_OK) return st;
    }
    // keys at or past vis_len[t] are -inf by definition: the top-k reads
    // only each row's visible prefix
    return run_topk(scores, row, n_tokens, n_pool, vis_len, k_top, idx, val, out_stride, topk_ws, s);
}

indexer_status indexer_score_topk_fused_decode(const void *q, int64_t q_stride_t, int64_t q_stride_h,
                                               const void *k_cache, int32_t block_size, int64_t k_stride_s,
                                               const int32_t *block_table, int64_t bt_stride,
                                               const int32_t *seq_lens, int32_t n_requests, int32_t query_len,
                                               int32_t max_seq_len, const float *w, const void *mask,
                                               int64_t mask_stride_t, int32_t n_heads, int32_t head_dim,
                                               int32_t k_top, int32_t *idx, float *val, int64_t out_stride,
                                               void *workspace, size_t workspace_bytes, void *stream) {
    indexer_status st = check_decode(q, q_stride_t, q_stride_h, k_cache, block_size, k_stride_s, block_table,
                                     bt_stride, seq_lens, n_requests, query_len, max_seq_len, w, mask,
                                     mask_stride_t, n_heads, head_dim);
    if (st != INDEXER_OK) return st;
    if ((st = check_topk_out(k_top, idx, val, out_stride)) != INDEXER_OK) return st;
    const int32_t n_rows = n_requests * query_len;
    const size_t need = fused_bytes(n_rows, max_seq_len, k_top);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(INDEXER_EWORKSPACE, "fused decode needs %zu bytes of 256-byte aligned workspace, got %zu", need,
                    workspace ? workspace_bytes : 0);
    if (n_rows == 0) return ok();
    return fused_decode(q, q_stride_t, q_stride_h, k_cache, block_size, k_stride_s, block_table, bt_stride,
                        seq_lens, n_requests, query_len, max_seq_len, w, mask, mask_stride_t, n_heads, head_dim,
                        k_top, idx, val, out_stride, workspace, (hipStream_t)stream);
}

indexer_status indexer_score_topk_fused_decode_noalloc(
    const void *q, int64_t q_stride_t, int64_t q_stride_h, const void *k_cache, int32_t block_size,
    int64_t k_stride_s, const int32_t *block_table, int64_t bt_stride, const int32_t *seq_lens, int32_t n_requests,
    int32_t query_len, int32_t max_seq_len, const float *w, const void *mask, int64_t mask_stride_t,
    int32_t n_heads, int32_t head_dim, int32_t k_top, int32_t *idx, float *val, int64_t out_stride, void *stream) {
    indexer_status st = check_decode(q, q_stride_t, q_stride_h, k_cache, block_size, k_stride_s, block_table,
                                     bt_stride, seq_lens, n_requests, query_len, max_seq_len, w, mask,
                                     mask_stride_t, n_heads, head_dim);
    if (st != INDEXER_OK) return st;
    if ((st = check_topk_out(k_top, idx, val, out_stride)) != INDEXER_OK) return st;
    const int32_t n_rows = n_requests * query_len;
    const size_t need = fused_bytes(n_rows, max_seq_len, k_top);
    if (need > INDEXER_NOALLOC_SCRATCH_BYTES)
        return fail(INDEXER_EWORKSPACE,
                    "no-allocation fused decode needs %zu bytes of scratch for %d rows of %d keys; its static "
                    "scratch holds %zu (INDEXER_NOALLOC_SCRATCH_BYTES)",
                    need, n_rows, max_seq_len, (size_t)INDEXER_NOALLOC_SCRATCH_BYTES);
    if (n_rows == 0) return ok();
    void *ptr = nullptr;
    if ((st = scratch_address(&ptr)) != INDEXER_OK) return st;
    return fused_decode(q, q_stride_t, q_stride_h, k_cache, block_size, k_stride_s, block_table, bt_stride,
                        seq_lens, n_requests, query_len, max_seq_len, w, mask, mask_stride_t, n_heads, head_dim,
                        k_top, idx, val, out_stride, ptr, (hipStream_t)stream);
}

}  // extern "C"
