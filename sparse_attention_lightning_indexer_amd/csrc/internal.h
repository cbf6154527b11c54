// Internal interface between the C-ABI layer (indexer_api.hip) and the
// kernels (score_kernel.hip, topk_kernel.hip).  Not exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lidx {

// Arguments of the score kernel.  One struct serves the contiguous path
// (block_table == nullptr: one "request" whose rows are all n_rows query
// tokens) and the paged path (rows r*q_per_req .. r*q_per_req+q_per_req-1
// belong to request r).  Strides are in elements.
struct ScoreArgs {
    const _Float16 *q;
    int64_t q_st, q_sh;
    const _Float16 *k;          // contiguous keys, or the paged cache base
    int64_t k_ss;               // stride between consecutive key slots
    const int32_t *block_table; // paged only
    int64_t bt_stride;
    int32_t block_size;
    int32_t bs_shift;           // log2(block_size) if a power of two, else -1
    const int32_t *seq_lens;    // paged only
    const float *w;
    int32_t n_heads;            // heads of q and w (of this pass); the kernel's tile may be larger (extra heads weigh 0)
    int32_t head_dim;           // real head dimension (multiple of 8); the kernel's tile may be wider (zero tail)
    int32_t accumulate;         // add this pass's head sum to the score already stored (visible entries)
    int32_t add_mask;           // add the mask's finite values (the last pass only)
    const _Float16 *mask;
    int64_t mask_st;
    const int32_t *vis_len;     // contiguous only (nullable)
    float *score;
    int64_t score_st;
    int32_t n_rows;
    int32_t n_cols;
    int32_t q_per_req;          // rows per request (contiguous: n_rows)
    int32_t groups_per_req;     // row groups (workgroups along rows) per request
    int32_t n_row_groups;       // total row groups
    int32_t chunk;              // keys per workgroup (multiple of the tile)
    int32_t n_chunks;
    int32_t nc;                 // waves side by side along keys (1, 2 or 4)
    int32_t mask_vec;           // mask rows allow 16-byte loads
    int32_t score_vec;          // score rows allow 16-byte stores
    int32_t fill_to_vis;        // -inf fill only below vis_len[t] (the fused top-k reads no further)
    // streaming score + top-k (no score rows): per row and key chunk a list
    // of candidate entries (order key << 32 | ~index) and its length
    unsigned long long *cand;   // [n_rows][n_chunks][cand_cap]
    int32_t *cand_count;        // [n_rows][n_chunks]
    int32_t cand_cap;
    int32_t k_top;
};



struct ScorePlan {
    int rows_per_group;
    int nc, nbw;
    int tile_keys;
    bool split;   // paged decode: one query row, heads split over the row slots
    bool stream;  // paged decode: persistent streaming kernel
    size_t lds_bytes;
    dim3 grid;
};

// Streaming score + top-k: list capacity and chunking (stream_topk.hip).
constexpr int kStreamSlack = 2048;   // list room beyond k_top
constexpr int kStreamCapMax = 4096;  // k_top <= 2048
constexpr int kStreamMaxChunks = 4;
constexpr int kStreamChunkKeys = 32768;
inline int stream_cap(int k_top) { return (k_top + kStreamSlack + 255) / 256 * 256; }
inline int stream_chunks(int n_cols) {
    const int c = (n_cols + kStreamChunkKeys - 1) / kStreamChunkKeys;
    return c < 1 ? 1 : (c > kStreamMaxChunks ? kStreamMaxChunks : c);
}
size_t stream_workspace_bytes(int n_rows, int n_cols, int k_top);
// The streaming score kernel (score_kernel.hip): a.cand, a.cand_count,
// a.cand_cap and a.k_top set; fills the launch fields like plan_score.
ScorePlan plan_score_stream(ScoreArgs &a, int n_heads, int head_dim);
hipError_t launch_score_stream(const ScoreArgs &a, const ScorePlan &p, int n_heads, int head_dim,
                               hipStream_t stream);
// The per-row merge of the candidate lists into the ordered top-k.
hipError_t launch_stream_merge(const ScoreArgs &a, int32_t *idx, float *val, int64_t out_st, hipStream_t stream);

bool score_shape_supported(int n_heads, int head_dim);
// The smallest compiled head count (4, 8, 16, 32, 64) holding n_heads.
int compiled_heads(int n_heads);
// Largest head count and supported head dimensions: head_dim a multiple of 8
// in [8, 256]; n_heads in [1, kMaxHeads].  Kernels are compiled for head
// dimensions 64, 128 and 256 (others run zero-padded to the next) and for up
// to 64 heads per pass (32 at 256); more heads run as several passes that
// accumulate into the same score rows.
constexpr int kMaxHeads = 1024;
// Head dimension padded to a compiled tile width, and the heads one pass of
// a score kernel covers at that width (the q fragments of a pass stay in
// registers: 64 heads at up to 128 dimensions, 32 at 256).
constexpr int compiled_dim(int d) { return d <= 64 ? 64 : (d <= 128 ? 128 : 256); }
constexpr int pass_heads(int dpad) { return dpad <= 128 ? 64 : 32; }
// Contiguous keys (score_kernel.hip).  Fills the launch-geometry fields of
// `a` and returns the plan.
ScorePlan plan_score(ScoreArgs &a, int n_heads, int head_dim);
hipError_t launch_score(const ScoreArgs &a, const ScorePlan &p, int n_heads,
                        int head_dim, hipStream_t stream);
// Paged keys (decode_kernel.hip).
ScorePlan plan_decode(ScoreArgs &a, int n_heads, int head_dim, int n_requests);
hipError_t launch_decode(const ScoreArgs &a, const ScorePlan &p, int n_heads,
                         int head_dim, hipStream_t stream);

struct TopkArgs {
    const float *score;
    int64_t score_st;
    int32_t n_rows;
    int32_t n_cols;
    const int32_t *row_len;     // candidates s < row_len[t] (nullable)
    const int32_t *seq_lens;    // else, paged rows: s < seq_lens[t / q_per_req] - q_per_req + 1 + t % q_per_req
    int32_t q_per_req;
    int32_t init_blocks;        // keys s < init_blocks of a row are always selected (when selectable)
    int32_t local_blocks;       // and so are its last local_blocks candidates
    int32_t k_top;
    int32_t *idx;
    float *val;
    int64_t out_st;
};

size_t topk_workspace_bytes(int n_rows, int n_cols, int k_top);
hipError_t launch_topk(const TopkArgs &a, void *workspace, hipStream_t stream);

// Pooled-key producer (pool_kernel.hip): mean of each window of `pool`
// consecutive keys, f16 out; pooled_count(n_keys, pool) rows.
constexpr int kMaxPool = 8192;  // windows whose f64 sum of f16 values is exact
int pooled_count(int n_keys, int pool);
hipError_t launch_pool(const _Float16 *k, int64_t k_ss, int n_keys, int head_dim, int pool, _Float16 *out,
                       int64_t out_ss, hipStream_t stream);

// Number of compute units of the current device (cached per device).
int device_cu_count();

}  // namespace lidx
