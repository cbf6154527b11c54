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
    int32_t n_heads;            // heads of q and w; the kernel's tile may be larger (extra heads weigh 0)
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

bool score_shape_supported(int n_heads, int head_dim);
// The smallest compiled head count (4, 8, 16, 32, 64) holding n_heads.
int compiled_heads(int n_heads);
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
    const int32_t *row_len;
    int32_t k_top;
    int32_t *idx;
    float *val;
    int64_t out_st;
};

size_t topk_workspace_bytes(int n_rows, int n_cols, int k_top);
hipError_t launch_topk(const TopkArgs &a, void *workspace, hipStream_t stream);

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Achievable-peak probes (peak_probe.hip): an LDS-fed f16 MFMA stream and a
// streaming read.  `sink` holds probe_sink_floats() floats.
hipError_t launch_probe_mfma(int iters, float *sink, double *flops, hipStream_t stream);
hipError_t launch_probe_read(const void *buf, size_t bytes, float *sink, hipStream_t stream);
int probe_sink_floats();

}  // namespace lidx
