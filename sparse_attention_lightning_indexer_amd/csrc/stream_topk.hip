// Streaming score + top-k, second step: per row, merge the candidate lists
// the streaming score kernel left for each key chunk into the row's top-k.
//
// The lists of a row hold, for every chunk, every key of the row's top-k in
// that chunk (and usually more), as 64-bit entries (order key << 32 |
// ~index; stream_select.h).  One workgroup per row loads them all into
// registers, finds the exact k_top-th best entry with the radix search, and
// orders the k_top best by a bitonic sort in LDS: score descending, ties to
// the lower index -- the same order, values and padding as the top-k of the
// stored score rows.
#include <math.h>

#include "../../include/indexer.h"
#include "device_common.h"
#include "internal.h"
#include "stream_select.h"

namespace lidx {
namespace {

constexpr int kMergeThreads = 1024;
constexpr int kMergeE = kStreamMaxChunks * kStreamCapMax / kMergeThreads;  // entries per thread

struct MergeLds {
    CutLds<kMergeThreads> cut;
    unsigned long long sorted[INDEXER_MAX_K_TOP];  // a power of two
};

__global__ void __launch_bounds__(kMergeThreads, 1)
    stream_merge_kernel(const unsigned long long *cand, const int32_t *cand_count, int n_chunks, int cap, int k_top,
                        int k_pad, int32_t *idx, float *val, int64_t out_st) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    MergeLds *L = reinterpret_cast<MergeLds *>(smem);
    const int tid = threadIdx.x;
    const int t = blockIdx.x;

    // the row's lists, concatenated: entry g is list c's entry g - start[c]
    int start[kStreamMaxChunks + 1];
    start[0] = 0;
#pragma unroll
    for (int c = 0; c < kStreamMaxChunks; ++c) {
        const int n = c < n_chunks ? min(max(cand_count[(int64_t)t * n_chunks + c], 0), cap) : 0;
        start[c + 1] = start[c] + n;
    }
    const int m = start[kStreamMaxChunks];
    unsigned long long e[kMergeE];
#pragma unroll
    for (int j = 0; j < kMergeE; ++j) {
        const int g = tid + j * kMergeThreads;
        unsigned long long v = 0ull;
        if (g < m) {
            int c = 0;
#pragma unroll
            for (int q = 1; q < kStreamMaxChunks; ++q) c += g >= start[q] ? 1 : 0;
            v = cand[((int64_t)t * n_chunks + c) * cap + (g - start[c])];
        }
        e[j] = v;
    }

    // the k_top best: every entry >= the exact k_top-th best (all when fewer)
    const unsigned long long bnd =
        m > k_top ? cut_bound<kMergeThreads, kMergeE>([&](int j) { return e[j]; }, k_top, k_top, &L->cut) : 1ull;
    int kept = 0;
#pragma unroll
    for (int j = 0; j < kMergeE; ++j) kept += e[j] != 0ull && e[j] >= bnd;
    int total;
    int off = block_excl_scan<kMergeThreads>(kept, &L->cut, &total);
    for (int i = tid; i < k_pad; i += kMergeThreads) L->sorted[i] = 0ull;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMergeE; ++j)
        if (e[j] != 0ull && e[j] >= bnd) L->sorted[off++] = e[j];
    __syncthreads();

    // bitonic sort of k_pad entries, descending (empty slots, 0, go last)
    for (int size = 2; size <= k_pad; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < k_pad / 2; i += kMergeThreads) {
                const int lo = 2 * i - (i & (stride - 1));  // first of the pair
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const unsigned long long x = L->sorted[lo], y = L->sorted[hi];
                if ((x < y) == desc) {
                    L->sorted[lo] = y;
                    L->sorted[hi] = x;
                }
            }
            __syncthreads();
        }
    }

    int32_t *idx_out = idx + (int64_t)t * out_st;
    float *val_out = val ? val + (int64_t)t * out_st : nullptr;
    for (int i = tid; i < k_top; i += kMergeThreads) {
        const unsigned long long v = i < total ? L->sorted[i] : 0ull;
        idx_out[i] = v ? (int)~(uint32_t)(v & 0xffffffffull) : -1;
        if (val_out) val_out[i] = v ? stream_value((uint32_t)(v >> 32)) : -INFINITY;
    }
}

}  // namespace

size_t stream_workspace_bytes(int n_rows, int n_cols, int k_top) {
    const size_t lists = (size_t)n_rows * stream_chunks(n_cols) * stream_cap(k_top) * 8;
    const size_t counts = (size_t)n_rows * stream_chunks(n_cols) * 4;
    return (lists + 255) / 256 * 256 + (counts + 255) / 256 * 256;
}

hipError_t launch_stream_merge(const ScoreArgs &a, int32_t *idx, float *val, int64_t out_st, hipStream_t stream) {
    int k_pad = 2;
    while (k_pad < a.k_top) k_pad <<= 1;
    const size_t bytes = sizeof(CutLds<kMergeThreads>) + (size_t)k_pad * 8;  // under 64 KiB
    hipLaunchKernelGGL(stream_merge_kernel, dim3(a.n_rows), dim3(kMergeThreads), bytes, stream, a.cand, a.cand_count,
                       a.n_chunks, a.cand_cap, a.k_top, k_pad, idx, val, out_st);
    return hipGetLastError();
}

}  // namespace lidx
