// Per-row top-k of f32 score rows for gfx950 (the selection step of vLLM PR
// #45743's index_topk module: score, then keep the best keys per token).
//
// Order: score descending, equal scores by lower key index; -inf and NaN are
// never selected; -0 ties with +0; short rows are padded with (-1, -inf).
//
// One workgroup (1024 threads) per row:
//  1. Every score maps to an order-preserving 32-bit key (0 = not
//     selectable).  Rows that fit in LDS are converted once into LDS; longer
//     rows are re-read from global memory on each pass.
//  2. Radix select over three digits (bits 31:21, 20:10, 9:0) with LDS
//     histograms finds the k-th largest key V and how many keys equal to V
//     are needed.
//  3. An index-ordered compaction (wave ballots + a block scan) gathers every
//     key > V and the lowest-index keys == V, so ties resolve to the lower
//     index.
//  4. The selected (key, ~index) pairs are sorted descending by a bitonic
//     network in LDS and written out; values are re-read from the row so
//     that they are reported exactly as stored.
#include "internal.h"

#include <math.h>

namespace lidx {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxK = 2048;
constexpr int kBins = 2048;  // widest digit: 11 bits
constexpr int kDigits = 3;  // bits 31:21, 20:10, 9:0
__device__ __forceinline__ int digit_shift(int p) { return p == 0 ? 21 : (p == 1 ? 10 : 0); }
__device__ __forceinline__ int digit_width(int p) { return p == 2 ? 10 : 11; }

__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if (x != x) return 0u;             // NaN: never selected
    if (u == 0xff800000u) return 0u;   // -inf: never selected
    if (u == 0x80000000u) u = 0u;      // -0 ties with +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long lanes_below(int lane) {
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Exclusive scan of one int per thread across the workgroup; also returns the
// total.  `tmp` holds kWaves ints.  Contains two barriers.
__device__ int block_exclusive_scan(int v, int *tmp, int &total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    if (lane == 63) tmp[wid] = incl;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int x = tmp[w];
        off += w < wid ? x : 0;
        tot += x;
    }
    __syncthreads();
    total = tot;
    return off + incl - v;
}

template <bool ROW_IN_LDS>
__global__ void __launch_bounds__(kThreads) topk_kernel(TopkArgs a, int k_pad) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint32_t *hist = reinterpret_cast<uint32_t *>(smem);
    unsigned long long *sel = reinterpret_cast<unsigned long long *>(smem + kBins * 4);
    int *tmp = reinterpret_cast<int *>(smem + kBins * 4 + (size_t)k_pad * 8);
    uint32_t *keys = reinterpret_cast<uint32_t *>(smem + kBins * 4 + (size_t)k_pad * 8 + 256);

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int t = blockIdx.x;
    const float *row = a.score + (int64_t)t * a.score_st;
    int n = a.n_cols;
    if (a.row_len) n = min(max(a.row_len[t], 0), n);
    const int k = a.k_top;

    if constexpr (ROW_IN_LDS) {
        for (int i = tid; i < n; i += kThreads) keys[i] = order_key(row[i]);
    }
    auto key_at = [&](int i) -> uint32_t {
        if constexpr (ROW_IN_LDS) return keys[i];
        else return order_key(row[i]);
    };

    // ---- radix select: V = k-th largest key, `need` keys == V to take ----
    uint32_t prefix = 0, pmask = 0;
    int need = k;     // still to take at or below the current prefix
    int nsel = 0;     // selectable keys in the row
    bool all = false; // row has <= k selectable keys
    for (int p = 0; p < kDigits; ++p) {
        const int shift = digit_shift(p);
        const int nb = 1 << digit_width(p);
        for (int i = tid; i < nb; i += kThreads) hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kThreads) {
            const uint32_t u = key_at(i);
            if (u != 0u && (u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
        }
        __syncthreads();
        // thread tid owns bins in descending order: rank r = nb-1-bin
        const int per = (nb + kThreads - 1) / kThreads;  // 2 or 1
        int local = 0;
        for (int q = 0; q < per; ++q) {
            const int r = tid * per + q;
            if (r < nb) local += (int)hist[nb - 1 - r];
        }
        int total;
        const int before = block_exclusive_scan(local, tmp, total);
        if (p == 0) {
            nsel = total;
            if (nsel <= k) {
                all = true;
                break;
            }
        }
        // the bin where the count from the top first reaches `need`
        int acc = before;
        for (int q = 0; q < per; ++q) {
            const int r = tid * per + q;
            if (r < nb) {
                const int c = (int)hist[nb - 1 - r];
                if (acc < need && acc + c >= need) {
                    tmp[kWaves] = nb - 1 - r;   // digit
                    tmp[kWaves + 1] = need - acc;
                }
                acc += c;
            }
        }
        __syncthreads();
        const uint32_t digit = (uint32_t)tmp[kWaves];
        need = tmp[kWaves + 1];
        prefix |= digit << shift;
        pmask |= (uint32_t)(nb - 1) << shift;
        __syncthreads();
    }
    const uint32_t V = all ? 0u : prefix;
    const int take_eq = all ? 0 : need;
    const int count_gt = all ? nsel : k - need;
    const int total_sel = all ? nsel : k;

    // ---- index-ordered compaction --------------------------------------
    int gt_base = 0, eq_base = 0;
    const unsigned long long below = lanes_below(lane);
    for (int i0 = 0; i0 < n; i0 += kThreads) {
        const int i = i0 + tid;
        const uint32_t u = i < n ? key_at(i) : 0u;
        const bool gt = u > V;
        const bool eq = take_eq > 0 && u == V;
        const unsigned long long mg = __builtin_amdgcn_ballot_w64(gt);
        const unsigned long long me = __builtin_amdgcn_ballot_w64(eq);
        if (lane == 0) {
            tmp[wid] = __popcll(mg);
            tmp[kWaves + wid] = __popcll(me);
        }
        __syncthreads();
        int og = 0, oe = 0, tg = 0, te = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int xg = tmp[w], xe = tmp[kWaves + w];
            og += w < wid ? xg : 0;
            oe += w < wid ? xe : 0;
            tg += xg;
            te += xe;
        }
        const unsigned long long packed = ((unsigned long long)u << 32) | (uint32_t)(~(uint32_t)i);
        if (gt) sel[gt_base + og + __popcll(mg & below)] = packed;
        if (eq) {
            const int r = eq_base + oe + __popcll(me & below);
            if (r < take_eq) sel[count_gt + r] = packed;
        }
        gt_base += tg;
        eq_base += te;
        __syncthreads();
    }

    // ---- bitonic sort, descending --------------------------------------
    int p2 = 1;
    while (p2 < total_sel) p2 <<= 1;
    for (int i = total_sel + tid; i < p2; i += kThreads) sel[i] = 0ull;
    __syncthreads();
    for (int size = 2; size <= p2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int q = tid; q < (p2 >> 1); q += kThreads) {
                const int i = 2 * q - (q & (stride - 1));
                const int l = i + stride;
                const unsigned long long x = sel[i], y = sel[l];
                const bool desc = (i & size) == 0;
                if (desc ? (x < y) : (x > y)) {
                    sel[i] = y;
                    sel[l] = x;
                }
            }
            __syncthreads();
        }
    }

    // ---- output ---------------------------------------------------------
    int32_t *idx_out = a.idx + (int64_t)t * a.out_st;
    float *val_out = a.val ? a.val + (int64_t)t * a.out_st : nullptr;
    for (int j = tid; j < k; j += kThreads) {
        if (j < total_sel) {
            const int s = (int)(~(uint32_t)(sel[j] & 0xffffffffull));
            idx_out[j] = s;
            if (val_out) val_out[j] = row[s];
        } else {
            idx_out[j] = -1;
            if (val_out) val_out[j] = -INFINITY;
        }
    }
}

size_t lds_bytes(int n_cols, int k_pad, bool row_in_lds) {
    return (size_t)kBins * 4 + (size_t)k_pad * 8 + 256 + (row_in_lds ? (size_t)n_cols * 4 : 0);
}

int max_lds_per_block() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 65536;
    if (cached[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0)
            v = 65536;
        cached[dev] = v;
    }
    return cached[dev];
}

template <typename K>
hipError_t allow_lds(K kern, size_t bytes) {
    static int allowed = 65536;
    if ((int)bytes <= allowed) return hipSuccess;
    hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) allowed = (int)bytes;
    return e;
}

}  // namespace

size_t topk_workspace_bytes(int, int, int) { return 0; }

hipError_t launch_topk(const TopkArgs &a, void *, hipStream_t stream) {
    if (a.n_rows <= 0 || a.k_top <= 0) return hipSuccess;
    int k_pad = 1;
    while (k_pad < a.k_top) k_pad <<= 1;
    const size_t in_lds = lds_bytes(a.n_cols, k_pad, true);
    if ((int)in_lds <= max_lds_per_block()) {
        auto kern = topk_kernel<true>;
        hipError_t e = allow_lds(kern, in_lds);
        if (e == hipSuccess) {
            hipLaunchKernelGGL(kern, dim3(a.n_rows), dim3(kThreads), in_lds, stream, a, k_pad);
            return hipGetLastError();
        }
        (void)hipGetLastError();  // fall through to the streaming variant
    }
    const size_t streamed = lds_bytes(a.n_cols, k_pad, false);
    auto kern = topk_kernel<false>;
    hipError_t e = allow_lds(kern, streamed);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(a.n_rows), dim3(kThreads), streamed, stream, a, k_pad);
    return hipGetLastError();
}

}  // namespace lidx
