// Per-row top-k of f32 score rows for gfx950 (the selection step of vLLM PR
// #45743's index_topk module: score, then keep the best keys per token).
//
// Order: score descending, equal scores by lower key index; -inf and NaN are
// never selected; -0 ties with +0; short rows are padded with (-1, -inf).
// Every score maps to an order-preserving 32-bit key (0 = not selectable);
// reported values are the keys mapped back (a zero is re-read from the row,
// so that -0 is reported as stored).  Three kernels, by row length:
//  * rows of up to 16384 keys (topk_rows_kernel): one workgroup per row, the
//    keys register-resident.  Fast path: one histogram of up to 4096 bins of
//    the keys' distance from the row's smallest selectable key selects and
//    orders at once (a descending scan gives every bin its
//    output offset; a key's position is its bin's offset plus its rank inside
//    the bin).  Crowded bins take an adaptive 12-bit radix select, an
//    index-ordered compaction and a bucketed or bitonic ordering.
//  * longer rows (topk_long_kernel): a sample of the row gives a bound that
//    somewhat more than k keys should reach, and one streaming pass gathers
//    every key at or above it into LDS; when the sample misjudges the row,
//    up to three passes find the bin of the k-th key and gather from it.
//    The gathered keys are then selected and ordered in LDS.
//  * topk_row_general: the fully general streaming fallback (heavy ties).
#include <atomic>

#include "device_common.h"
#include "indexer.h"
#include "internal.h"
#include "stream_select.h"

#include <math.h>

namespace lidx {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;  // widest digit: 11 bits
constexpr int kDigits = 3;  // bits 31:21, 20:10, 9:0
__device__ __forceinline__ int digit_shift(int p) { return p == 0 ? 21 : (p == 1 ? 10 : 0); }
__device__ __forceinline__ int digit_width(int p) { return p == 2 ? 10 : 11; }

// Order-preserving u32 key of a score: a negative score maps to the two's
// complement of its bit pattern (so -0 lands on the key of +0, 0x80000000),
// the rest keep their bits with the top one set; NaN and -inf map to 0 and
// are never selected.  Selectable keys lie in [0x00800001, 0xff800000]
// (-FLT_MAX .. +inf).
__device__ __forceinline__ uint32_t order_key(float x) {
    const uint32_t b = __builtin_bit_cast(uint32_t, x);
    const uint32_t u = (int)b < 0 ? 0u - b : (b | 0x80000000u);
    return x > -INFINITY ? u : 0u;
}

// Block ranking (the vLLM decode kernel's init_blocks / local_blocks): the
// first init_blocks and the last local_blocks candidates of a row are always
// selected when selectable, ahead of every other key and among themselves by
// index.  They take the one key no score maps to (the largest finite key is
// that of +inf, 0xff800000), so every later step ranks them first and breaks
// their ties by index like any other.
constexpr uint32_t kForcedKey = 0xffffffffu;

// Candidates of row t: s < row_len[t], or the row's visible keys when the
// rows are paged decode rows, or every column.
__device__ __forceinline__ int topk_row_len(const TopkArgs &a, int t) {
    int n = a.n_cols;
    if (a.row_len) {
        n = min(max(a.row_len[t], 0), n);
    } else if (a.seq_lens) {
        const int r = t / a.q_per_req;
        n = min(max(a.seq_lens[r] - a.q_per_req + 1 + (t - r * a.q_per_req), 0), n);
    }
    return n;
}

// The forced keys of a row of n candidates are s < f_lo and s >= f_hi.
__device__ __forceinline__ int forced_lo(const TopkArgs &a, int n) { return min(a.init_blocks, n); }
__device__ __forceinline__ int forced_hi(const TopkArgs &a, int n) { return a.local_blocks > 0 ? max(n - a.local_blocks, 0) : n; }

// FORCED: the kernel instance that ranks blocks; the plain top-k instances
// carry no window test.
template <bool FORCED>
__device__ __forceinline__ uint32_t select_key(float x, int s, int f_lo, int f_hi) {
    const uint32_t u = order_key(x);
    if constexpr (!FORCED) return u;
    return (u != 0u && (s < f_lo || s >= f_hi)) ? kForcedKey : u;
}

// The score a selectable key stands for (order_key inverted).  +0 and -0
// share a key, so a zero is read back from the row to report it as stored;
// so is a forced key's score.
__device__ __forceinline__ float key_value(uint32_t u, const float *row, int s) {
    if (u == 0x80000000u || u == kForcedKey) return row[s];
    return __builtin_bit_cast(float, (u & 0x80000000u) ? (u & 0x7fffffffu) : 0u - u);
}

__device__ __forceinline__ unsigned long long lanes_below(int lane) {
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Over one thread's bins of a descending walk (counts c; `run` = position
// of the first), fills off[] with each bin's start position, finds the bin B
// holding position total_sel - 1 and returns the largest bin taken whole
// (ending at or before total_sel).  The one thread holding B stores (bin,
// keys to take from it, its count) in sc[0..2]; the rest run no branch.
// Bins past the walk have count 0 and change nothing.
template <int MAXPER>
__device__ __forceinline__ int find_boundary_bin(const int (&c)[MAXPER], int run, int total_sel, int nb, int per,
                                                 int tid, uint32_t (&off)[MAXPER], int *sc) {
    int fullmax = 0, bq = -1, rb = 0, cb = 0;
#pragma unroll
    for (int q = 0; q < MAXPER; ++q) {
        off[q] = (uint32_t)run;
        const int end = run + c[q];
        const bool inb = run < total_sel && end >= total_sel;
        bq = inb ? q : bq;
        rb = inb ? run : rb;
        cb = inb ? c[q] : cb;
        fullmax = max(fullmax, !inb && end <= total_sel ? c[q] : 0);
        run = end;
    }
    if (bq >= 0) {
        sc[0] = nb - 1 - (tid * per + bq);
        sc[1] = total_sel - rb;
        sc[2] = cb;
    }
    return fullmax;
}

// Combining one value per wave: lane l < NW takes wave l's value from LDS
// (the identity elsewhere) and DPP moves reduce or scan the first row of 16
// lanes, a handful of instructions where a loop over the NW words costs a
// read and an operation per wave, in every wave.
template <int NW>
__device__ __forceinline__ int waves_sum(const int *p) {
    static_assert(NW <= 16, "one row of lanes");
    const int l = threadIdx.x & 63;
    const int v = row_reduce(l < NW ? p[l] : 0, 0, [](int a, int b) { return a + b; });
    return __builtin_amdgcn_readlane(v, 0);
}
template <int NW>
__device__ __forceinline__ uint32_t waves_max_u32(const int *p) {
    static_assert(NW <= 16, "one row of lanes");
    const int l = threadIdx.x & 63;
    const int v = row_reduce(l < NW ? p[l] : 0, 0, [](int a, int b) { return (int)max((uint32_t)a, (uint32_t)b); });
    return (uint32_t)__builtin_amdgcn_readlane(v, 0);
}
template <int NW>
__device__ __forceinline__ uint32_t waves_min_u32(const int *p) {
    static_assert(NW <= 16, "one row of lanes");
    const int l = threadIdx.x & 63;
    const int v = row_reduce(l < NW ? p[l] : -1, -1, [](int a, int b) { return (int)min((uint32_t)a, (uint32_t)b); });
    return (uint32_t)__builtin_amdgcn_readlane(v, 0);
}
// Exclusive prefix of the NW per-wave values p[0..NW) at this wave, and
// their total.
template <int NW>
__device__ __forceinline__ int waves_excl(const int *p, int &total) {
    static_assert(NW <= 16, "one row of lanes");
    const int l = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int s = row_incl_scan(l < NW ? p[l] : 0);
    total = __builtin_amdgcn_readlane(s, NW - 1);
    return wid > 0 ? __builtin_amdgcn_readlane(s, wid - 1) : 0;
}

// A descending walk over nb bins gives thread tid the ranks per*tid ..
// per*tid + per - 1 (rank r is bin nb - 1 - r; per is 1, 2 or 4).  Those
// bins are adjacent, so they are read or written with one 8- or 16-byte LDS
// access: consecutive lanes then touch consecutive words, where per 4-byte
// accesses 4*per bytes apart would collide on the same banks.
template <int MAXPER>
__device__ __forceinline__ void read_bins_desc(const uint32_t *h, int nb, int per, int tid, int (&c)[MAXPER]) {
#pragma unroll
    for (int q = 0; q < MAXPER; ++q) c[q] = 0;
    if (MAXPER >= 4 && per == 4) {
        const uint4 v = *reinterpret_cast<const uint4 *>(h + nb - 4 * (tid + 1));
        c[0] = (int)v.w;
        c[MAXPER > 1 ? 1 : 0] = (int)v.z;
        c[MAXPER > 2 ? 2 : 0] = (int)v.y;
        c[MAXPER > 3 ? 3 : 0] = (int)v.x;
    } else if (MAXPER >= 2 && per == 2) {
        const uint2 v = *reinterpret_cast<const uint2 *>(h + nb - 2 * (tid + 1));
        c[0] = (int)v.y;
        c[MAXPER > 1 ? 1 : 0] = (int)v.x;
    } else if (tid < nb) {
        c[0] = (int)h[nb - 1 - tid];
    }
}
template <int MAXPER>
__device__ __forceinline__ void write_bins_desc(uint32_t *h, int nb, int per, int tid, const uint32_t (&o)[MAXPER]) {
    if (MAXPER >= 4 && per == 4) {
        *reinterpret_cast<uint4 *>(h + nb - 4 * (tid + 1)) =
            make_uint4(o[MAXPER > 3 ? 3 : 0], o[MAXPER > 2 ? 2 : 0], o[MAXPER > 1 ? 1 : 0], o[0]);
    } else if (MAXPER >= 2 && per == 2) {
        *reinterpret_cast<uint2 *>(h + nb - 2 * (tid + 1)) = make_uint2(o[MAXPER > 1 ? 1 : 0], o[0]);
    } else if (tid < nb) {
        h[nb - 1 - tid] = o[0];
    }
}

// Exclusive scan of one int per thread across the workgroup; also returns the
// total.  `tmp` holds kWaves ints.  Contains two barriers.
__device__ int block_exclusive_scan(int v, int *tmp, int &total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int incl = wave_incl_scan(v);
    if (lane == 63) tmp[wid] = incl;
    __syncthreads();
    const int off = waves_excl<kWaves>(tmp, total);
    __syncthreads();
    return off + incl - v;
}

// General row top-k for one row per workgroup of kThreads: radix select over
// three digits, each pass re-reading the row from memory, then an
// index-ordered compaction and a bitonic sort.  Slow but unconditional: the
// fallback of the long-row kernel below.
template <bool FORCED>
__device__ void topk_row_general(const TopkArgs &a, int k_pad, unsigned char *smem) {
    uint32_t *hist = reinterpret_cast<uint32_t *>(smem);
    unsigned long long *sel = reinterpret_cast<unsigned long long *>(smem + kBins * 4);
    int *tmp = reinterpret_cast<int *>(smem + kBins * 4 + (size_t)k_pad * 8);

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int t = blockIdx.x;
    const float *row = a.score + (int64_t)t * a.score_st;
    const int n = topk_row_len(a, t);
    const int f_lo = forced_lo(a, n), f_hi = forced_hi(a, n);
    const int k = a.k_top;

    auto key_at = [&](int i) -> uint32_t { return select_key<FORCED>(row[i], i, f_lo, f_hi); };

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
        int tg, te;
        const int og = waves_excl<kWaves>(tmp, tg);
        const int oe = waves_excl<kWaves>(tmp + kWaves, te);
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
            if (val_out) val_out[j] = key_value((uint32_t)(sel[j] >> 32), row, s);
        } else {
            idx_out[j] = -1;
            if (val_out) val_out[j] = -INFINITY;
        }
    }
}

// ---------------------------------------------------------------------------
// Long rows (more keys than the register-resident kernel holds): one
// workgroup per row, two per compute unit, never orders the row itself.
// Rows of at least kSampleRowMin keys first take the sampled one-pass
// gather (below); when it misjudges the row, or for shorter rows, the row
// is streamed twice (three times when the first histogram is too coarse):
//  1. count, min/max of the selectable keys and a histogram of their top 12
//     bits, whose descending scan gives the bin B holding the k-th key;
//  2. when B holds more than kLongCand keys, a histogram of the 12 bits just
//     below the common prefix of min and max instead (which spreads the
//     keys over many bins);
//  3. every key of a bin >= B is gathered into LDS (at most k plus the
//     kLongCand keys of B).
// The gathered set is then selected and ordered in LDS: a histogram of up
// to 2048 bins of the keys' distance from the set's smallest key gives every
// bin its output offset and the bin holding the last selected position; keys of higher bins
// go to their bin's range and are placed by their rank inside it, keys of
// that bin are ranked among themselves.  Sets with a bin of more than
// kMaxBucket selected keys, or more than 512 keys in the boundary bin, are
// bitonic-sorted instead; rows whose B holds more than kLongCand keys (or
// whose selectable keys are all equal) use topk_row_general.
// ---------------------------------------------------------------------------

constexpr int kMaxBucket = 64;     // largest bin ordered by ranking inside it
constexpr int kLongCand = 2048;
constexpr int kLongS = 4096;       // gathered-set capacity (a power of two >= k + kLongCand)
static_assert(INDEXER_MAX_K_TOP + kLongCand <= kLongS, "gathered set");
constexpr int kLongCand2 = 512;    // boundary-bin keys ranked directly in the final ordering

// LDS: one 4096-bin histogram (the gathered set's 2048-bin histogram and
// bin cursors reuse it), the gathered set, the ordered output, the boundary
// bin's keys, scalars.  About 68 KB for k = 2048: two rows per compute unit.
size_t long_lds_bytes(int k_pad) {
    return 16384 + 8 * (size_t)kLongS + 8 * (size_t)k_pad + 8 * (size_t)kLongCand2 + 4 * 128;
}

// Calls f(index, value) for every key of the row; 16-byte loads, four per
// thread in flight, when the row is 16-byte aligned.
template <typename F>
__device__ __forceinline__ void stream_row(const float *row, int n, F &&f) {
    const int tid = threadIdx.x;
    if (((uintptr_t)row & 15) == 0) {
        const int n4 = n >> 2;
        const float4 *r4 = reinterpret_cast<const float4 *>(row);
        int i = tid;
        for (; i + 3 * kThreads < n4; i += 4 * kThreads) {
            float4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = r4[i + u * kThreads];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int b = (i + u * kThreads) * 4;
                f(b, v[u].x);
                f(b + 1, v[u].y);
                f(b + 2, v[u].z);
                f(b + 3, v[u].w);
            }
        }
        for (; i < n4; i += kThreads) {
            const float4 v = r4[i];
            f(4 * i, v.x);
            f(4 * i + 1, v.y);
            f(4 * i + 2, v.z);
            f(4 * i + 3, v.w);
        }
        for (int j = 4 * n4 + tid; j < n; j += kThreads) f(j, row[j]);
    } else {
        for (int j = tid; j < n; j += kThreads) f(j, row[j]);
    }
}

// Descending exclusive scan of nb <= 4096 bin counts (each thread owns
// 4096 / kThreads consecutive bins from the top).  Writes every bin's offset
// to start[] (unless it is null) and reports the bin holding position `total_sel - 1` in
// sc[0..2] (bin, keys to take from it, its count) and, in sc[8 + wave], the
// largest bin above it.  Ends with a barrier.
__device__ void scan_bins_desc(const uint32_t *h, uint32_t *start, int nb, int total_sel, int *sc) {
    constexpr int MAXPER = 4096 / kThreads;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int per = nb > kThreads ? nb / kThreads : 1;
    int c[MAXPER];
    read_bins_desc<MAXPER>(h, nb, per, tid, c);
    int local = 0;
#pragma unroll
    for (int q = 0; q < MAXPER; ++q) local += c[q];
    int total;
    int run = block_exclusive_scan(local, sc + 64, total);
    uint32_t off[MAXPER];
    int fullmax = find_boundary_bin<MAXPER>(c, run, total_sel, nb, per, tid, off, sc);
    if (start) write_bins_desc<MAXPER>(start, nb, per, tid, off);
    fullmax = (int)wave_max_u32((uint32_t)fullmax);
    if (lane == 0) sc[8 + wid] = fullmax;
    __syncthreads();
}

// ---------------------------------------------------------------------------
// One pass instead of two for long rows.  A sample of the row (32 blocks of
// 256 consecutive keys spread evenly over it, 8 keys per thread) gives a
// bound tau, the key of about the r-th best sampled entry, with r chosen so
// that about 1.4 k to 1.5 k of the row's keys should reach it.  One pass then
// counts the row's selectable keys and gathers every key >= tau.  When at
// least k and at most the gathered set's capacity arrive, the set holds the
// whole top k (at least k keys are >= tau, so the k-th best is >= tau) and
// the selection goes on from it; otherwise the row takes the passes below.
// The result is the same either way; only the work differs.
// ---------------------------------------------------------------------------
constexpr int kSampleBlocks = 32, kSampleBlock = 256;  // 8192 sampled keys, 8 per thread
constexpr int kSampleRowMin = 65536;                   // rows at least this long are sampled
static_assert(kSampleBlocks * kSampleBlock == 8 * kThreads, "8 sampled keys per thread");

// The bound tau, or 0 when the sample cannot give a useful one (too few
// selectable sampled keys, or a k too large for the gathered set).  Every
// thread must call it and gets the same value.  Rows of n >= kSampleRowMin.
template <bool FORCED>
__device__ uint32_t sample_bound(const float *row, int n, int k, int f_lo, int f_hi, CutLds<kThreads> *L) {
    const int tid = threadIdx.x;
    constexpr int TPB = kSampleBlock / 8;  // threads per sampled block
    const int j = tid / TPB;
    const int i0 = (int)((int64_t)j * (n - kSampleBlock) / (kSampleBlocks - 1)) + (tid % TPB) * 8;
    unsigned long long e[8];
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int i = i0 + q;
        const uint32_t u = select_key<FORCED>(row[i], i, f_lo, f_hi);
        e[q] = u ? stream_entry(u, i) : 0ull;
        cnt += u != 0;
    }
    int total;
    (void)block_excl_scan<kThreads>(cnt, L, &total);
    // sampled ranks [lo, hi] stand for about 1.4 k .. 1.5 k row keys
    constexpr int64_t ns = kSampleBlocks * kSampleBlock;
    int lo = (int)((14LL * k * ns + 10LL * n - 1) / (10LL * n));
    int hi = (int)((15LL * k * ns) / (10LL * n));
    lo = max(lo, 48);
    hi = max(hi, lo + 8);
    if ((int64_t)hi * n > (int64_t)(kLongS * 4 / 5) * ns || total <= lo) return 0u;
    const unsigned long long b = cut_bound<kThreads, 8>([&](int q) { return e[q]; }, lo, hi, L);
    return (uint32_t)(b >> 32);
}

// One pass over the row: every key >= tau (> 0) is appended to S (up to
// kLongS of them; sc[3] counts them all and must be 0 on entry).  A wave claims its slots with one LDS atomic per
// batch of loads; the loop bounds are the same for every thread, so every
// wave runs its appends whole.  An appended key's score is read again
// from the row right away (its line was loaded moments before, so the read
// is served by the cache), so that no score has to be picked out of a
// thread's loads by a runtime index.  Every thread must call it; ends with
// a barrier, after which sc[3] and S are final.
//
// Without forced keys the tests run on the floats: the key map is monotonic
// (NaN and -inf map to 0, -0 ties with +0), and tau is the key of a finite
// or infinite score (at least that of -FLT_MAX), so key(x) >= tau exactly
// when x >= value(tau).
template <bool FORCED>
__device__ void gather_above(const float *row, int n, uint32_t tau, int f_lo, int f_hi, unsigned long long *S,
                             int *sc) {
    const int tid = threadIdx.x, lane = tid & 63;
    const float ftau = __builtin_bit_cast(float, (tau & 0x80000000u) ? (tau & 0x7fffffffu) : 0u - tau);
    // appends the keys of the set bits of `hits` (bit b: index idx_of(b));
    // a lane loops over its own set bits only
    auto append = [&](uint32_t hits, auto &&idx_of) {
        const int h = __popc(hits);
        const int incl = wave_incl_scan(h);
        const int wtot = __builtin_amdgcn_readlane(incl, 63);
        if (wtot == 0) return;
        int base = 0;
        if (lane == 63) base = (int)atomicAdd((uint32_t *)&sc[3], (uint32_t)wtot);
        base = __builtin_amdgcn_readlane(base, 63);
        int pos = base + incl - h;
        while (hits) {
            const int bit = __builtin_ctz(hits);
            hits &= hits - 1u;
            if (pos < kLongS) {
                const int i = idx_of(bit);
                S[pos] = ((unsigned long long)select_key<FORCED>(row[i], i, f_lo, f_hi) << 32) |
                         (uint32_t)(~(uint32_t)i);
            }
            ++pos;
        }
    };
    auto test = [&](int i, float x) -> uint32_t {
        if constexpr (FORCED) {
            return select_key<FORCED>(x, i, f_lo, f_hi) >= tau ? 1u : 0u;
        } else {
            (void)i;
            return x >= ftau ? 1u : 0u;
        }
    };
    int done = 0;  // keys handled by the 16-byte loops
    if (((uintptr_t)row & 15) == 0) {
        const int n4 = n >> 2;
        const float4 *r4 = reinterpret_cast<const float4 *>(row);
        int i0 = 0;
        for (; i0 + 4 * kThreads <= n4; i0 += 4 * kThreads) {  // four 16-byte loads per thread in flight
            const int i = i0 + tid;
            float4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = r4[i + u * kThreads];
            uint32_t hits = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int b = (i + u * kThreads) * 4;
                hits |= test(b, v[u].x) << (4 * u);
                hits |= test(b + 1, v[u].y) << (4 * u + 1);
                hits |= test(b + 2, v[u].z) << (4 * u + 2);
                hits |= test(b + 3, v[u].w) << (4 * u + 3);
            }
            append(hits, [&](int bit) { return (i + (bit >> 2) * kThreads) * 4 + (bit & 3); });
        }
        for (; i0 < n4; i0 += kThreads) {  // the remaining 16-byte chunks, one per thread
            const int ii = i0 + tid;
            float4 w = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            uint32_t hits = 0;
            if (ii < n4) {
                w = r4[ii];
                hits |= test(4 * ii, w.x);
                hits |= test(4 * ii + 1, w.y) << 1;
                hits |= test(4 * ii + 2, w.z) << 2;
                hits |= test(4 * ii + 3, w.w) << 3;
            }
            append(hits, [&](int bit) { return 4 * ii + bit; });
        }
        done = 4 * n4;
    }
    for (int j0 = done; j0 < n; j0 += kThreads) {  // the tail, or a row not 16-byte aligned
        const int jj = j0 + tid;
        float x = -INFINITY;
        uint32_t hits = 0;
        if (jj < n) {
            x = row[jj];
            hits = test(jj, x);
        }
        append(hits, [&](int) { return jj; });
    }
    __syncthreads();
}

template <bool FORCED>
__global__ void __launch_bounds__(kThreads, 8) topk_long_kernel(TopkArgs a, int k_pad) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint32_t *hist = reinterpret_cast<uint32_t *>(smem);
    uint32_t *hcur = hist + 2048;  // the gathered set's bin cursors (its histogram has <= 2048 bins)
    unsigned long long *S = reinterpret_cast<unsigned long long *>(smem + 16384);
    unsigned long long *O = S + kLongS;
    unsigned long long *cand2 = O + k_pad;
    int *sc = reinterpret_cast<int *>(cand2 + kLongCand2);

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int t = blockIdx.x;
    const float *row = a.score + (int64_t)t * a.score_st;
    const int n = topk_row_len(a, t);
    const int f_lo = forced_lo(a, n), f_hi = forced_hi(a, n);
    const int k = a.k_top;
    int32_t *const idx_out = a.idx + (int64_t)t * a.out_st;
    float *const val_out = a.val ? a.val + (int64_t)t * a.out_st : nullptr;
    auto emit = [&](int pos, unsigned long long e) {
        const int s = (int)(~(uint32_t)(e & 0xffffffffull));
        idx_out[pos] = s;
        if (val_out) val_out[pos] = key_value((uint32_t)(e >> 32), row, s);
    };
    auto pack = [](int i, uint32_t u) {
        return ((unsigned long long)u << 32) | (uint32_t)(~(uint32_t)i);
    };

    // ---- 0. the sampled one-pass gather (rows long enough to sample) -------
    int total_sel = 0, m = 0;
    bool gathered = false;
    if (n >= kSampleRowMin) {
        if (tid == 0) sc[3] = 0;  // published by the barriers in sample_bound
        const uint32_t tau = sample_bound<FORCED>(row, n, k, f_lo, f_hi, reinterpret_cast<CutLds<kThreads> *>(smem));
        if (tau != 0u) {
            // at least k keys at or above a selectable bound: the k best of
            // the row are among them (and the row has at least k selectable
            // keys), so the set settles the row
            gather_above<FORCED>(row, n, tau, f_lo, f_hi, S, sc);
            const int got = sc[3];
            if (got >= k && got <= kLongS) {
                gathered = true;
                total_sel = k;
                m = got;
            }
        }
        __syncthreads();  // every thread has read sc before the passes below may reuse it
    }
    if (!gathered) {
        // ---- 1. count, min, max, and a histogram of the keys' top 12 bits ------
        for (int i = tid; i < 4096; i += kThreads) hist[i] = 0u;
        __syncthreads();
        int cnt = 0;
        uint32_t mn = 0xffffffffu, mx = 0u;
        stream_row(row, n, [&](int i, float x) {
            const uint32_t u = select_key<FORCED>(x, i, f_lo, f_hi);
            if (u) {
                ++cnt;
                mn = min(mn, u);
                mx = max(mx, u);
                atomicAdd(&hist[u >> 20], 1u);
            }
        });
        cnt = wave_sum(cnt);
        mn = wave_min_u32(mn);
        mx = wave_max_u32(mx);
        if (lane == 0) {
            sc[8 + wid] = cnt;
            sc[8 + kWaves + wid] = (int)mn;
            sc[8 + 2 * kWaves + wid] = (int)mx;
        }
        if (tid == 0) sc[3] = 0;
        __syncthreads();
        const int nsel = waves_sum<kWaves>(sc + 8);
        mn = waves_min_u32<kWaves>(sc + 8 + kWaves);
        mx = waves_max_u32<kWaves>(sc + 8 + 2 * kWaves);
        const bool all = nsel <= k;
        total_sel = all ? nsel : k;
        for (int j = total_sel + tid; j < k; j += kThreads) {
            idx_out[j] = -1;
            if (val_out) val_out[j] = -INFINITY;
        }
        if (nsel == 0) return;

        // ---- 2. boundary bin: of the top-12-bit histogram when its bin is small
        // enough to gather, else of a second histogram of the 12 bits below the
        // common prefix of the row's largest and smallest keys (the same bins
        // when the row has keys of both signs) ---------------------------------
        int B = -1, shift = 0, nb = 1;
        if (!all) {
            if (mn == mx) {  // every selectable key equal: index order decides
                __syncthreads();
                topk_row_general<FORCED>(a, k_pad, smem);
                return;
            }
            scan_bins_desc(hist, nullptr, 4096, k, sc);
            const int cnt_top = sc[2];
            __syncthreads();  // every thread has read sc[2] before it may change
            if (cnt_top <= kLongCand) {
                B = sc[0];
                shift = 20;
                nb = 4096;
            } else {
                const int pos = 32 - __clz(mn ^ mx);
                const int width = pos < 12 ? pos : 12;
                shift = pos - width;
                nb = 1 << width;
                for (int i = tid; i < 4096; i += kThreads) hist[i] = 0u;
                __syncthreads();
                stream_row(row, n, [&](int i, float x) {
                    const uint32_t u = select_key<FORCED>(x, i, f_lo, f_hi);
                    if (u) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
                });
                __syncthreads();
                scan_bins_desc(hist, nullptr, nb, k, sc);
                B = sc[0];
                const int cnt_b = sc[2];
                if (cnt_b > kLongCand) {
                    __syncthreads();
                    topk_row_general<FORCED>(a, k_pad, smem);
                    return;
                }
            }
        }

        // ---- 3. gather every key of a bin >= B ----------------------------------
        stream_row(row, n, [&](int i, float x) {
            const uint32_t u = select_key<FORCED>(x, i, f_lo, f_hi);
            if (u && (int)((u >> shift) & (nb - 1)) >= B) S[atomicAdd((uint32_t *)&sc[3], 1u)] = pack(i, u);
        });
        __syncthreads();
        m = sc[3];
    }  // steps 1-3

    // ---- 4. select and order the gathered set ------------------------------
    uint32_t smn = 0xffffffffu, smx = 0u;
    for (int q = tid; q < m; q += kThreads) {
        const uint32_t u = (uint32_t)(S[q] >> 32);
        smn = min(smn, u);
        smx = max(smx, u);
    }
    smn = wave_min_u32(smn);
    smx = wave_max_u32(smx);
    if (lane == 0) {
        sc[16 + wid] = (int)smn;
        sc[16 + kWaves + wid] = (int)smx;
    }
    for (int i = tid; i < 4096; i += kThreads) hist[i] = 0u;
    if (tid == 0) sc[4] = 0;
    __syncthreads();
    smn = waves_min_u32<kWaves>(sc + 16);
    smx = waves_max_u32<kWaves>(sc + 16 + kWaves);
    bool sorted_out = false;
    if (smn != smx) {
        // bins of the key's distance from the set's smallest key: order
        // preserving, and spread over up to 2048 bins wherever the set's
        // scores lie (bins of a common bit prefix collapse when the set
        // straddles a power of two whose exponent bits all differ, 2.0
        // say, and its ordering then falls back to the bitonic sort)
        const uint32_t span = smx - smn;
        const int bits = 32 - __clz(span);
        const int shift2 = bits > 11 ? bits - 11 : 0;
        const int nb2 = 1 << (32 - __clz(span >> shift2));  // a power of two above the largest bin, <= 2048
        auto bin2 = [&](unsigned long long e) { return (int)(((uint32_t)(e >> 32) - smn) >> shift2); };
        for (int q = tid; q < m; q += kThreads) atomicAdd(&hist[bin2(S[q])], 1u);
        __syncthreads();
        scan_bins_desc(hist, hcur, nb2, total_sel, sc);
        const int bmax = (int)waves_max_u32<kWaves>(sc + 8);
        const int B2 = sc[0], need2 = sc[1], cnt2 = sc[2];
        if (bmax <= kMaxBucket && cnt2 <= kLongCand2) {
            const int start2 = total_sel - need2;
            for (int q = tid; q < m; q += kThreads) {
                const unsigned long long e = S[q];
                const int d = bin2(e);
                if (d > B2) O[atomicAdd(&hcur[d], 1u)] = e;
                else if (d == B2) cand2[atomicAdd((uint32_t *)&sc[4], 1u)] = e;
            }
            __syncthreads();
            for (int j = tid; j < start2; j += kThreads) {
                const unsigned long long e = O[j];
                const int d = bin2(e);
                const int c = (int)hist[d];
                const int s0 = (int)hcur[d] - c;
                int rank = 0;
                for (int q = 0; q < c; ++q) rank += O[s0 + q] > e;
                emit(s0 + rank, e);
            }
            for (int j = tid; j < cnt2; j += kThreads) {
                const unsigned long long e = cand2[j];
                int rank = 0;
                for (int q = 0; q < cnt2; ++q) rank += cand2[q] > e;
                if (rank < need2) emit(start2 + rank, e);
            }
            sorted_out = true;
        }
    }
    if (!sorted_out) {
        // bitonic sort of the gathered set, descending
        int P2 = 1;
        while (P2 < m) P2 <<= 1;
        for (int i = m + tid; i < P2; i += kThreads) S[i] = 0ull;
        __syncthreads();
        for (int size = 2; size <= P2; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int q = tid; q < (P2 >> 1); q += kThreads) {
                    const int i = 2 * q - (q & (stride - 1));
                    const int l = i + stride;
                    const unsigned long long x = S[i], y = S[l];
                    const bool desc = (i & size) == 0;
                    if (desc ? (x < y) : (x > y)) {
                        S[i] = y;
                        S[l] = x;
                    }
                }
                __syncthreads();
            }
        }
        for (int j = tid; j < total_sel; j += kThreads) emit(j, S[j]);
    }
}

// ---------------------------------------------------------------------------
// Register-resident variant for rows of up to THREADS*E keys.
//
//  * Each thread holds E keys, striped (key t + THREADS*j): coalesced loads,
//    index order (j, thread).
//  * Radix select with adaptive 12-bit digits: the bits shared by the row's
//    largest and smallest selectable keys are skipped; each pass resolves the
//    12 bits just below the prefix found so far and stops as soon as the bin
//    holding the k-th key is taken whole.  Histograms are double buffered and
//    the threshold bin is found by a two-level (wave, lane) search, so a pass
//    costs three barriers.
//  * Compaction keeps index order with one scan over a (j, wave) table.
//  * Ordering: every selected key lies in [threshold prefix, row max], so a
//    12-bit bucket just below their common prefix spreads them out.  After a
//    counting-sort scatter into buckets, each element's final position is
//    its bucket's start plus the number of bucket members that precede it in
//    (key descending, index ascending) order.  Rows whose largest bucket is
//    bigger than kMaxBucket (heavy ties) use a plain bitonic sort instead.
// ---------------------------------------------------------------------------

template <auto Kern>
hipError_t allow_lds(size_t bytes) {
    static std::atomic<int> allowed{65536};  // per kernel instance: the attribute is per kernel
    if ((int)bytes <= allowed.load(std::memory_order_relaxed)) return hipSuccess;
    hipError_t e = hipFuncSetAttribute((const void *)Kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) allowed.store((int)bytes, std::memory_order_relaxed);
    return e;
}


// Block-wide exclusive scan through tmp[0..NW).  TRAIL: end with a barrier,
// so that tmp may be written again at once; without it the caller must pass
// a barrier before the next write to tmp.
template <int THREADS, bool TRAIL = true>
__device__ __forceinline__ int scan_excl(int v, int *tmp, int &total) {
    constexpr int NW = THREADS / 64;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int incl = wave_incl_scan(v);
    if (lane == 63) tmp[wid] = incl;
    __syncthreads();
    const int off = waves_excl<NW>(tmp, total);
    if (TRAIL) __syncthreads();
    return off + incl - v;
}

// Histogram bins of the row kernel: 4096 (12-bit digits) with 1024 threads;
// 2048 (11-bit digits) with 512 threads, so that three workgroups (rows)
// fit in a compute unit's LDS.
constexpr int rows_bits(int threads) { return threads == 512 ? 11 : 12; }
constexpr int rows_bins(int threads) { return 1 << rows_bits(threads); }
// Capacity of the row kernel's tmp[] (keys of the boundary bin; the
// bucketed ordering of the general path): 512 keys with 512 threads, so
// that four rows fit in a compute unit's LDS (the general path then orders
// larger sets with the bitonic sort), else the padded k.
constexpr int rows_tmp_cap(int threads) { return threads == 512 ? 512 : 1 << 30; }

// Finds, over nb bins read in descending order, the bin where the running
// count first reaches `need`.  Returns (bin, need within the bin, bin count)
// through sc[0..2]; ends with a barrier.  Uses sc[4..4+NW).
template <int THREADS>
__device__ void threshold_bin(const uint32_t *h, int nb, int need, int *sc) {
    constexpr int NW = THREADS / 64;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    constexpr int MAXPER = rows_bins(THREADS) / THREADS;
    const int per = nb > THREADS ? nb / THREADS : 1;  // bins per thread
    int c[MAXPER];
    read_bins_desc<MAXPER>(h, nb, per, tid, c);
    int local = 0;
#pragma unroll
    for (int q = 0; q < MAXPER; ++q) local += c[q];
    int wsum = local;
    wsum = wave_sum(wsum);
    if (lane == 0) sc[4 + wid] = wsum;
    __syncthreads();
    // the wave whose bins contain the crossing (the first whose running
    // total reaches need), and the count before it
    const int srun = row_incl_scan(lane < NW ? sc[4 + lane] : 0);
    const unsigned long long hit = __builtin_amdgcn_ballot_w64(lane < NW && srun >= need);
    const int wstar = hit ? (int)__builtin_ctzll(hit) : NW;
    const int before = wstar > 0 && wstar < NW ? __builtin_amdgcn_readlane(srun, wstar - 1) : 0;
    if (wid == wstar) {
        const int incl = wave_incl_scan(local);
        int acc = before + incl - local;
#pragma unroll
        for (int q = 0; q < MAXPER; ++q) {
            if (q < per && acc < need && acc + c[q] >= need) {
                sc[0] = nb - 1 - (tid * per + q);
                sc[1] = need - acc;
                sc[2] = c[q];
            }
            acc += c[q];
        }
    }
    __syncthreads();
}

template <int THREADS, int E, bool FORCED>
__global__ void __launch_bounds__(THREADS, THREADS == 512 ? 8 : 1) topk_rows_kernel(TopkArgs a, int p2) {
    constexpr int NW = THREADS / 64;
    constexpr int BITS = rows_bits(THREADS), NBINS = rows_bins(THREADS);
    constexpr int HB = 4 * NBINS;  // bytes of one histogram
    const int tcap = min(p2, rows_tmp_cap(THREADS));
    // LDS: hist0 | hist1 (HB each) | sel (p2*8) | tmp (tcap*8) | table | scalars
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint32_t *hist0 = reinterpret_cast<uint32_t *>(smem);
    uint32_t *hist1 = reinterpret_cast<uint32_t *>(smem + HB);
    unsigned long long *sel = reinterpret_cast<unsigned long long *>(smem + 2 * HB);
    unsigned long long *tmp = reinterpret_cast<unsigned long long *>(smem + 2 * HB + 8 * (size_t)p2);
    uint32_t *table = reinterpret_cast<uint32_t *>(smem + 2 * HB + 8 * (size_t)(p2 + tcap));
    int *sc = reinterpret_cast<int *>(smem + 2 * HB + 8 * (size_t)(p2 + tcap) + 4 * E * NW);

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int t = blockIdx.x;
    const float *row = a.score + (int64_t)t * a.score_st;
    const int n = topk_row_len(a, t);
    const int f_lo = forced_lo(a, n), f_hi = forced_hi(a, n);
    const int k = a.k_top;

    // every load is issued before the first one is used
    float xv[E];
#pragma unroll
    for (int j = 0; j < E; ++j) {
        const int i = tid + THREADS * j;
        xv[j] = i < n ? row[i] : -INFINITY;
    }
    uint32_t key[E];
#pragma unroll
    for (int j = 0; j < E; ++j) key[j] = select_key<FORCED>(xv[j], tid + THREADS * j, f_lo, f_hi);
    for (int i = tid; i < NBINS; i += THREADS) hist0[i] = 0u;

    // ---- min and max of the selectable keys ----------------------------
    // (key - 1 wraps an unselectable 0 to the top, out of the minimum's way;
    // the count of selectable keys comes from the histogram below, or from
    // a count of its own when every selectable key is the same)
    uint32_t mn1 = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int j = 0; j < E; ++j) {
        mn1 = min(mn1, key[j] - 1u);
        mx = max(mx, key[j]);
    }
    mn1 = wave_min_u32(mn1);
    mx = wave_max_u32(mx);
    if (lane == 0) {
        sc[8 + NW + wid] = (int)mn1;
        sc[8 + 2 * NW + wid] = (int)mx;
    }
    __syncthreads();
    const uint32_t mn = waves_min_u32<NW>(sc + 8 + NW) + 1u;  // 0 when no key is selectable
    mx = waves_max_u32<NW>(sc + 8 + 2 * NW);
    int nsel = 0;  // selectable keys

    int32_t *const idx_out = a.idx + (int64_t)t * a.out_st;
    float *const val_out = a.val ? a.val + (int64_t)t * a.out_st : nullptr;
    auto emit = [&](int pos, unsigned long long e) {
        const int s = (int)(~(uint32_t)(e & 0xffffffffull));
        idx_out[pos] = s;
        if (val_out) val_out[pos] = key_value((uint32_t)(e >> 32), row, s);
    };

    // ---- fast path: one 12-bit histogram serves as both the select and the
    // ordering buckets.  Bins are the keys' distance from the row's smallest
    // selectable key, scaled to at most 4096 (2048) bins: order preserving,
    // and spread over the row's range wherever it lies (bins of a common bit
    // prefix collapse for rows that straddle a power of two whose exponent
    // bits all differ, 2.0 say).  A descending scan gives
    // every bin its output offset and finds the bin B holding the last
    // selected position; keys in higher bins are placed by their rank inside
    // their bin, the keys of B are ranked among themselves and the best of
    // them kept (with every key selectable, all bins are taken whole).
    // Rows with a bin of more than kMaxBucket selected keys, or more than
    // kMaxCand keys in B, take the general path below instead.
    {
        const uint32_t span = mx - mn;
        if (mx != 0u && mx != mn) {
            const int bits = 32 - __clz(span);
            const int shift = bits > BITS ? bits - BITS : 0;
            const int nb = 1 << (32 - __clz(span >> shift));  // a power of two above the largest bin
            auto bin = [&](uint32_t u) { return (int)((u - mn) >> shift); };
#pragma unroll
            for (int j = 0; j < E; ++j)
                if (key[j]) atomicAdd(&hist0[bin(key[j])], 1u);
            __syncthreads();
            // descending exclusive scan of the bin counts
            constexpr int MAXPER = NBINS / THREADS;
            const int per = nb > THREADS ? nb / THREADS : 1;
            int c[MAXPER];
            read_bins_desc<MAXPER>(hist0, nb, per, tid, c);
            int local = 0;
#pragma unroll
            for (int q = 0; q < MAXPER; ++q) local += c[q];
            int total;
            // sc[64..] is next written after the barrier below
            int run = scan_excl<THREADS, false>(local, sc + 64, total);
            nsel = total;  // every selectable key is in one bin
            const bool all0 = nsel <= k;
            const int sel_total = all0 ? nsel : k;
            // output offsets of the bins, B (the bin holding the last
            // selected position) and the largest bin above it, taken whole
            uint32_t off[MAXPER];
            int fullmax = find_boundary_bin<MAXPER>(c, run, sel_total, nb, per, tid, off, sc);
            write_bins_desc<MAXPER>(hist1, nb, per, tid, off);
            fullmax = (int)wave_max_u32((uint32_t)fullmax);
            if (lane == 0) sc[8 + wid] = fullmax;
            if (tid == 0) sc[3] = 0;  // keys gathered from bin B
            __syncthreads();
            const int bmax = (int)waves_max_u32<NW>(sc + 8);
            // every thread has read sc[8..]; B and its counts stay in sc[0..2]
            const int B = all0 ? -1 : sc[0];
            const int need_b = all0 ? 0 : sc[1];
            const int cnt_b = all0 ? 0 : sc[2];
            const int kMaxCand = p2 < 512 ? p2 : 512;
            if (bmax <= kMaxBucket && cnt_b <= kMaxCand) {
                const int start_b = sel_total - need_b;
                // scatter: whole bins into their ranges, B's keys to tmp[].
                // A key is in bin B or above exactly when it is at least the
                // smallest key of bin B, uB (>= mn >= 1, so unselectable 0
                // keys fail the one test); with every key selected uB = mn.
                const uint32_t uB = B < 0 ? mn : mn + ((uint32_t)B << shift);
#pragma unroll
                for (int j = 0; j < E; ++j) {
                    const uint32_t u = key[j];
                    if (u >= uB) {
                        const int d = bin(u);
                        const unsigned long long e =
                            ((unsigned long long)u << 32) | (uint32_t)(~(uint32_t)(tid + THREADS * j));
                        if (d > B) sel[atomicAdd(&hist1[d], 1u)] = e;
                        else tmp[atomicAdd((uint32_t *)&sc[3], 1u)] = e;
                    }
                }
                for (int j = sel_total + tid; j < k; j += THREADS) {
                    idx_out[j] = -1;
                    if (val_out) val_out[j] = -INFINITY;
                }
                __syncthreads();
                // whole bins: position = bin start + rank inside the bin
                for (int j = tid; j < start_b; j += THREADS) {
                    const unsigned long long e = sel[j];
                    const int d = bin((uint32_t)(e >> 32));
                    const int cnt = (int)hist0[d];
                    const int s0 = (int)hist1[d] - cnt;
                    int rank = 0;
                    for (int q = 0; q < cnt; ++q) rank += sel[s0 + q] > e;
                    emit(s0 + rank, e);
                }
                // the partial bin: rank among its keys, keep the best need_b
                for (int j = tid; j < cnt_b; j += THREADS) {
                    const unsigned long long e = tmp[j];
                    int rank = 0;
                    for (int q = 0; q < cnt_b; ++q) rank += tmp[q] > e;
                    if (rank < need_b) emit(start_b + rank, e);
                }
                return;
            }
            // general path: clear what the fast path used
            for (int i = tid; i < NBINS; i += THREADS) hist0[i] = 0u;
            __syncthreads();
        }
    }

    if (mx != 0u && mx == mn) {
        // every selectable key is the same: count them
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < E; ++j) cnt += key[j] != 0u;
        cnt = wave_sum(cnt);
        if (lane == 0) sc[8 + wid] = cnt;
        __syncthreads();
        nsel = waves_sum<NW>(sc + 8);
        __syncthreads();  // every thread has read sc[8..] before it is written again
    }

    // ---- adaptive radix select -----------------------------------------
    const bool all = nsel <= k;
    uint32_t prefix = 0u, pmask = 0u;
    int need = k;
    if (!all) {
        const uint32_t diff = mn ^ mx;
        int pos = diff ? 32 - __clz(diff) : 0;  // bits below the common prefix
        pmask = pos >= 32 ? 0u : ~((1u << pos) - 1u);
        prefix = mx & pmask;
        int pass = 0;
        while (pos > 0) {
            const int width = pos < BITS ? pos : BITS;
            const int shift = pos - width;
            const int nb = 1 << width;
            uint32_t *h = (pass & 1) ? hist1 : hist0;
            uint32_t *hn = (pass & 1) ? hist0 : hist1;
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const uint32_t u = key[j];
                if (u && (u & pmask) == prefix) atomicAdd(&h[(u >> shift) & (nb - 1)], 1u);
            }
            for (int i = tid; i < NBINS; i += THREADS) hn[i] = 0u;  // next pass
            __syncthreads();
            threshold_bin<THREADS>(h, nb, need, sc);
            const uint32_t digit = (uint32_t)sc[0];
            need = sc[1];
            const int cbin = sc[2];
            prefix |= digit << shift;
            pmask |= (uint32_t)(nb - 1) << shift;
            pos = shift;
            ++pass;
            if (cbin == need) break;  // the whole bin is taken
        }
    }
    const int count_gt = all ? nsel : k - need;
    const int take_eq = all ? 0 : need;
    const int total_sel = all ? nsel : k;

    // ---- index-ordered compaction into sel[] ---------------------------
    const unsigned long long below = lanes_below(lane);
    auto is_gt = [&](uint32_t u) { return all ? u != 0u : (u & pmask) > prefix; };
    auto is_eq = [&](uint32_t u) { return !all && u != 0u && (u & pmask) == prefix; };
#pragma unroll
    for (int j = 0; j < E; ++j) {
        const unsigned long long mg = __builtin_amdgcn_ballot_w64(is_gt(key[j]));
        const unsigned long long me = __builtin_amdgcn_ballot_w64(is_eq(key[j]));
        if (lane == 0) table[j * NW + wid] = (uint32_t)__popcll(mg) | ((uint32_t)__popcll(me) << 16);
    }
    __syncthreads();
    if (wid == 0) {
        constexpr int N = E * NW;
        constexpr int PER = (N + 63) / 64;
        uint32_t v[PER];
        uint32_t s = 0;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int e = lane * PER + q;
            v[q] = e < N ? table[e] : 0u;
            s += v[q];
        }
        const uint32_t incl = (uint32_t)wave_incl_scan((int)s);
        uint32_t run = incl - s;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int e = lane * PER + q;
            if (e < N) table[e] = run;
            run += v[q];
        }
    }
    // bucket histogram of the next phase lives in hist0/hist1's free buffer
    uint32_t *bh = hist0;
    uint32_t *bstart = hist1;
    for (int i = tid; i < NBINS; i += THREADS) bh[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < E; ++j) {
        const uint32_t base = table[j * NW + wid];
        const bool gt = is_gt(key[j]), eq = is_eq(key[j]);
        const unsigned long long mg = __builtin_amdgcn_ballot_w64(gt);
        const unsigned long long me = __builtin_amdgcn_ballot_w64(eq);
        const unsigned long long packed =
            ((unsigned long long)key[j] << 32) | (uint32_t)(~(uint32_t)(tid + THREADS * j));
        if (gt) sel[(base & 0xffffu) + __popcll(mg & below)] = packed;
        if (eq) {
            const int r = (int)(base >> 16) + __popcll(me & below);
            if (r < take_eq) sel[count_gt + r] = packed;
        }
    }
    __syncthreads();

    for (int j = total_sel + tid; j < k; j += THREADS) {
        idx_out[j] = -1;
        if (val_out) val_out[j] = -INFINITY;
    }

    // ---- ordering: bucket by the 12 bits below the selection's prefix ---
    const uint32_t lo_key = all ? mn : prefix;  // every selected key is in [lo_key, mx]
    const uint32_t d2 = lo_key ^ mx;
    if (d2 == 0u) {
        // all selected keys equal: index order is the answer
        for (int j = tid; j < total_sel; j += THREADS) emit(j, sel[j]);
        return;
    }
    const int pos2 = 32 - __clz(d2);
    const int bshift = pos2 > BITS ? pos2 - BITS : 0;
    const int bnb = 1 << (pos2 - bshift);
    for (int j = tid; j < total_sel; j += THREADS)
        atomicAdd(&bh[(uint32_t)(sel[j] >> (32 + bshift)) & (bnb - 1)], 1u);
    __syncthreads();
    // descending exclusive scan of bucket counts -> start offsets; max count
    constexpr int MAXPER = NBINS / THREADS;
    const int per = bnb > THREADS ? bnb / THREADS : 1;
    int c4[MAXPER];
    read_bins_desc<MAXPER>(bh, bnb, per, tid, c4);
    int local = 0, cmax = 0;
#pragma unroll
    for (int q = 0; q < MAXPER; ++q) {
        local += c4[q];
        cmax = max(cmax, c4[q]);
    }
    cmax = (int)wave_max_u32((uint32_t)cmax);
    if (lane == 0) sc[8 + wid] = cmax;
    int total;
    int run = scan_excl<THREADS>(local, sc + 64, total);  // its barriers publish sc[8..]
    uint32_t off4[MAXPER];
#pragma unroll
    for (int q = 0; q < MAXPER; ++q) {
        off4[q] = (uint32_t)run;
        run += c4[q];
    }
    write_bins_desc<MAXPER>(bstart, bnb, per, tid, off4);
    const int bmax = (int)waves_max_u32<NW>(sc + 8);

    if (bmax <= kMaxBucket && total_sel <= tcap) {
        // scatter into buckets (order inside a bucket arbitrary), then rank
        for (int i = tid; i < bnb; i += THREADS) bh[i] = 0u;  // reuse as cursors
        __syncthreads();
        for (int j = tid; j < total_sel; j += THREADS) {
            const unsigned long long e = sel[j];
            const uint32_t b = (uint32_t)(e >> (32 + bshift)) & (bnb - 1);
            tmp[bstart[b] + atomicAdd(&bh[b], 1u)] = e;
        }
        __syncthreads();
        for (int j = tid; j < total_sel; j += THREADS) {
            const unsigned long long e = tmp[j];
            const uint32_t b = (uint32_t)(e >> (32 + bshift)) & (bnb - 1);
            const int s0 = (int)bstart[b];
            const int c = (int)bh[b];
            int rank = 0;
            for (int q = 0; q < c; ++q) rank += tmp[s0 + q] > e;
            emit(s0 + rank, e);
        }
        return;
    }

    // ---- heavy ties: bitonic sort of sel[] in LDS, descending ----------
    int P2 = 1;
    while (P2 < total_sel) P2 <<= 1;
    for (int i = total_sel + tid; i < P2; i += THREADS) sel[i] = 0ull;
    __syncthreads();
    for (int size = 2; size <= P2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int q = tid; q < (P2 >> 1); q += THREADS) {
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
    for (int j = tid; j < total_sel; j += THREADS) emit(j, sel[j]);
}

template <int THREADS, int E>
size_t rows_lds_bytes(int p2) {
    return 8 * (size_t)rows_bins(THREADS) + 8 * (size_t)(p2 + min(p2, rows_tmp_cap(THREADS))) + 4 * (size_t)E * (THREADS / 64) + 4 * (64 + THREADS / 64) + 16;
}

template <int THREADS, int E, bool FORCED>
hipError_t launch_rows_f(const TopkArgs &a, int k_pad, hipStream_t stream) {
    auto kern = topk_rows_kernel<THREADS, E, FORCED>;
    const size_t bytes = rows_lds_bytes<THREADS, E>(k_pad);
    hipError_t e = allow_lds<topk_rows_kernel<THREADS, E, FORCED>>(bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(a.n_rows), dim3(THREADS), bytes, stream, a, k_pad);
    return hipGetLastError();
}

bool ranks_blocks(const TopkArgs &a) { return a.init_blocks > 0 || a.local_blocks > 0; }

template <int THREADS, int E>
hipError_t launch_rows(const TopkArgs &a, int k_pad, hipStream_t stream) {
    return ranks_blocks(a) ? launch_rows_f<THREADS, E, true>(a, k_pad, stream)
                           : launch_rows_f<THREADS, E, false>(a, k_pad, stream);
}

template <bool FORCED>
hipError_t launch_long(const TopkArgs &a, int k_pad, hipStream_t stream) {
    const size_t bytes = long_lds_bytes(k_pad);
    hipError_t e = allow_lds<topk_long_kernel<FORCED>>(bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_long_kernel<FORCED>, dim3(a.n_rows), dim3(kThreads), bytes, stream, a, k_pad);
    return hipGetLastError();
}



}  // namespace

size_t topk_workspace_bytes(int, int, int) { return 0; }

hipError_t launch_topk(const TopkArgs &a, void *, hipStream_t stream) {
    if (a.n_rows <= 0 || a.k_top <= 0) return hipSuccess;
    int k_pad = 1;
    while (k_pad < a.k_top) k_pad <<= 1;
    const int n = a.n_cols;
    // many rows: 512-thread workgroups so that four rows share a compute
    // unit; few rows: 1024 threads per row for the shortest latency
    const bool many = a.n_rows >= 2 * device_cu_count();
    if (many && n <= 512 * 16) {
        if (n <= 512 * 2) return launch_rows<512, 2>(a, k_pad, stream);
        if (n <= 512 * 4) return launch_rows<512, 4>(a, k_pad, stream);
        if (n <= 512 * 8) return launch_rows<512, 8>(a, k_pad, stream);
        return launch_rows<512, 16>(a, k_pad, stream);
    }
    if (n <= 1024 * 16) {
        if (n <= 1024) return launch_rows<1024, 1>(a, k_pad, stream);
        if (n <= 2048) return launch_rows<1024, 2>(a, k_pad, stream);
        if (n <= 4096) return launch_rows<1024, 4>(a, k_pad, stream);
        if (n <= 8192) return launch_rows<1024, 8>(a, k_pad, stream);
        return launch_rows<1024, 16>(a, k_pad, stream);
    }
    return ranks_blocks(a) ? launch_long<true>(a, k_pad, stream) : launch_long<false>(a, k_pad, stream);
}

}  // namespace lidx
