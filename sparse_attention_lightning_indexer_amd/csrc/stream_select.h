// Block-wide selection helpers of the streaming score + top-k (gfx950).
//
// A candidate is one 64-bit entry: the score's order-preserving 32-bit key
// (the top-k's map: larger score = larger key, -0 as +0, -inf and NaN never
// selectable) in the high half and the bitwise complement of the key index
// in the low half.  Entries are unique, and a larger entry is a better key:
// score descending, then index ascending -- the top-k's order.
//
// The selection works with one 64-bit bound L: keeping the entries >= L is
// safe for a top-`need` selection as soon as at least `need` entries are >=
// L, since every entry below L is then beaten by `need` others and can never
// be among the best `need`.  cut_bound() finds such an L by a radix search
// from the top (six digits of 11, 11, 11, 11, 11 and 9 bits): at each digit
// it finds the bin holding the need-th best entry and stops as soon as the
// entries at or above that bin number at most `limit`.  With limit = need
// the search runs to the exact need-th best entry, so exactly `need` are kept.
#pragma once

#include "device_common.h"

namespace lidx {

__device__ __forceinline__ uint32_t stream_key(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if (x != x) return 0u;             // NaN: never selected
    if (u == 0xff800000u) return 0u;   // -inf: never selected
    if (u == 0x80000000u) u = 0u;      // -0 ties with +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The score an order key stands for (stream_key inverted; a zero comes back
// as +0).
__device__ __forceinline__ float stream_value(uint32_t u) {
    return __builtin_bit_cast(float, (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

__device__ __forceinline__ unsigned long long stream_entry(uint32_t key, int s) {
    return ((unsigned long long)key << 32) | (uint32_t)(~(uint32_t)s);
}

constexpr int kCutBins = 2048;

// LDS scratch of the block-wide helpers.
template <int THREADS>
struct CutLds {
    uint32_t hist[kCutBins];
    int wsum[THREADS / 64];
    int word[4];
};

// Exclusive prefix sum of v over the workgroup in thread order; *total gets
// the sum.  Every thread must call it.
template <int THREADS>
__device__ __forceinline__ int block_excl_scan(int v, CutLds<THREADS> *L, int *total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int incl = wave_incl_scan(v);
    if (lane == 63) L->wsum[wid] = incl;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < THREADS / 64; ++w) {
        const int x = L->wsum[w];
        off += w < wid ? x : 0;
        tot += x;
    }
    __syncthreads();  // wsum is free again
    *total = tot;
    return off + incl - v;
}

// Digit p of the radix search: its shift and width (bits 63..53, 52..42,
// 41..31, 30..20, 19..9, 8..0).
__device__ __forceinline__ int cut_shift(int p) { return p < 5 ? 53 - 11 * p : 0; }
__device__ __forceinline__ int cut_width(int p) { return p < 5 ? 11 : 9; }

// The bound L described above, over the entries get(j), j < E, of every
// thread (0 = empty slot; a real entry is >= 2^32).  Requires more than
// `need` real entries in all; every thread must call it and gets the same L.
// get() is called once per entry per digit, so the entries may stay in
// memory.
template <int THREADS, int E, typename GET>
__device__ unsigned long long cut_bound(GET &&get, int need, int limit, CutLds<THREADS> *L) {
    constexpr int PER = kCutBins / THREADS;  // bins per thread in the walk
    static_assert(PER >= 1 && PER * THREADS == kCutBins, "bins per thread");
    unsigned long long prefix = 0, pmask = 0;
    int above = 0;  // entries above the current prefix's range
    for (int p = 0; p < 6; ++p) {
        const int shift = cut_shift(p);
        const int nb = 1 << cut_width(p);
        for (int i = threadIdx.x; i < kCutBins; i += THREADS) L->hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const unsigned long long v = get(j);
            if (v != 0ull && (v & pmask) == prefix)
                atomicAdd(&L->hist[(int)((v >> shift) & (unsigned long long)(nb - 1))], 1u);
        }
        __syncthreads();
        // descending walk: thread i owns bins nb-1-i*PER .. nb-1-i*PER-PER+1
        int c[PER];
        int mine = 0;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int b = nb - 1 - (int)threadIdx.x * PER - q;
            c[q] = b >= 0 ? (int)L->hist[b] : 0;
            mine += c[q];
        }
        int total;
        int run = above + block_excl_scan<THREADS>(mine, L, &total);  // entries in higher bins
        if (threadIdx.x == 0) L->word[0] = -1;
        __syncthreads();
        // the thread whose bins hold the need-th best entry records its bin
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            if (run < need && run + c[q] >= need) {
                L->word[0] = nb - 1 - (int)threadIdx.x * PER - q;
                L->word[1] = run;
                L->word[2] = c[q];
            }
            run += c[q];
        }
        __syncthreads();
        const int b = L->word[0];
        const int gt = L->word[1];   // entries in higher bins, and above
        const int cb = L->word[2];   // entries in bin b
        __syncthreads();             // every thread has read the words
        prefix |= (unsigned long long)b << shift;
        pmask |= (unsigned long long)(nb - 1) << shift;
        if (gt + cb <= limit || p == 5) return prefix;  // keep every entry from bin b up
        above = gt;
    }
    return prefix;  // not reached
}

}  // namespace lidx
