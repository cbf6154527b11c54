// Lightning-indexer score kernel for gfx950 (CDNA4).
//
//   score[t][s] = sum_h w[h] * max(q[t][h][:] . k[s][:], 0) + mask[t][s]
//
// (llama.cpp b11372: every head's product is rectified and summed in place
// into one [n_pool, n_tokens] score, keys read once for all heads, f16 pool
// mask; vLLM PR #45743: decode batches all query tokens of a request into
// one matrix product and uses no implicit scale.)
//
// Design
// ------
// The per-key work is a dense contraction: for a group of query rows the
// [rows*heads, d] x [d, keys] product feeds a rectify/weight/head-sum
// epilogue.  It runs on v_mfma_f32_32x32x16_f16 with fp32 accumulation.
//
//  * A workgroup (4 waves) owns a few query rows and a range of keys.  Each
//    wave keeps its rows' q fragments (all heads) in registers for the whole
//    key loop, so q is read once per workgroup.
//  * Key tiles are streamed global -> LDS with gfx950's direct-to-LDS 16-byte
//    loads, double buffered, into an XOR-swizzled layout that makes the
//    per-lane 16-byte fragment reads bank-conflict free.  Every key tile is
//    read from LDS by every wave, i.e. once for all heads and all rows of the
//    workgroup.
//  * M-block row mapping: the 32 rows of one MFMA block are 16/8/4 heads of
//    2/4/8 query rows, arranged so that accumulator register r of a lane
//    always holds the same head.  The head weight is then a wave-uniform
//    (scalar) operand, and the sum over heads stays inside each lane: no
//    cross-lane reduction and no per-head [rows, heads, keys] tensor.
//  * Visibility: the workgroup first bounds its key range by the rows'
//    visible prefixes (vis_len) and,
//    when a mask is given, by its last non -inf entry; key tiles past that
//    bound are filled with -inf without being loaded.  A wave whose entries
//    in a 32-key block are all invisible skips the MFMAs for that block.
//
// This kernel serves contiguous keys (prefill, chunked prefill); paged decode
// has its own latency-oriented kernel (decode_kernel.hip).
#include <float.h>
#include <math.h>

#include <atomic>

#include "device_common.h"
#include "internal.h"
#include "stream_select.h"

namespace lidx {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kStreamE = kStreamCapMax / kThreads;  // list entries per thread in a compaction
constexpr int kMiscBytes = 4 * (2 + 32);           // two bounds, then up to 32 rows' visible lengths

// LDS of the streaming variant, after the key tiles: the selection scratch
// and each row's list length and bound.
struct StreamLds {
    CutLds<kThreads> cut;
    unsigned long long bound[32];
    int cnt[32];
    // "some list may overflow in the next tile", set by tile i in flag[i % 3],
    // read by every wave after the barrier that starts tile i + 1 and cleared
    // after the one that starts tile i + 2: a slot is never written while a
    // wave may still be about to read it, so every wave sees the same value
    int flag[3];
};

// PAD: the general instance -- fewer real heads than H (the extra heads
// weigh 0), a head dimension below D (zero tail), or one pass of several over
// head groups (accumulate into the stored sums; the mask on the last pass).
// Kept separate so that the exact-shape kernel keeps its weights as plain
// scalar loads and carries none of these checks.
//
// STREAM: the scores are not stored.  Each row keeps, for this workgroup's
// key chunk, a list of candidate entries (order key << 32 | ~index): a score
// joins when its entry is at least the row's bound, which starts at the
// smallest selectable entry.  Before a tile that could overflow a list, the
// workgroup compacts it: the bound rises to one that at least k_top of the
// list's entries reach (stream_select.h), and only those are kept.  Every
// key of the row's top-k within the chunk stays, so the chunk lists of a row
// hold its top-k (merged by stream_merge_kernel).
template <int H, int D, int NBW, bool PAD, bool STREAM>
__global__ void __launch_bounds__(kThreads, 2) score_kernel(ScoreArgs a) {
    using G = Geo<H, D>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int tid = threadIdx.x;
    const int wid = tid >> 6;
    const int lane = tid & 63;
    const int nc = a.nc;
    const int tg = wid / nc;       // row group slot of this wave
    const int col = wid - tg * nc; // key column of this wave
    const int NK = 32 * nc * NBW;  // keys per tile
    const int tile_bytes = NK * G::ROWB;
    const int rows_per_wg = (kWaves / nc) * G::TPB;

    // ---- the rows and keys this workgroup owns --------------------------
    const int chunk_id = blockIdx.x % a.n_chunks;
    // Row groups are dispatched last-first: under causal masks the later rows
    // see more keys, so the longest workgroups start earliest.
    const int rg = a.n_row_groups - 1 - (int)(blockIdx.x / a.n_chunks);
    const int req = rg / a.groups_per_req;
    const int sub = rg - req * a.groups_per_req;
    const int req_row0 = req * a.q_per_req;
    const int row_lo = req_row0 + sub * rows_per_wg;
    const int row_hi = min(req_row0 + a.q_per_req, row_lo + rows_per_wg);
    const int key_lo = chunk_id * a.chunk;
    const int key_hi = min(a.n_cols, key_lo + a.chunk);

    auto row_vis = [&](int t) -> int {
        return a.vis_len ? min(max(a.vis_len[t], 0), a.n_cols) : a.n_cols;
    };

    int *misc = reinterpret_cast<int *>(smem + 2 * tile_bytes);
    StreamLds *sl = reinterpret_cast<StreamLds *>(smem + 2 * tile_bytes + kMiscBytes);

    // ---- bound the key range: prefix lengths, then the mask ------------
    if (tid == 0) {
        misc[0] = key_lo;
        misc[1] = key_lo;
    }
    if constexpr (STREAM) {
        if (tid < 32) {
            sl->cnt[tid] = 0;
            sl->bound[tid] = 1ull << 32;  // every selectable entry
        }
        if (tid < 3) sl->flag[tid] = 0;
    }
    __syncthreads();
    if (tid < row_hi - row_lo) atomicMax(&misc[0], min(row_vis(row_lo + tid), key_hi));
    __syncthreads();
    int bound = misc[0];  // no row of this workgroup sees a key >= bound

    if (a.mask != nullptr && bound > key_lo) {
        // the last visible key: scan windows of 2048 keys from the bound
        // down and stop at the first window holding any visible entry (for
        // a causal mask that is the first one)
        const int nrows = row_hi - row_lo;
        const int nch = (bound - key_lo + 7) >> 3;  // 8-key chunks
        constexpr int WCH = 256;                      // chunks per window
        for (int whi = nch; whi > 0; whi -= WCH) {
            const int wlo = whi > WCH ? whi - WCH : 0;
            const int wn = whi - wlo;
            int last = key_lo;  // 1 + the last visible key seen by this thread
            for (int c = tid; c < nrows * wn; c += kThreads) {
                const int r = c / wn;
                const int s = key_lo + (wlo + (c - r * wn)) * 8;
                const int t = row_lo + r;
                const int rv = min(row_vis(t), bound);
                if (s >= rv) continue;
                const _Float16 *mrow = a.mask + (int64_t)t * a.mask_st;
                if (a.mask_vec && s + 8 <= a.n_cols) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(mrow + s);
                    const unsigned int wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 7; e >= 0; --e) {
                        const unsigned int hbits = (wv[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
                        if (s + e < rv && hbits != 0xfc00u) {
                            last = max(last, s + e + 1);
                            break;
                        }
                    }
                } else {
                    for (int e = min(8, rv - s) - 1; e >= 0; --e) {
                        if (!half_is_neg_inf(mrow[s + e])) {
                            last = max(last, s + e + 1);
                            break;
                        }
                    }
                }
            }
            if (last > key_lo) atomicMax(&misc[1], last);
            __syncthreads();
            const bool found = misc[1] > key_lo;
            __syncthreads();  // every thread has read misc[1] before any later update
            if (found) break;
        }
        bound = misc[1];
    }

    const int load_limit = bound;  // keys past it are visible to no row
    const int n_tiles = bound > key_lo ? (bound - key_lo + NK - 1) / NK : 0;

    // ---- q fragments (A operand) for this wave's rows -------------------
    const int m = lane & 31;
    const int kh = lane >> 5;
    const int tok_m = (((m >> 3) / G::G) << 1) + ((m >> 2) & 1);
    const int head_m = ((m >> 3) % G::G) * 4 + (m & 3);
    const int wave_row0 = row_lo + tg * G::TPB;
    half8 qa[G::MBLK][G::KSTEPS];
    {
        const int t = wave_row0 + tok_m;
        const bool ok = t < row_hi && n_tiles > 0;
#pragma unroll
        for (int mb = 0; mb < G::MBLK; ++mb) {
            const _Float16 *src = a.q + (int64_t)t * a.q_st +
                                  (int64_t)(PAD ? real_head(mb * G::HPB + head_m, a.n_heads) : mb * G::HPB + head_m) * a.q_sh +
                                  kh * (D / 2);
#pragma unroll
            for (int kk = 0; kk < G::KSTEPS; ++kk) {
                // elements past the real head dimension are zero (padded tile)
                if (ok && (!PAD || kh * (D / 2) + kk * 8 < a.head_dim)) {
                    qa[mb][kk] = *reinterpret_cast<const half8 *>(src + kk * 8);
                } else {
                    qa[mb][kk] = half8{};
                }
            }
        }
    }

    const_f32 *wc = (const_f32 *)a.w;

    // rows this lane writes, and their visible prefixes
    int out_t[G::SLOTS];
    int out_vis[G::SLOTS];
#pragma unroll
    for (int j = 0; j < G::SLOTS; ++j) {
        out_t[j] = wave_row0 + 2 * j + kh;
        out_vis[j] = out_t[j] < row_hi ? row_vis(out_t[j]) : 0;
    }

    auto key_src = [&](int s) -> const _Float16 * { return a.k + (int64_t)s * a.k_ss; };

    // chunks past the real head dimension come from a zero chunk
    const bool dim_tail = PAD && a.head_dim < D;
    auto issue_tile = [&](int tile, int buf) {
        const int s0 = key_lo + tile * NK;
        unsigned char *base = smem + buf * tile_bytes;
        const int n_iter = (NK * G::CPR) / kThreads;
        for (int it = 0; it < n_iter; ++it) {
            const int c = (it * kWaves + wid) * 64 + lane;
            const int n = c / G::CPR;
            const int lc = (c & (G::CPR - 1)) ^ swz<D>(n);
            const int s = s0 + n;
            const _Float16 *src = s < load_limit ? key_src(s) + lc * 8 : a.k;
            if (dim_tail && lc * 8 >= a.head_dim) src = reinterpret_cast<const _Float16 *>(kZeroChunk);
            __builtin_amdgcn_global_load_lds(
                src, (__attribute__((address_space(3))) void *)(base + (it * kWaves + wid) * 1024),
                16, 0, 0);
        }
    };

    _Float16 mnext[NBW][G::SLOTS];
    auto load_mask = [&](int tile) {
        const int s0 = key_lo + tile * NK;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const int s = s0 + (col * NBW + nb) * 32 + m;
#pragma unroll
            for (int j = 0; j < G::SLOTS; ++j) {
                _Float16 v = (_Float16)0.0f;
                if (a.mask != nullptr && s < out_vis[j]) v = a.mask[(int64_t)out_t[j] * a.mask_st + s];
                mnext[nb][j] = v;
            }
        }
    };

    // streaming: each lane's row lists and bounds
    unsigned long long *lst[G::SLOTS];
    // a row's bound L as a score and an index: entry(x, s) >= L exactly when
    // x > lbf, or x == lbf and s <= lbs (unsigned), for x neither NaN nor
    // -inf (those never join: every comparison below is false for them)
    float lbf[G::SLOTS];
    uint32_t lbs[G::SLOTS];
    const int trigger = a.cand_cap - NK;  // a list longer than this could overflow in one tile
#pragma unroll
    for (int j = 0; j < G::SLOTS; ++j) {
        lst[j] = STREAM ? a.cand + ((int64_t)out_t[j] * a.n_chunks + chunk_id) * a.cand_cap : nullptr;
        lbf[j] = INFINITY;
        lbs[j] = 0u;
    }
    // keep the entries >= a bound that at least k_top of them reach, in place
    auto compact = [&](int r) {
        unsigned long long *list = a.cand + ((int64_t)(row_lo + r) * a.n_chunks + chunk_id) * a.cand_cap;
        const int mlen = sl->cnt[r];
        unsigned long long e[kStreamE];
#pragma unroll
        for (int j = 0; j < kStreamE; ++j) {
            const int i = tid * kStreamE + j;  // a contiguous segment per thread
            e[j] = i < mlen ? __hip_atomic_load(list + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
        }
        const unsigned long long bnd =
            cut_bound<kThreads, kStreamE>([&](int j) { return e[j]; }, a.k_top, a.k_top + kStreamSlack / 8, &sl->cut);
        int kept = 0;
#pragma unroll
        for (int j = 0; j < kStreamE; ++j) kept += e[j] != 0ull && e[j] >= bnd;
        int total;
        int off = block_excl_scan<kThreads>(kept, &sl->cut, &total);  // every segment is read by now
#pragma unroll
        for (int j = 0; j < kStreamE; ++j)
            if (e[j] != 0ull && e[j] >= bnd) list[off++] = e[j];
        if (tid == 0) {
            sl->cnt[r] = total;
            sl->bound[r] = bnd;
        }
    };

    // results of the previous tile, stored after the next tile's loads are
    // issued so that their write latency overlaps the following compute
    float pend[NBW][G::SLOTS];
    int pend_s = -1;
    auto flush = [&]() {
        if (STREAM || pend_s < 0) return;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const int s = pend_s + nb * 32;
            if (s < key_hi) {
#pragma unroll
                for (int j = 0; j < G::SLOTS; ++j)
                    if (out_t[j] < row_hi) {
                        float *dst = a.score + (int64_t)out_t[j] * a.score_st + s;
                        // a later pass over more heads adds to the stored
                        // partial sum (-inf stays -inf)
                        *dst = PAD && a.accumulate ? pend[nb][j] + *dst : pend[nb][j];
                    }
            }
        }
    };

    if (n_tiles > 0) {
        load_mask(0);
        issue_tile(0, 0);
    }
    for (int i = 0; i < n_tiles; ++i) {
        wait_vmem_all();
        __syncthreads();  // tile i is in LDS; every wave is done with tile i-1
        if constexpr (STREAM) {
            // every candidate of tile i-1 is stored and counted; compact the
            // lists that the next tile could overflow
            const int must = i > 0 ? sl->flag[(i - 1) % 3] : 0;
            if (tid == 0 && i > 1) sl->flag[(i - 2) % 3] = 0;
            if (must) {
                for (int r = 0; r < rows_per_wg; ++r)
                    if (sl->cnt[r] > trigger) {  // cnt changes only in compact() here
                        compact(r);
                        __syncthreads();
                    }
            }
#pragma unroll
            for (int j = 0; j < G::SLOTS; ++j) {
                const unsigned long long bnd = out_t[j] < row_hi ? sl->bound[out_t[j] - row_lo] : ~0ull;
                const uint32_t bk = (uint32_t)(bnd >> 32);
                // keys below 0x00800000 (that of -FLT_MAX) stand for no finite
                // score: such a bound admits every finite score and +inf; a
                // row past the group gets a NaN bound that admits nothing
                lbf[j] = bk < 0x00800000u ? -FLT_MAX : stream_value(bk);
                lbs[j] = bk < 0x00800000u ? 0xffffffffu : ~(uint32_t)bnd;
            }
        }
        _Float16 mcur[NBW][G::SLOTS];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
            for (int j = 0; j < G::SLOTS; ++j) mcur[nb][j] = mnext[nb][j];
        if (i + 1 < n_tiles) {
            load_mask(i + 1);
            issue_tile(i + 1, (i + 1) & 1);
        }
        flush();

        const unsigned char *buf = smem + (i & 1) * tile_bytes;
        const int s0 = key_lo + i * NK;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const int nloc = (col * NBW + nb) * 32;
            const int s = s0 + nloc + m;
            bool vis[G::SLOTS];
            bool any = false;
#pragma unroll
            for (int j = 0; j < G::SLOTS; ++j) {
                vis[j] = s < out_vis[j] && !half_is_neg_inf(mcur[nb][j]);
                any |= vis[j];
            }
            float res[G::SLOTS];
#pragma unroll
            for (int j = 0; j < G::SLOTS; ++j) res[j] = -INFINITY;
            if (__builtin_amdgcn_ballot_w64(any) != 0) {
                f32x16 acc[G::MBLK];
#pragma unroll
                for (int mb = 0; mb < G::MBLK; ++mb) acc[mb] = f32x16{};
                const int n = nloc + m;
                const unsigned char *rowp = buf + n * G::ROWB;
                const int f = swz<D>(n);
                auto bfrag = [&](int kk) {
                    return *reinterpret_cast<const half8 *>(rowp + (((kh * G::KSTEPS + kk) ^ f) << 4));
                };
                half8 b = bfrag(0);
#pragma unroll
                for (int kk = 0; kk < G::KSTEPS; ++kk) {
                    // fetch the next K step's key fragment while these MFMAs run
                    const half8 bn = kk + 1 < G::KSTEPS ? bfrag(kk + 1) : b;
#pragma unroll
                    for (int mb = 0; mb < G::MBLK; ++mb)
                        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[mb][kk], b, acc[mb], 0, 0, 0);
                    b = bn;
                }
                // epilogue: register r of M-block mb is head mb*HPB + r % (4G)
                // of row slot r / (4G); rectify, weight, sum over heads
#pragma unroll
                for (int j = 0; j < G::SLOTS; ++j) {
                    float sum = 0.0f;
#pragma unroll
                    for (int mb = 0; mb < G::MBLK; ++mb)
#pragma unroll
                        for (int rr = 0; rr < 4 * G::G; ++rr)
                            sum = fmaf(relu(acc[mb][4 * G::G * j + rr]),
                                       PAD ? head_weight(wc, mb * G::HPB + rr, a.n_heads) : wc[mb * G::HPB + rr], sum);
                    if (vis[j]) res[j] = !PAD || a.add_mask ? sum + (float)mcur[nb][j] : sum;
                }
            }
            if constexpr (STREAM) {
                // candidates: a wave's two lane halves hold two rows; one
                // LDS atomic per half claims the half's slots
#pragma unroll
                for (int j = 0; j < G::SLOTS; ++j) {
                    const bool take = vis[j] && (res[j] > lbf[j] || (res[j] == lbf[j] && (uint32_t)s <= lbs[j]));
                    const unsigned long long bal = __builtin_amdgcn_ballot_w64(take);
                    if (bal != 0ull) {
                        const uint32_t hb = kh ? (uint32_t)(bal >> 32) : (uint32_t)bal;
                        const int rl = out_t[j] - row_lo;
                        int base = 0;
                        if ((lane & 31) == 0 && hb != 0u) {
                            const int nadd = __popc(hb);
                            base = atomicAdd(&sl->cnt[rl], nadd);
                            if (base + nadd > trigger) sl->flag[i % 3] = 1;
                        }
                        base = __shfl(base, lane & 32, 64);
                        if (take) {
                            const int pos = base + __popc(hb & ((1u << (lane & 31)) - 1u));
                            if (pos < a.cand_cap) lst[j][pos] = stream_entry(stream_key(res[j]), s);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < G::SLOTS; ++j) pend[nb][j] = res[j];
            }
        }
        pend_s = s0 + col * NBW * 32 + m;
    }
    flush();
    if constexpr (STREAM) {
        wait_vmem_all();
        __syncthreads();  // every candidate counted
        if (tid < row_hi - row_lo) a.cand_count[(int64_t)(row_lo + tid) * a.n_chunks + chunk_id] = sl->cnt[tid];
        return;  // no score rows to fill
    }

    // ---- keys past the bound: -inf without loading anything ------------
    // (for the fused entry point only below each row's vis_len: its top-k
    // reads no further, so the rest of the workspace row is left unwritten)
    const int fill_lo = min(key_lo + n_tiles * NK, key_hi);
    if (fill_lo < key_hi) {
        const int nrows = row_hi - row_lo;
        const int width = key_hi - fill_lo;
        const bool to_vis = a.fill_to_vis && a.vis_len != nullptr;
        if (to_vis && tid < nrows) misc[2 + tid] = row_vis(row_lo + tid);  // misc holds 32 + 2 words
        if (to_vis) __syncthreads();
        auto row_end = [&](int r) { return to_vis ? misc[2 + r] : key_hi; };
        if (a.score_vec && (fill_lo & 3) == 0) {
            const int w4 = width >> 2;
            const float4 ninf = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            for (int c = tid; c < nrows * w4; c += kThreads) {
                const int r = c / w4;
                const int i4 = c - r * w4;
                if (fill_lo + 4 * i4 >= row_end(r)) continue;
                *reinterpret_cast<float4 *>(a.score + (int64_t)(row_lo + r) * a.score_st + fill_lo + 4 * i4) = ninf;
            }
            const int tail = width & 3;
            for (int c = tid; c < nrows * tail; c += kThreads) {
                const int r = c / tail;
                const int sidx = fill_lo + 4 * w4 + (c - r * tail);
                if (sidx >= row_end(r)) continue;
                a.score[(int64_t)(row_lo + r) * a.score_st + sidx] = -INFINITY;
            }
        } else {
            for (int c = tid; c < nrows * width; c += kThreads) {
                const int r = c / width;
                const int sidx = fill_lo + (c - r * width);
                if (sidx >= row_end(r)) continue;
                a.score[(int64_t)(row_lo + r) * a.score_st + sidx] = -INFINITY;
            }
        }
    }
}

// Dynamic LDS above 64 KiB must be enabled per kernel; done once per
// instantiation for the largest size used so far.
template <auto Kern>
hipError_t allow_lds(size_t bytes) {
    static std::atomic<int> allowed{65536};  // per kernel instance: the attribute is per kernel
    if ((int)bytes <= allowed.load(std::memory_order_relaxed)) return hipSuccess;
    hipError_t e = hipFuncSetAttribute((const void *)Kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) allowed.store((int)bytes, std::memory_order_relaxed);
    return e;
}

template <int H, int D, int NBW, bool PAD, bool STREAM>
hipError_t launch_one(const ScoreArgs &a, const ScorePlan &p, hipStream_t stream) {
    auto kern = score_kernel<H, D, NBW, PAD, STREAM>;
    hipError_t e = allow_lds<score_kernel<H, D, NBW, PAD, STREAM>>(p.lds_bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, p.grid, dim3(kThreads), p.lds_bytes, stream, a);
    return hipGetLastError();
}

template <int H, int D, bool PAD, bool STREAM>
hipError_t launch_nbw(const ScoreArgs &a, const ScorePlan &p, hipStream_t stream) {
    if constexpr (D == 256) {
        return p.nbw == 2 ? launch_one<H, D, 2, PAD, STREAM>(a, p, stream) : launch_one<H, D, 1, PAD, STREAM>(a, p, stream);
    } else {
        return p.nbw == 4 ? launch_one<H, D, 4, PAD, STREAM>(a, p, stream) : launch_one<H, D, 1, PAD, STREAM>(a, p, stream);
    }
}

template <int H, int D, bool STREAM>
hipError_t launch_hd(const ScoreArgs &a, const ScorePlan &p, hipStream_t stream) {
    if (a.n_heads == H && a.head_dim == D && !a.accumulate && a.add_mask)
        return launch_nbw<H, D, false, STREAM>(a, p, stream);
    return launch_nbw<H, D, true, STREAM>(a, p, stream);
}

template <int H, bool STREAM>
hipError_t launch_h(const ScoreArgs &a, const ScorePlan &p, int D, hipStream_t stream) {
    if (D == 64) return launch_hd<H, 64, STREAM>(a, p, stream);
    if (D == 128) return launch_hd<H, 128, STREAM>(a, p, stream);
    if constexpr (H <= 32) return launch_hd<H, 256, STREAM>(a, p, stream);  // a pass holds 32 heads at 256
    return hipErrorInvalidValue;
}

}  // namespace

bool score_shape_supported(int n_heads, int head_dim) {
    return n_heads >= 1 && n_heads <= kMaxHeads && head_dim >= 8 && head_dim <= 256 && head_dim % 8 == 0;
}

int compiled_heads(int n_heads) {
    int h = 4;
    while (h < n_heads) h *= 2;
    return h;
}

ScorePlan plan_score(ScoreArgs &a, int n_heads, int head_dim) {
    ScorePlan p{};
    const int hpb = n_heads < 16 ? n_heads : 16;
    const int tpb = 32 / hpb;
    // waves along rows: enough row groups for the rows one request owns
    const int rows = a.q_per_req;
    int ng = 1;
    while (ng < kWaves && ng * tpb < rows) ng *= 2;
    p.nc = kWaves / ng;
    // 32 KB key tiles: 128 keys of 128 dimensions (64 at 256)
    p.nbw = p.nc == 1 ? (head_dim == 256 ? 2 : 4) : 1;
    p.tile_keys = 32 * p.nc * p.nbw;
    p.rows_per_group = ng * tpb;
    a.nc = p.nc;
    a.groups_per_req = rows > 0 ? (rows + p.rows_per_group - 1) / p.rows_per_group : 0;
    a.n_row_groups = a.groups_per_req;

    // keys per workgroup: aim for a few workgroups per compute unit (two
    // are resident at a time).  With fewer row groups than compute units (a
    // chunk of tokens against a long key range) eight per compute unit ran
    // 1.3% faster than four on 1024 tokens x 131072 keys (finer key chunks,
    // a shorter tail); with many row groups their own count already gives
    // several per compute unit, and splitting their keys only reloads q.
    const int cus = device_cu_count();
    const int target = (a.n_row_groups < cus ? 8 : 4) * cus;
    const int max_tiles = (a.n_cols + p.tile_keys - 1) / p.tile_keys;
    int n_chunks = a.n_row_groups > 0 ? (target + a.n_row_groups - 1) / a.n_row_groups : 1;
    n_chunks = n_chunks < 1 ? 1 : (n_chunks > max_tiles ? max_tiles : n_chunks);
    if (n_chunks < 1) n_chunks = 1;
    const int tiles_per_chunk = (max_tiles + n_chunks - 1) / n_chunks;
    a.chunk = (tiles_per_chunk > 0 ? tiles_per_chunk : 1) * p.tile_keys;
    a.n_chunks = (a.n_cols + a.chunk - 1) / a.chunk;
    if (a.n_chunks < 1) a.n_chunks = 1;

    const size_t tile_bytes = (size_t)p.tile_keys * 2 * head_dim;
    p.lds_bytes = 2 * tile_bytes + kMiscBytes;
    p.grid = dim3((unsigned)(a.n_row_groups * a.n_chunks));
    return p;
}

template <bool STREAM>
hipError_t launch_any(const ScoreArgs &a, const ScorePlan &p, int n_heads, int head_dim, hipStream_t stream) {
    switch (n_heads) {
        case 4: return launch_h<4, STREAM>(a, p, head_dim, stream);
        case 8: return launch_h<8, STREAM>(a, p, head_dim, stream);
        case 16: return launch_h<16, STREAM>(a, p, head_dim, stream);
        case 32: return launch_h<32, STREAM>(a, p, head_dim, stream);
        default: return launch_h<64, STREAM>(a, p, head_dim, stream);
    }
}

hipError_t launch_score(const ScoreArgs &a, const ScorePlan &p, int n_heads, int head_dim, hipStream_t stream) {
    return launch_any<false>(a, p, n_heads, head_dim, stream);
}

ScorePlan plan_score_stream(ScoreArgs &a, int n_heads, int head_dim) {
    ScorePlan p = plan_score(a, n_heads, head_dim);
    // key chunks: at most kStreamMaxChunks of whole tiles, fixed by the row
    // width alone (the workspace is sized from it)
    const int want = stream_chunks(a.n_cols);
    const int max_tiles = (a.n_cols + p.tile_keys - 1) / p.tile_keys;
    const int tiles_per_chunk = (max_tiles + want - 1) / want;
    a.chunk = (tiles_per_chunk > 0 ? tiles_per_chunk : 1) * p.tile_keys;
    a.n_chunks = (a.n_cols + a.chunk - 1) / a.chunk;
    if (a.n_chunks < 1) a.n_chunks = 1;
    p.lds_bytes = p.lds_bytes + sizeof(StreamLds);
    p.grid = dim3((unsigned)(a.n_row_groups * a.n_chunks));
    return p;
}

hipError_t launch_score_stream(const ScoreArgs &a, const ScorePlan &p, int n_heads, int head_dim,
                               hipStream_t stream) {
    return launch_any<true>(a, p, n_heads, head_dim, stream);
}

}  // namespace lidx
