// Paged decode / speculative-decode score kernel for gfx950 (CDNA4).
//
//   score[r*Q + j][s] = sum_h w[h] * max(q[r*Q + j][h][:] . k_r[s][:], 0) + mask
//   for s < seq_len[r] - Q + 1 + j, -inf beyond
//
// (vLLM PR #45743: one program per request batches that request's query
// tokens into the QK matrix product and uses no implicit scale; keys come
// from a paged cache through the block table.  llama.cpp b11372: rectify each
// head, then sum, keys read once for all heads.)
//
// Decode moves ~256 bytes of keys per (request, key) and does little math on
// them, so this kernel is organised around memory latency rather than MFMA
// throughput:
//  * A workgroup owns one request's query rows and a chunk of at most 256 of
//    its keys.  Everything that does not depend on the request's length --
//    the block ids of the chunk, the q fragments, the sequence length -- is
//    requested at once, so the prologue costs one memory round trip.
//  * All key tiles of the chunk are then requested together (16-byte
//    direct-to-LDS loads into swizzled rows) and consumed in order, each wave
//    waiting only for the tiles it needs; the scores stay in registers and
//    are stored after the last tile, so loads and stores never interleave.
//  * With one query row (plain decode) and >= 32 heads, the two row slots of
//    each 32-row MFMA block carry the two halves of the heads instead of a
//    padding row: half the MFMAs and half the q registers of the general
//    mapping, and one cross-lane add per key.
#include <math.h>

#include <atomic>

#include "device_common.h"
#include "internal.h"

namespace lidx {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kMaxTiles = 8;
constexpr int kChunkBytes = 65536;  // keys staged per workgroup

template <int H, int D, bool SPLIT>
__global__ void __launch_bounds__(kThreads, 2) decode_kernel(ScoreArgs a) {
    using G = Geo<H, D>;
    constexpr int MB = SPLIT ? H / 32 : G::MBLK;   // M-blocks per wave
    constexpr int TPB = SPLIT ? 1 : G::TPB;        // query rows per wave
    constexpr int SLOTS = SPLIT ? 1 : G::SLOTS;    // query rows per lane
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int tid = threadIdx.x;
    const int wid = tid >> 6;
    const int lane = tid & 63;
    const int m = lane & 31;
    const int kh = lane >> 5;
    const int nc = a.nc;
    const int tg = wid / nc;
    const int col = wid - tg * nc;
    const int NK = 32 * nc;                 // keys per tile
    const int tile_bytes = NK * G::ROWB;
    const int rows_per_wg = (kWaves / nc) * TPB;
    const int dpt = NK * G::CPR / kThreads; // 16-byte loads per thread per tile

    const int chunk_id = blockIdx.x % a.n_chunks;
    const int rg = blockIdx.x / a.n_chunks;
    const int req = rg / a.groups_per_req;
    const int sub = rg - req * a.groups_per_req;
    const int req_row0 = req * a.q_per_req;
    const int row_lo = req_row0 + sub * rows_per_wg;
    const int row_hi = min(req_row0 + a.q_per_req, row_lo + rows_per_wg);
    const int key_lo = chunk_id * a.chunk;
    const int key_hi = min(a.n_cols, key_lo + a.chunk);

    int *bt_lds = reinterpret_cast<int *>(smem + a.chunk * G::ROWB);
    int *misc = bt_lds + (a.chunk + a.block_size - 1) / a.block_size + 2;

    // ---- 1. prologue: block ids, sequence length, q, all at once --------
    const int bs = a.block_size;
    int b_lo, b_hi;
    if (a.bs_shift >= 0) {
        b_lo = key_lo >> a.bs_shift;
        b_hi = (key_hi + bs - 1) >> a.bs_shift;
    } else {
        b_lo = key_lo / bs;
        b_hi = (key_hi + bs - 1) / bs;
    }
    // entries exist up to ceil(max_seq_len / block_size) <= bt_stride; the
    // ones past the request's length are staged but never used
    for (int i = tid; i < b_hi - b_lo; i += kThreads)
        bt_lds[i] = a.block_table[(int64_t)req * a.bt_stride + b_lo + i];
    const int seq_len = max(0, ((const_i32 *)a.seq_lens)[req]);

    // q fragments (A operand): row m of M-block mb is (query row, head)
    half8 qa[MB][G::KSTEPS];
    {
        int t, head0;
        if constexpr (SPLIT) {
            t = row_lo;
            head0 = ((m >> 2) & 1) * (H / 2) + (m >> 3) * 4 + (m & 3);
        } else {
            t = row_lo + tg * TPB + (((m >> 3) / G::G) << 1) + ((m >> 2) & 1);
            head0 = ((m >> 3) % G::G) * 4 + (m & 3);
        }
        const bool ok = t < row_hi;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int head = head0 + mb * (SPLIT ? 16 : G::HPB);
            const _Float16 *src = a.q + (int64_t)t * a.q_st + (int64_t)real_head(head, a.n_heads) * a.q_sh + kh * (D / 2);
#pragma unroll
            for (int kk = 0; kk < G::KSTEPS; ++kk)  // zero past the real head dimension
                qa[mb][kk] = ok && kh * (D / 2) + kk * 8 < a.head_dim ? *reinterpret_cast<const half8 *>(src + kk * 8)
                                                                     : half8{};
        }
    }
    // weights: SGPR operands in the general mapping; per-lane registers when
    // the two lane halves hold different heads
    const_f32 *wc = (const_f32 *)a.w;
    float wv[SPLIT ? MB : 1][16];
    if constexpr (SPLIT) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float w_lo = head_weight((const_f32 *)a.w, mb * 16 + r, a.n_heads);
                const float w_hi = head_weight((const_f32 *)a.w, H / 2 + mb * 16 + r, a.n_heads);
                wv[mb][r] = kh ? w_hi : w_lo;
            }
    }

    // rows this lane writes and their visible prefixes (query j of the
    // request sees s < seq_len - Q + 1 + j)
    int out_t[SLOTS], out_vis[SLOTS];
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
        out_t[j] = SPLIT ? row_lo : row_lo + tg * TPB + 2 * j + kh;
        out_vis[j] = out_t[j] < row_hi
                         ? min(max(seq_len - a.q_per_req + 1 + (out_t[j] - req_row0), 0), a.n_cols)
                         : 0;
    }
    __syncthreads();  // bt_lds

    // ---- 2. keys visible to any row of this workgroup -------------------
    int bound = min(key_hi, min(max(seq_len - a.q_per_req + 1 + (row_hi - 1 - req_row0), 0), a.n_cols));
    if (bound < key_lo) bound = key_lo;
    if (a.mask != nullptr && bound > key_lo) {
        if (tid == 0) misc[0] = key_lo;
        __syncthreads();
        int last = key_lo;
        const int span = bound - key_lo;
        const int nrows = row_hi - row_lo;
        for (int c = tid; c < nrows * span; c += kThreads) {
            const int r = c / span;
            const int s = key_lo + (c - r * span);
            const int t = row_lo + r;
            const int rv = min(max(seq_len - a.q_per_req + 1 + (t - req_row0), 0), a.n_cols);
            if (s < rv && !half_is_neg_inf(a.mask[(int64_t)t * a.mask_st + s])) last = max(last, s + 1);
        }
        if (last > key_lo) atomicMax(&misc[0], last);
        __syncthreads();
        bound = misc[0];
    }
    const int n_tiles = bound > key_lo ? (bound - key_lo + NK - 1) / NK : 0;

    // ---- 3. mask values, then every tile's keys -------------------------
    _Float16 mv[kMaxTiles][SLOTS];
#pragma unroll
    for (int i = 0; i < kMaxTiles; ++i) {
        const int s = key_lo + i * NK + col * 32 + m;
#pragma unroll
        for (int j = 0; j < SLOTS; ++j) {
            _Float16 v = (_Float16)0.0f;
            if (i < n_tiles && a.mask != nullptr && s < out_vis[j]) v = a.mask[(int64_t)out_t[j] * a.mask_st + s];
            mv[i][j] = v;
        }
    }
    for (int i = 0; i < n_tiles; ++i) {
        const int s0 = key_lo + i * NK;
        unsigned char *base = smem + i * tile_bytes;
        for (int it = 0; it < dpt; ++it) {
            const int c = (it * kWaves + wid) * 64 + lane;
            const int n = c / G::CPR;
            const int lc = (c & (G::CPR - 1)) ^ swz<D>(n);
            const int s = s0 + n;
            const _Float16 *src = a.k;  // any valid address for keys past the bound
            if (s < bound) {
                int blk, slot;
                if (a.bs_shift >= 0) {
                    blk = s >> a.bs_shift;
                    slot = s - (blk << a.bs_shift);
                } else {
                    blk = s / bs;
                    slot = s - blk * bs;
                }
                const int64_t phys = bt_lds[blk - b_lo];
                src = a.k + (phys * bs + slot) * a.k_ss + lc * 8;
            }
            if (lc * 8 >= a.head_dim) src = reinterpret_cast<const _Float16 *>(kZeroChunk);  // padded tile
            dma16(src, base + (it * kWaves + wid) * 1024);
        }
    }

    // ---- 4. tiles in order ------------------------------------------------
    float res[kMaxTiles][SLOTS];
#pragma unroll
    for (int i = 0; i < kMaxTiles; ++i) {
#pragma unroll
        for (int j = 0; j < SLOTS; ++j) res[i][j] = -INFINITY;
        if (i < n_tiles) {
            wait_vmem_below(dpt * (n_tiles - 1 - i));
            __syncthreads();  // tile i is in LDS for every wave
            const int s = key_lo + i * NK + col * 32 + m;
            bool vis[SLOTS];
            bool any = false;
#pragma unroll
            for (int j = 0; j < SLOTS; ++j) {
                vis[j] = s < out_vis[j] && !half_is_neg_inf(mv[i][j]);
                any |= vis[j];
            }
            if (__builtin_amdgcn_ballot_w64(any) != 0) {
                f32x16 acc[MB];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16{};
                const int n = col * 32 + m;
                const unsigned char *rowp = smem + i * tile_bytes + n * G::ROWB;
                const int f = swz<D>(n);
                auto bfrag = [&](int kk) {
                    return *reinterpret_cast<const half8 *>(rowp + (((kh * G::KSTEPS + kk) ^ f) << 4));
                };
                half8 b = bfrag(0);
#pragma unroll
                for (int kk = 0; kk < G::KSTEPS; ++kk) {
                    const half8 bn = kk + 1 < G::KSTEPS ? bfrag(kk + 1) : b;
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[mb][kk], b, acc[mb], 0, 0, 0);
                    b = bn;
                }
                if constexpr (SPLIT) {
                    // this lane half's heads, then the other half's via lane ^ 32
                    float sum = 0.0f;
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) sum = fmaf(relu(acc[mb][r]), wv[mb][r], sum);
                    sum += __shfl_xor(sum, 32, 64);
                    if (vis[0]) res[i][0] = a.add_mask ? sum + (float)mv[i][0] : sum;
                } else {
#pragma unroll
                    for (int j = 0; j < SLOTS; ++j) {
                        float sum = 0.0f;
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                            for (int rr = 0; rr < 4 * G::G; ++rr)
                                sum = fmaf(relu(acc[mb][4 * G::G * j + rr]), head_weight(wc, mb * G::HPB + rr, a.n_heads), sum);
                        if (vis[j]) res[i][j] = a.add_mask ? sum + (float)mv[i][j] : sum;
                    }
                }
            }
        }
    }

    // ---- 5. stores, then -inf past the last tile -------------------------
#pragma unroll
    for (int i = 0; i < kMaxTiles; ++i) {
        const int s = key_lo + i * NK + col * 32 + m;
        if (i < n_tiles && s < key_hi) {
#pragma unroll
            for (int j = 0; j < SLOTS; ++j)
                if (out_t[j] < row_hi && (!SPLIT || kh == 0)) {
                    float *dst = a.score + (int64_t)out_t[j] * a.score_st + s;
                    // a later pass over more heads adds to the stored partial
                    // sum (-inf stays -inf)
                    *dst = a.accumulate ? res[i][j] + *dst : res[i][j];
                }
        }
    }
    const int fill_lo = min(key_lo + n_tiles * NK, key_hi);
    if (fill_lo < key_hi) {
        const int nrows = row_hi - row_lo;
        const int width = key_hi - fill_lo;
        if (a.score_vec && (fill_lo & 3) == 0) {
            const int w4 = width >> 2;
            const float4 ninf = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            for (int c = tid; c < nrows * w4; c += kThreads) {
                const int r = c / w4;
                const int i4 = c - r * w4;
                *reinterpret_cast<float4 *>(a.score + (int64_t)(row_lo + r) * a.score_st + fill_lo + 4 * i4) = ninf;
            }
            const int tail = width & 3;
            for (int c = tid; c < nrows * tail; c += kThreads) {
                const int r = c / tail;
                a.score[(int64_t)(row_lo + r) * a.score_st + fill_lo + 4 * w4 + (c - r * tail)] = -INFINITY;
            }
        } else {
            for (int c = tid; c < nrows * width; c += kThreads) {
                const int r = c / width;
                a.score[(int64_t)(row_lo + r) * a.score_st + fill_lo + (c - r * width)] = -INFINITY;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Persistent producer/consumer score kernel, for paged keys (decode,
// speculative decode).
//
// One workgroup per compute unit.  The work is the list of (row group, key
// tile) pairs of all rows, row group by row group, where a row group's tiles
// cover the keys visible to any of its rows; each workgroup takes an equal
// contiguous share of it, computed in the kernel from seq_lens,
// so short and long rows balance and no workgroup is idle.
//
// A wave can keep only so many loads in flight; issuing one more stalls it
// until an earlier one returns, and while it stalls it computes nothing.  So
// the loads and the arithmetic run on different waves:
//  * four producers (one per SIMD) fetch, for every tile, a quarter of its
//    keys (16-byte direct-to-LDS loads into swizzled rows of a ring of 3 or
//    4 tiles),
//    its f16 mask rows when a mask is given (same loads, into a mask ring)
//    and the tile's block ids three tiles ahead (4-byte
//    direct-to-LDS loads into a small ring per producer, issued behind the
//    loads of the current tile); with one query row
//    per request also the q row of each new row group (fragment order, one
//    of two LDS slots).  A producer issues only direct-to-LDS loads, so
//    exact vmcnt counts tell when its part of a tile has landed; it then
//    publishes its count of landed tiles in LDS.
//  * each consumer (four, one per SIMD) waits
//    until every producer has published the tile it needs, computes its
//    32-key blocks and writes the scores straight to memory, then publishes
//    how many tiles it has finished; a producer reuses a ring slot (or a q
//    slot) only when every consumer is done with it.  Consumers load from
//    memory only when their row group changes (q, visible lengths), so the
//    compiler never has to wait for their score stores.
//  * with >= 32 heads every consumer owns one query row and uses the split
//    head mapping (q in 64 registers, two accumulator sets so the products
//    of one 32-key block overlap the epilogue of the one before); fewer
//    heads pack 32/heads rows per M-block.
// ---------------------------------------------------------------------------

constexpr int kPcProducers = 4;                        // load waves, one per SIMD
constexpr int kStreamTK = 128;                         // keys per tile
constexpr int kStreamNBUF = 3;                         // tiles in the LDS rings (4 where they fit, below)
constexpr int kMaxRG = 1536;                           // row groups handled in-kernel
constexpr int kBtLead = 3;                             // block ids fetched this many tiles ahead
constexpr int kBtRing = kBtLead + 3;                   // block-id ring slots
constexpr int kFlagReady = 12;                         // misc words: tiles landed, per producer
constexpr int kFlagDone = 16;                          // misc words: tiles done, per consumer

constexpr int kPcConsumers = 4;                        // compute waves, one per SIMD

template <int H, int D, bool SPLIT, int NC>
struct StreamGeo {
    static constexpr int NCONS = kPcConsumers;
    using G = Geo<H, D>;
    static constexpr int NG = NCONS / NC;                      // consumer waves along rows
    static constexpr int MB = SPLIT ? H / 32 : G::MBLK;        // M-blocks per consumer
    static constexpr int QL = MB * G::KSTEPS;                  // 16-byte q fragments per lane
    static constexpr int TPB = SPLIT ? 1 : G::TPB;             // query rows per consumer
    static constexpr int ROWS = NG * TPB;                      // rows of one row group
    static constexpr bool QLDS = SPLIT && NG == 1;             // q through the LDS slots
    static constexpr int TILE_BYTES = kStreamTK * G::ROWB;
    static constexpr int QSLOT = QLDS ? QL * 1024 : 0;         // bytes of one q slot
    static constexpr int MROWS4 = (ROWS + 3) / 4;              // mask loads per tile (4 rows of 128 keys each)
    static constexpr int MSLOT = MROWS4 * 1024;                // bytes of one mask slot
    static constexpr int DPT = kStreamTK * G::CPR / 64 / kPcProducers;  // key loads per producer per tile
    static constexpr int NBW = kStreamTK / (32 * NC);          // 32-key blocks per consumer per tile
    static constexpr size_t lds_bytes_for(int nbuf) {
        return (size_t)nbuf * (TILE_BYTES + MSLOT) + 2 * (size_t)QSLOT + 4 * (3 * (size_t)kMaxRG + 1) +
               4 * (size_t)kPcProducers * kBtRing * 64 + 128;
    }
    // Ring depth and publication lag.  A producer publishes tile j once it
    // has issued tile j + LAG, so LAG + 1 tiles are in flight while the
    // consumers work on an older one; that needs NBUF >= LAG + 2.  With q
    // through the LDS slots a new row group's slot waits for the consumers
    // to pass the first tile of the group two back, which may be the tile
    // just before: only LAG 1 lets them get there, so those keep 3 and 1.
    static constexpr int NBUF = (!QLDS && lds_bytes_for(4) <= 160 * 1024) ? 4 : kStreamNBUF;
    static constexpr int LAG = NBUF - 2;
    static constexpr size_t lds_bytes() { return lds_bytes_for(NBUF); }
};

static_assert(StreamGeo<64, 128, true, 4>::lds_bytes() <= 160 * 1024, "LDS budget");
static_assert(StreamGeo<4, 128, false, 1>::lds_bytes() <= 160 * 1024, "LDS budget");

// q fragments (A operand) of one query row t with the split head mapping:
// row m of M-block mb is head (m>>2 & 1)*H/2 + (m>>3)*4 + (m&3) + 16*mb.
template <int H, int D, int MB, int KS>
__device__ __forceinline__ void load_q_split(half8 (&qa)[MB][KS], const _Float16 *qp, int64_t q_st,
                                             int64_t q_sh, int t, int m, int kh, int n_heads) {
    const int head0 = ((m >> 2) & 1) * (H / 2) + (m >> 3) * 4 + (m & 3);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const _Float16 *src = qp + (int64_t)t * q_st + (int64_t)real_head(head0 + mb * 16, n_heads) * q_sh + kh * (D / 2);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) qa[mb][kk] = *reinterpret_cast<const half8 *>(src + kk * 8);
    }
}

// q fragments of the general mapping for consumer tg of a row group: rows
// row0.. (rhi exclusive).  Rows past rhi repeat row0; their scores are
// never kept.
template <int H, int D, int MB, int KS>
__device__ __forceinline__ void load_q_rows(half8 (&qa)[MB][KS], const _Float16 *qp, int64_t q_st,
                                            int64_t q_sh, int row0, int rhi, int tg, int m, int kh, int n_heads) {
    using G = Geo<H, D>;
    const int t = row0 + tg * G::TPB + (((m >> 3) / G::G) << 1) + ((m >> 2) & 1);
    const int tc = t < rhi ? t : row0;
    const int head0 = ((m >> 3) % G::G) * 4 + (m & 3);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const _Float16 *src = qp + (int64_t)tc * q_st + (int64_t)real_head(head0 + mb * G::HPB, n_heads) * q_sh + kh * (D / 2);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) qa[mb][kk] = *reinterpret_cast<const half8 *>(src + kk * 8);
    }
}

// acc[mb] = q fragments (M-block mb) x the 32 keys of LDS rows rowp.. .
template <int H, int D, int MB, int KS>
__device__ __forceinline__ void mfma_keys(f32x16 (&acc)[MB], const half8 (&qa)[MB][KS],
                                          const lds_u8 *rowp, int kh, int f) {
    using G = Geo<H, D>;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16{};
    half8 b = *reinterpret_cast<const lds_half8 *>(rowp + (((kh * G::KSTEPS) ^ f) << 4));
#pragma unroll
    for (int kk = 0; kk < G::KSTEPS; ++kk) {
        half8 bn = b;
        if (kk + 1 < G::KSTEPS) bn = *reinterpret_cast<const lds_half8 *>(rowp + (((kh * G::KSTEPS + kk + 1) ^ f) << 4));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[mb][kk], b, acc[mb], 0, 0, 0);
        b = bn;
    }
}

__device__ __forceinline__ int lds_flag(const lds_i32 *p) { return uni(*(const volatile lds_i32 *)p); }
__device__ __forceinline__ void set_lds_flag(lds_i32 *p, int v) {
    asm volatile("" ::: "memory");
    *(volatile lds_i32 *)p = v;
}

typedef __attribute__((address_space(3))) unsigned short lds_u16;

template <int H, int D, bool SPLIT, int NC>
__global__ void __launch_bounds__((kPcConsumers + kPcProducers) * 64, 1) stream_pc_kernel(ScoreArgs args, int n_req) {
    using G = Geo<H, D>;
    using SG = StreamGeo<H, D, SPLIT, NC>;
    constexpr int NCONS = kPcConsumers;
    constexpr int TK = kStreamTK;
    constexpr int NT = (NCONS + kPcProducers) * 64;
    constexpr int NW = NCONS + kPcProducers;
    constexpr int NBW = SG::NBW, MB = SG::MB, KS = G::KSTEPS, TPB = SG::TPB, ROWS = SG::ROWS;
    constexpr int SLOTS = SPLIT ? 1 : G::SLOTS;
    constexpr int TILE_BYTES = SG::TILE_BYTES, DPT = SG::DPT;
    constexpr bool QLDS = SG::QLDS;
    static_assert(NBW >= 1, "tile too small");
    static_assert(NCONS + kPcProducers <= 16, "flag words");

    // plain scalars (no argument struct is captured anywhere)
    const _Float16 *const qp = args.q;
    const int64_t q_st = args.q_st, q_sh = args.q_sh;
    const _Float16 *const kp = args.k;
    const int64_t k_ss = args.k_ss;
    const int32_t *const btab = args.block_table;
    const int64_t bt_stride = args.bt_stride;
    const int bs = args.block_size, sh = args.bs_shift;
    const int32_t *const seqp = args.seq_lens;
    const _Float16 *const maskp = args.mask;        // nullable
    const int64_t mask_st = args.mask_st;
    const float *const wp = args.w;
    const int nh = args.n_heads;
    float *const scorep = args.score;
    const int64_t score_st = args.score_st;
    const int n_cols = args.n_cols, Q = args.q_per_req, gpr = args.groups_per_req, n_rg = args.n_row_groups;

    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    lds_u8 *const smem = (lds_u8 *)smem_raw;
    lds_u8 *const keys = smem;
    lds_u8 *const mslots = smem + SG::NBUF * TILE_BYTES;                           // [NBUF][MSLOT]
    lds_u8 *const qslots = mslots + SG::NBUF * SG::MSLOT;                          // QLDS: 2 slots
    lds_i32 *const pref = (lds_i32 *)(qslots + 2 * SG::QSLOT);                     // [n_rg + 1]
    lds_i32 *const gbd = pref + kMaxRG + 1;                                        // [n_rg] keys visible to the group
    lds_i32 *const slen = gbd + kMaxRG;                                            // [n_req]
    lds_i32 *const btr = slen + kMaxRG;                                            // [producer][ring][64]
    lds_i32 *const misc = btr + kPcProducers * kBtRing * 64;                       // 32 words

    const int tid = threadIdx.x, wid = uni(tid >> 6), lane = tid & 63;
    const int m = lane & 31, kh = lane >> 5;

    // keys visible to row t = req*Q + j of a request whose sequence holds sl keys
    auto vis_of = [=](int sl, int req, int t) { return min(max(sl - Q + 1 + (t - req * Q), 0), n_cols); };

    // ---- 1. keys visible to each row group, tiles, prefix sum ------------
    // With at most 64 row groups and requests every wave works the split out
    // itself, one row group (and one request) per lane, and later reads it
    // back with readlane: no LDS arrays, and one barrier (for the flags),
    // passed while the sequence lengths are on their way.  Otherwise the
    // split goes through LDS.
    const bool small = n_rg <= 64 && n_req <= 64;
    // The producers read the block table only once the split is known: a
    // dependent round trip before the first key load.  While the sequence
    // lengths are on their way, every lane loads one table entry, so that
    // together the workgroups of one XCD (blockIdx.x mod 8) bring the table
    // rows' first ceil(n_cols / block_size) entries into that XCD's L2 (up
    // to one entry per thread of a workgroup).  The values are not used;
    // the index is clamped, not branched on, so the load stays in straight
    // code and waiting for the lengths does not wait for it, and every entry
    // loaded lies inside the [n_req][bt_stride] table (n_req >= 1).
    int bt_warm;
    auto warm_block_table = [&]() {
        const int nbm = sh >= 0 ? (n_cols + bs - 1) >> sh : (n_cols + bs - 1) / bs;
        const int n_e = (int)min((int64_t)n_req * nbm, (int64_t)0x7fffffff);
        const int per_xcd = (int)((gridDim.x + 7) / 8);
        const int csz = min((n_e + per_xcd - 1) / per_xcd, NT);
        const int e = min((int)(blockIdx.x / 8 % per_xcd) * csz + min(tid, csz - 1), n_e - 1);
        const int r = (int)((unsigned)e / (unsigned)nbm);
        bt_warm = btab[(int64_t)r * bt_stride + (e - r * nbm)];
    };
    int sl_l = 0, gbd_l = 0, pref_l = 0, tiles_l = 0, total_l = 0;
    int64_t T;
    int rg_first = 0;
    if (small) {
        // one load per lane (n_req >= 1), the warming load behind it, then
        // the wait; a row group's length comes from its request's lane
        const int sl_raw = seqp[min(lane, n_req - 1)];
        warm_block_table();
        asm volatile("" ::"v"(sl_raw) : "memory");  // wait for the lengths here, after both loads are issued
        sl_l = lane < n_req ? max(0, sl_raw) : 0;
        const int sl_g = __builtin_amdgcn_ds_bpermute((lane / gpr) << 2, sl_l);
        if (tid < 32) misc[tid] = 0;
        lds_barrier();
        if (lane < n_rg) {
            const int req = lane / gpr, sub = lane - req * gpr;
            const int r0 = req * Q + sub * ROWS, r1 = min(req * Q + Q, r0 + ROWS);
            gbd_l = vis_of(sl_g, req, r1 - 1);
            tiles_l = (gbd_l + TK - 1) / TK;
        }
        const int incl = wave_incl_scan(tiles_l);
        pref_l = incl - tiles_l;
        total_l = __builtin_amdgcn_readlane(incl, 63);
        T = total_l;
    } else {
        for (int r = tid; r < n_req; r += NT) slen[r] = max(0, seqp[r]);
        warm_block_table();
        if (tid < 32) misc[tid] = 0;
        lds_barrier();
        for (int e = tid; e < n_rg; e += NT) {
            const int req = e / gpr, sub = e - (e / gpr) * gpr;
            const int r0 = req * Q + sub * ROWS, r1 = min(req * Q + Q, r0 + ROWS);
            gbd[e] = vis_of(slen[req], req, r1 - 1);
        }
        lds_barrier();
        {
            const int per = (n_rg + NT - 1) / NT;
            int local = 0;
            for (int q = 0; q < per; ++q) {
                const int e = tid * per + q;
                if (e < n_rg) local += (gbd[e] + TK - 1) / TK;
            }
            const int incl = wave_incl_scan(local);
            if (lane == 63) misc[wid] = incl;
            lds_barrier();
            int run = incl - local, total = 0;
            for (int w = 0; w < NW; ++w) {
                run += w < wid ? misc[w] : 0;
                total += misc[w];
            }
            for (int q = 0; q < per; ++q) {
                const int e = tid * per + q;
                if (e < n_rg) {
                    pref[e] = run;
                    run += (gbd[e] + TK - 1) / TK;
                }
            }
            if (tid == 0) pref[n_rg] = total;
            lds_barrier();
        }
        T = uni(pref[n_rg]);
    }
    // Consecutive shares of the work (the tiles of one request, in order)
    // go to the workgroups of one XCD (workgroup b runs on XCD b mod 8), so
    // that a request's q rows and block-table lines, read by every
    // workgroup sharing the request, are fetched into one L2.
    const unsigned share = gridDim.x % 8 == 0 ? (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8 : blockIdx.x;
    const int t_begin = (int)(T * share / gridDim.x);
    const int t_end = (int)(T * (share + 1) / gridDim.x);
    const int n_mine = t_end - t_begin;
    if (small) {
        const unsigned long long hit = __builtin_amdgcn_ballot_w64(
            lane < n_rg && pref_l <= t_begin && t_begin < pref_l + tiles_l);
        rg_first = n_mine > 0 ? (int)__builtin_ctzll(hit) : 0;
    } else {
        if (n_mine > 0)
            for (int e = tid; e < n_rg; e += NT)
                if (pref[e] <= t_begin && t_begin < pref[e + 1]) misc[8] = e;
        lds_barrier();
        rg_first = n_mine > 0 ? uni(misc[8]) : 0;
    }
    // the split, read back: first tile of row group e (e <= n_rg), keys
    // visible to row group e, keys visible to row t of request req
    auto pref_at = [&](int e) -> int {
        if (small) return e >= n_rg ? total_l : __builtin_amdgcn_readlane(pref_l, e);
        return uni(pref[e]);
    };
    auto gbd_at = [&](int e) -> int { return small ? __builtin_amdgcn_readlane(gbd_l, e) : uni(gbd[e]); };
    auto row_vis = [&](int req, int t) {
        return vis_of(small ? __builtin_amdgcn_readlane(sl_l, req) : slen[req], req, t);
    };

    // per-tile cursor (wave-uniform): row group, its ordinal among this
    // workgroup's row groups, first key, keys visible to the group, and the
    // group's tile range [lo, hi) in registers, so that a step inside the
    // group reads no LDS (advance: the cursor of tile j from that of j-1)
#define LIDX_ADVANCE(rg, ord, s0, bound, lo, hi, j)          \
    do {                                                     \
        const int t_ = t_begin + (j);                        \
        if (t_ >= hi) {                                      \
            int e_ = rg + 1;                                 \
            while (pref_at(e_ + 1) <= t_) ++e_;              \
            ++ord;                                           \
            rg = e_;                                         \
            lo = pref_at(e_);                                \
            hi = pref_at(e_ + 1);                            \
            bound = gbd_at(e_);                              \
        }                                                    \
        s0 = (t_ - lo) * TK;                                 \
    } while (0)

    const int lo_first = n_mine > 0 ? pref_at(rg_first) : 0;
    const int hi_first = n_mine > 0 ? pref_at(rg_first + 1) : 0;
    const int s0_first = (t_begin - lo_first) * TK;
    const int bd_first = n_mine > 0 ? gbd_at(rg_first) : 0;

    if (wid >= NCONS) {
        // ================= producers =================
        // producer p issues loads p, p+4, p+8, ... of every tile
        const int p = wid - NCONS;
        lds_i32 *const bt_mine = btr + p * kBtRing * 64;
        int k_rg = rg_first, k_ord = 0, k_s0 = s0_first, k_bd = bd_first;     // tile j
        int k_lo = lo_first, k_hi = hi_first;
        int b_rg = rg_first, b_ord = 0, b_s0 = s0_first, b_bd = bd_first;     // tile next_bt
        int b_lo = lo_first, b_hi = hi_first;
        int next_bt = 0, issued = 0;
        int mbt0 = 0, mbt1 = 0, mbt2 = 0, mbt3 = 0;  // `issued` after the block ids of tiles j..j+3
        int last_ord = -1, gf1 = -1, gf2 = -1;
        int mk1 = 0, mk2 = 0;  // `issued` after the loads of tiles j-1 and j-2

        // One 16-byte-per-lane load covers KPI consecutive keys (lane l: key
        // l / CPR, chunk l % CPR).  When the block size is a multiple of KPI
        // those keys always share a cache block, so a load's address is a
        // wave-uniform row address plus a lane offset; load g = it*4 + p covers
        // keys g*KPI.., and with 4*KPI a multiple of the swizzle period every
        // load of this producer has the same lane offset.
        constexpr int KPI = 64 / G::CPR;
        constexpr int NPAT = (G::CPR * G::ROWS_PER_256B) / KPI;
        static_assert((kPcProducers * KPI) % (NPAT * KPI) == 0, "swizzle period");
        const bool kpi_blocks = bs % KPI == 0;
        const unsigned lane_off = (unsigned)(((lane / G::CPR) * k_ss +
                                              (((lane & (G::CPR - 1)) ^ swz<D>(p * KPI + lane / G::CPR)) * 8)) * 2);

#define LIDX_ISSUE_BT(upto)                                                                         \
        while (next_bt < n_mine && next_bt <= (upto)) {                                             \
            const int b0 = sh >= 0 ? b_s0 >> sh : b_s0 / bs;                                       \
            const int b_last = sh >= 0 ? (b_s0 + TK - 1) >> sh : (b_s0 + TK - 1) / bs;             \
            const int b_used = sh >= 0 ? (b_bd - 1) >> sh : (b_bd - 1) / bs;                       \
            const int b = min(min(b0 + lane, b_last), b_used);                                     \
            dma4(btab + (int64_t)(b_rg / gpr) * bt_stride + b, bt_mine + (next_bt % kBtRing) * 64); \
            ++issued;                                                                              \
            const int o_ = next_bt - j;                                                            \
            if (o_ == 0) mbt0 = issued;                                                            \
            else if (o_ == 1) mbt1 = issued;                                                       \
            else if (o_ == 2) mbt2 = issued;                                                       \
            else mbt3 = issued;                                                                    \
            ++next_bt;                                                                             \
            if (next_bt < n_mine) LIDX_ADVANCE(b_rg, b_ord, b_s0, b_bd, b_lo, b_hi, next_bt);      \
        }

        for (int j = 0; j < n_mine; ++j) {
            if (j > 0) LIDX_ADVANCE(k_rg, k_ord, k_s0, k_bd, k_lo, k_hi, j);
            // the block ids of tile j: already in flight except for the first
            // tile (the look-ahead loads go out behind each tile's own loads,
            // so the first tile's keys wait for one block-id load only)
            LIDX_ISSUE_BT(j);

            // the ring slot of tile j last held tile j - NBUF; a new row
            // group's q slot last held the group two back
            const bool newg = k_ord != last_ord;
            int need = j - SG::NBUF + 1;
            if (QLDS && newg && gf2 >= 0) need = max(need, gf2 + 1);
            if (need > 0) {
                for (;;) {
                    int md = lds_flag(misc + kFlagDone);
#pragma unroll
                    for (int w = 1; w < NCONS; ++w) md = min(md, lds_flag(misc + kFlagDone + w));
                    if (md >= need) break;
                    __builtin_amdgcn_s_sleep(1);
                }
                asm volatile("" ::: "memory");
            }
            const int req_k = k_rg / gpr;
            const int row0_k = req_k * Q + (k_rg - req_k * gpr) * ROWS;
            const int rhi_k = min(req_k * Q + Q, row0_k + ROWS);
            if (newg) {
                if constexpr (QLDS) {
                    // fragment f = mb*KS + kk of lane l at slot + f*1024 + l*16
                    lds_u8 *slot = qslots + (k_ord & 1) * SG::QSLOT;
                    const int head0 = ((m >> 2) & 1) * (H / 2) + (m >> 3) * 4 + (m & 3);
                    const _Float16 *src0 = qp + (int64_t)row0_k * q_st + kh * (D / 2);
#pragma unroll
                    for (int x = 0; x < SG::QL / kPcProducers; ++x) {
                        const int f = x * kPcProducers + p;
                        const int hq = nh == H ? head0 + (f / KS) * 16 : real_head(head0 + (f / KS) * 16, nh);
                        dma16(src0 + (int64_t)hq * q_sh + (f % KS) * 8, slot + f * 1024);
                    }
                    issued += SG::QL / kPcProducers;
                }
                gf2 = gf1;
                gf1 = j;
                last_ord = k_ord;
            }
            wait_vmem_below(issued - mbt0);  // block ids of tile j are in LDS

            // keys of tile j; keys past the group's bound repeat its last
            // visible key (their scores are discarded), so every address is a
            // key that exists
            {
                lds_u8 *base = keys + (j % SG::NBUF) * TILE_BYTES;
                if (kpi_blocks) {
                    const lds_i32 *bt = bt_mine + (j % kBtRing) * 64;
                    const int b0 = sh >= 0 ? k_s0 >> sh : k_s0 / bs;
                    int sk[DPT], bk[DPT], pk[DPT];
#pragma unroll
                    for (int it = 0; it < DPT; ++it) {
                        int s = k_s0 + (it * kPcProducers + p) * KPI;
                        if (s >= k_bd) s = (k_bd - 1) & ~(KPI - 1);
                        sk[it] = s;
                        bk[it] = sh >= 0 ? s >> sh : s / bs;
                        pk[it] = bt[bk[it] - b0];
                    }
#pragma unroll
                    for (int it = 0; it < DPT; ++it) {
                        const int phys = uni(pk[it]);
                        const char *row = (const char *)(kp + ((int64_t)phys * bs + (sk[it] - bk[it] * bs)) * k_ss);
                        dma16(row + lane_off, base + (it * kPcProducers + p) * 1024);
                    }
                } else {
                    const lds_i32 *bt = bt_mine + (j % kBtRing) * 64;
                    const int b0 = sh >= 0 ? k_s0 >> sh : k_s0 / bs;
#pragma unroll 4
                    for (int it = 0; it < DPT; ++it) {
                        const int c = (it * kPcProducers + p) * 64 + lane;
                        const int n = c / G::CPR;
                        const int lc = (c & (G::CPR - 1)) ^ swz<D>(n);
                        const int s = min(k_s0 + n, k_bd - 1);
                        const int blk = sh >= 0 ? s >> sh : s / bs;
                        const int64_t phys = bt[blk - b0];
                        dma16(kp + (phys * bs + (s - blk * bs)) * k_ss + lc * 8, base + (it * kPcProducers + p) * 1024);
                    }
                }
                issued += DPT;
            }
            // mask rows of tile j: load x covers rows 4x..4x+3 (lane l: row
            // l / 16, keys 8*(l % 16)..), into [row][128 keys] of the slot;
            // rows past the group repeat its first row, chunks past the last
            // column repeat the last full chunk (neither is ever used)
            if (maskp) {
                lds_u8 *mslot = mslots + (j % SG::NBUF) * SG::MSLOT;
                for (int x = p; x < SG::MROWS4; x += kPcProducers) {
                    const int r = x * 4 + (lane >> 4);
                    const int t = row0_k + r < rhi_k ? row0_k + r : row0_k;
                    const int s = min(k_s0 + (lane & 15) * 8, n_cols - 8);  // n_cols is a multiple of 8
                    dma16(maskp + (int64_t)t * mask_st + s, mslot + x * 1024);
                    ++issued;
                }
            }
            const int mk_now = issued;  // the last load of tile j
            LIDX_ISSUE_BT(j + kBtLead);
            mbt0 = mbt1;
            mbt1 = mbt2;
            mbt2 = mbt3;
            // tile j-LAG is published once it has landed
            if constexpr (SG::LAG == 1) {
                if (j > 0) {
                    wait_vmem_below(issued - mk1);
                    if (lane == 0) set_lds_flag(misc + kFlagReady + p, j);
                }
            } else {
                if (j > 1) {
                    wait_vmem_below(issued - mk2);
                    if (lane == 0) set_lds_flag(misc + kFlagReady + p, j - 1);
                }
            }
            mk2 = mk1;
            mk1 = mk_now;
        }
        if (n_mine > 0) {
            wait_vmem_all();
            if (lane == 0) set_lds_flag(misc + kFlagReady + p, n_mine);
        }
#undef LIDX_ISSUE_BT
        (void)b_ord;
    } else {
        // ================= consumers =================
        const int tg = wid / NC, col = wid - tg * NC;
        int c_rg = rg_first, c_ord = 0, c_s0 = s0_first, c_bd = bd_first, q_ord = -1;
        int c_lo = lo_first, c_hi = hi_first;
        half8 qa[MB][KS];
        int rvis[SLOTS];  // keys visible to this consumer's rows
        const_f32 *wc = (const_f32 *)wp;
        float wv[SPLIT ? MB : 1][16];
        if constexpr (SPLIT) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float w_lo, w_hi;  // uniform indices: scalar loads, batched when no head is padded
                    if (nh == H) {
                        w_lo = wc[mb * 16 + r];
                        w_hi = wc[H / 2 + mb * 16 + r];
                    } else {
                        w_lo = head_weight(wc, mb * 16 + r, nh);
                        w_hi = head_weight(wc, H / 2 + mb * 16 + r, nh);
                    }
                    wv[mb][r] = kh ? w_hi : w_lo;
                    asm volatile("" : "+v"(wv[mb][r]));  // keep in a register, not reloaded per tile
                }
        }
        // q from memory (without the LDS slots) and the visible lengths of
        // this consumer's rows, for the row group of rows row0 .. rhi-1
        auto load_q_mem = [&](int row0, int rhi) {
            if constexpr (SPLIT) {
                const int t = row0 + tg < rhi ? row0 + tg : row0;
                load_q_split<H, D, MB, KS>(qa, qp, q_st, q_sh, t, m, kh, nh);
            } else {
                load_q_rows<H, D, MB, KS>(qa, qp, q_st, q_sh, row0, rhi, tg, m, kh, nh);
            }
        };
        auto row_lengths = [&](int req_c, int row0, int rhi) {
#pragma unroll
            for (int j = 0; j < SLOTS; ++j) {
                const int tr = SPLIT ? row0 + tg : row0 + tg * TPB + 2 * j + kh;
                rvis[j] = tr < rhi ? row_vis(req_c, tr) : 0;
            }
        };
        // -inf past the last tile of every row group (shared out over the
        // workgroups; no tile writes there), while the first tile is on its way
        for (int e = blockIdx.x; e < n_rg; e += gridDim.x) {
            const int lo = (pref_at(e + 1) - pref_at(e)) * TK;
            if (lo >= n_cols) continue;
            const int req_ = e / gpr, sub_ = e - req_ * gpr;
            const int row0 = req_ * Q + sub_ * ROWS;
            const int nrows = min(req_ * Q + Q, row0 + ROWS) - row0;
            const int width = n_cols - lo;
            for (int c = tid; c < nrows * width; c += NCONS * 64) {
                const int r = c / width;
                scorep[(int64_t)(row0 + r) * score_st + lo + (c - r * width)] = -INFINITY;
            }
        }
        if constexpr (!QLDS) {
            // the first row group's q loads now, while its first tile is on its way
            if (n_mine > 0) {
                const int req_c = c_rg / gpr, sub_c = c_rg - req_c * gpr;
                const int row0 = req_c * Q + sub_c * ROWS;
                const int rhi = min(req_c * Q + Q, row0 + ROWS);
                load_q_mem(row0, rhi);
                row_lengths(req_c, row0, rhi);
                q_ord = c_ord;
            }
        }
        wait_vmem_all_known();
        for (int i = 0; i < n_mine; ++i) {
            if (i > 0) LIDX_ADVANCE(c_rg, c_ord, c_s0, c_bd, c_lo, c_hi, i);
            for (;;) {  // every producer's part of tile i has landed
                int mr = lds_flag(misc + kFlagReady);
#pragma unroll
                for (int w = 1; w < kPcProducers; ++w) mr = min(mr, lds_flag(misc + kFlagReady + w));
                if (mr > i) break;
                __builtin_amdgcn_s_sleep(1);
            }
            asm volatile("" ::: "memory");

            const int req_c = c_rg / gpr, sub_c = c_rg - req_c * gpr;
            const int row0 = req_c * Q + sub_c * ROWS;
            const int rhi = min(req_c * Q + Q, row0 + ROWS);
            int trow[SLOTS];
#pragma unroll
            for (int j = 0; j < SLOTS; ++j) trow[j] = SPLIT ? row0 + tg : row0 + tg * TPB + 2 * j + kh;
            if (c_ord != q_ord) {  // first tile of a row group: its q, its rows' lengths
                if constexpr (QLDS) {
                    const lds_u8 *slot = qslots + (c_ord & 1) * SG::QSLOT + lane * 16;
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int kk = 0; kk < KS; ++kk)
                            qa[mb][kk] = *reinterpret_cast<const lds_half8 *>(slot + (mb * KS + kk) * 1024);
                } else {
                    load_q_mem(row0, rhi);
                }
                row_lengths(req_c, row0, rhi);
                // a wait the compiler sees: otherwise it cannot tell on later
                // tiles that q has landed and waits for the score stores too
                wait_vmem_all_known();
                q_ord = c_ord;
            }
            const lds_u8 *tbase = keys + (i % SG::NBUF) * TILE_BYTES;
            const lds_u16 *mbase = (const lds_u16 *)(mslots + (i % SG::NBUF) * SG::MSLOT);

            // visibility, mask, store of the row sums of 32-key block nb
            auto store_block = [&](const float (&res)[SLOTS], int nb) {
                const int nloc = (col * NBW + nb) * 32;
                const int s = c_s0 + nloc + m;
#pragma unroll
                for (int j = 0; j < SLOTS; ++j) {
                    bool vis = s < rvis[j];
                    float add = 0.0f;
                    if (maskp) {
                        const int r = trow[j] - row0;
                        const _Float16 mv = __builtin_bit_cast(_Float16, mbase[r * TK + nloc + m]);
                        vis = vis && !half_is_neg_inf(mv);
                        add = (float)mv;
                    }
                    const float v = vis ? res[j] + add : -INFINITY;
                    if ((!SPLIT || kh == 0) && trow[j] < rhi && s < n_cols)
                        scorep[(int64_t)trow[j] * score_st + s] = v;
                }
            };

            if constexpr (SPLIT) {
                // One wave per SIMD runs this, so the matrix core, the LDS
                // and the vector ALU overlap only as far as the wave's own
                // instruction stream interleaves them.  The tile's NBW
                // blocks are one software pipeline of NBW * KS K steps:
                // step st reads the B fragment of step st + PF, issues the
                // MB products of its own fragment, and does 1/KS of the
                // epilogue of the block before (whose products are done).
                // Scheduling barriers keep that order.
                constexpr int NS = NBW * KS;   // K steps of the tile
                constexpr int PF = 3;          // fragments read ahead of their step
                constexpr int PER = MB * 16 / KS;  // epilogue terms per step
                static_assert((MB * 16) % KS == 0, "epilogue split");
                f32x16 acc[2][MB];
                half8 bq[PF + 1];
                auto frag = [&](int st) -> half8 {
                    const int n = (col * NBW + st / KS) * 32 + m;
                    return *reinterpret_cast<const lds_half8 *>(tbase + n * G::ROWB +
                                                                (((kh * KS + st % KS) ^ swz<D>(n)) << 4));
                };
#pragma unroll
                for (int st = 0; st < PF && st < NS; ++st) bq[st] = frag(st);
                // A block's head sum needs the other row half's partial sum
                // (a cross-lane move through the LDS unit); it is used two
                // steps later, so that waiting for it does not also wait for
                // the fragment reads issued behind it.
                constexpr int LATE = KS > 2 ? 2 : KS - 1;
                float sum = 0.0f, done_sum = 0.0f, other = 0.0f;
                auto store_sum = [&](int nb) {
                    const float res[SLOTS] = {done_sum + other};
                    store_block(res, nb);
                };
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    const int nb = st / KS, kk = st % KS;
                    if (st + PF < NS) bq[(st + PF) % (PF + 1)] = frag(st + PF);
                    const half8 b = bq[st % (PF + 1)];
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[nb & 1][mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            qa[mb][kk], b, kk == 0 ? f32x16{} : acc[nb & 1][mb], 0, 0, 0);
                    if (nb > 0) {
#pragma unroll
                        for (int e = kk * PER; e < (kk + 1) * PER; ++e)
                            sum = fmaf(relu(acc[(nb - 1) & 1][e / 16][e % 16]), wv[e / 16][e % 16], sum);
                        if (nb > 1 && kk == LATE) store_sum(nb - 2);
                        if (kk == KS - 1) {
                            done_sum = sum;
                            other = __shfl_xor(sum, 32, 64);
                            sum = 0.0f;
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (NBW > 1) store_sum(NBW - 2);
                // the last block's epilogue
#pragma unroll
                for (int e = 0; e < MB * 16; ++e)
                    sum = fmaf(relu(acc[(NBW - 1) & 1][e / 16][e % 16]), wv[e / 16][e % 16], sum);
                done_sum = sum;
                other = __shfl_xor(sum, 32, 64);
                store_sum(NBW - 1);
            } else {
                // general mapping (fewer than 32 heads: one M-block of
                // 32/heads rows).  The products of a 32-key block, K step by
                // K step:
                static_assert(MB == 1, "general mapping: fewer than 32 heads");
                auto mfma_block = [&](f32x16 &acc, int nb) {
                    const int n = (col * NBW + nb) * 32 + m;
                    const lds_u8 *rowp = tbase + n * G::ROWB;
                    const int f = swz<D>(n);
                    acc = f32x16{};
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk) {
                        const half8 b = *reinterpret_cast<const lds_half8 *>(rowp + (((kh * KS + kk) ^ f) << 4));
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[0][kk], b, acc, 0, 0, 0);
                    }
                };
                // two accumulator sets: block nb+1 is multiplied while block
                // nb is rectified, weighted and summed over its heads
                f32x16 accA, accB;
                mfma_block(accA, 0);
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) {
                    f32x16 &cur = (nb & 1) ? accB : accA;
                    f32x16 &nxt = (nb & 1) ? accA : accB;
                    if (nb + 1 < NBW) mfma_block(nxt, nb + 1);
                    float res[SLOTS];
#pragma unroll
                    for (int j = 0; j < SLOTS; ++j) {
                        res[j] = 0.0f;
#pragma unroll
                        for (int rr = 0; rr < 4 * G::G; ++rr)
                            res[j] = fmaf(relu(cur[4 * G::G * j + rr]), head_weight(wc, rr, nh), res[j]);
                    }
                    store_block(res, nb);
                }
            }
            // every LDS read of tile i (and of the q slot) has returned
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (lane == 0) set_lds_flag(misc + kFlagDone + wid, i + 1);
        }
        (void)c_bd;
    }
    asm volatile("" ::"v"(bt_warm));  // the warming load has returned before the wave ends
#undef LIDX_ADVANCE
}

template <int H, int D, bool SPLIT, int NC>
hipError_t launch_stream(const ScoreArgs &a, int n_req, hipStream_t stream) {
    auto kern = stream_pc_kernel<H, D, SPLIT, NC>;
    const size_t bytes = StreamGeo<H, D, SPLIT, NC>::lds_bytes();
    static std::atomic<bool> attr{false};  // per kernel instance
    if (!attr.load(std::memory_order_relaxed)) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
        if (e != hipSuccess) return e;
        attr.store(true, std::memory_order_relaxed);
    }
    hipLaunchKernelGGL(kern, dim3(device_cu_count()), dim3((kPcConsumers + kPcProducers) * 64), bytes, stream, a, n_req);
    return hipGetLastError();
}

template <int H, int D>
hipError_t launch_stream_hd(const ScoreArgs &a, const ScorePlan &p, int n_req, hipStream_t stream) {
    if constexpr (H >= 32) {  // >= 32 heads: always the split mapping
        switch (p.nc) {
            case 4: return launch_stream<H, D, true, 4>(a, n_req, stream);
            case 2: return launch_stream<H, D, true, 2>(a, n_req, stream);
            default: return launch_stream<H, D, true, 1>(a, n_req, stream);
        }
    } else {
        switch (p.nc) {
            case 4: return launch_stream<H, D, false, 4>(a, n_req, stream);
            case 2: return launch_stream<H, D, false, 2>(a, n_req, stream);
            default: return launch_stream<H, D, false, 1>(a, n_req, stream);
        }
    }
}

template <int H>
hipError_t launch_stream_h(const ScoreArgs &a, const ScorePlan &p, int D, int n_req, hipStream_t stream) {
    return D == 64 ? launch_stream_hd<H, 64>(a, p, n_req, stream) : launch_stream_hd<H, 128>(a, p, n_req, stream);
}

template <int H, int D>
hipError_t launch_hd(const ScoreArgs &a, const ScorePlan &p, bool split, hipStream_t stream) {
    if constexpr (H >= 32) {
        if (split) {
            hipLaunchKernelGGL((decode_kernel<H, D, true>), p.grid, dim3(kThreads), p.lds_bytes, stream, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((decode_kernel<H, D, false>), p.grid, dim3(kThreads), p.lds_bytes, stream, a);
    return hipGetLastError();
}

template <int H>
hipError_t launch_h(const ScoreArgs &a, const ScorePlan &p, int D, bool split, hipStream_t stream) {
    if (D == 64) return launch_hd<H, 64>(a, p, split, stream);
    if (D == 128) return launch_hd<H, 128>(a, p, split, stream);
    if constexpr (H <= 32) return launch_hd<H, 256>(a, p, split, stream);  // a pass holds 32 heads at 256
    return hipErrorInvalidValue;
}

}  // namespace

ScorePlan plan_decode(ScoreArgs &a, int n_heads, int head_dim, int n_requests) {
    ScorePlan p{};
    const int Q = a.q_per_req;
    // persistent producer/consumer kernel when its limits hold: every query
    // row of a request with >= 32 heads gets its own consumer wave (split
    // head mapping); fewer heads pack 32/heads rows per M-block
    // the mask travels in 8-key (16-byte) chunks: aligned rows, whole chunks
    const bool mask_ok = a.mask == nullptr || (a.mask_vec && a.n_cols >= 8 && a.n_cols % 8 == 0);
    // the persistent kernel runs single passes at the exact tile widths 64
    // and 128; padded head dimensions, 256 and multi-pass head groups take
    // the chunked kernel
    const bool shape_ok = head_dim <= 128 && a.head_dim == head_dim && !a.accumulate && a.add_mask;
    if (shape_ok && mask_ok && a.block_size >= 4 && n_requests <= kMaxRG) {
        const bool split = n_heads >= 32;
        const int tpb = split ? 1 : 32 / (n_heads < 16 ? n_heads : 16);
        int ng = 1;
        while (ng < 4 && ng * tpb < Q) ng *= 2;
        const int rows = ng * tpb;
        const int gpr = (Q + rows - 1) / rows;
        if ((int64_t)gpr * n_requests <= kMaxRG) {
            p.stream = true;
            p.split = split;
            p.nc = 4 / ng;
            p.rows_per_group = rows;
            p.nbw = kStreamTK / (32 * p.nc);
            p.tile_keys = kStreamTK;
            a.nc = p.nc;
            a.groups_per_req = gpr;
            a.n_row_groups = gpr * n_requests;
            a.chunk = kStreamTK;
            a.n_chunks = 1;
            p.grid = dim3((unsigned)device_cu_count());
            return p;
        }
    }
    // chunked kernel: one workgroup per (row group, key chunk)
    const bool split = Q == 1 && n_heads >= 32;
    const int hpb = n_heads < 16 ? n_heads : 16;
    const int tpb = split ? 1 : 32 / hpb;
    int ng = 1;
    while (ng < kWaves && ng * tpb < Q) ng *= 2;
    if (split) ng = 1;
    p.nc = kWaves / ng;
    p.rows_per_group = ng * tpb;
    p.split = split;
    a.nc = p.nc;
    a.groups_per_req = (Q + p.rows_per_group - 1) / p.rows_per_group;
    a.n_row_groups = a.groups_per_req * n_requests;
    p.nbw = 1;
    p.tile_keys = 32 * p.nc;
    const int max_tiles_lds = kChunkBytes / (p.tile_keys * 2 * head_dim);
    const int tiles = max_tiles_lds < kMaxTiles ? max_tiles_lds : kMaxTiles;
    a.chunk = tiles * p.tile_keys;
    a.n_chunks = (a.n_cols + a.chunk - 1) / a.chunk;
    if (a.n_chunks < 1) a.n_chunks = 1;
    p.lds_bytes = (size_t)a.chunk * 2 * head_dim + 4 * ((size_t)(a.chunk + a.block_size - 1) / a.block_size + 2) + 16;
    p.grid = dim3((unsigned)(a.n_row_groups * a.n_chunks));
    return p;
}

hipError_t launch_decode(const ScoreArgs &a, const ScorePlan &p, int n_heads, int head_dim, hipStream_t stream) {
    const int n_req = a.n_row_groups / (a.groups_per_req > 0 ? a.groups_per_req : 1);
    if (p.stream) {
        switch (n_heads) {
            case 4: return launch_stream_h<4>(a, p, head_dim, n_req, stream);
            case 8: return launch_stream_h<8>(a, p, head_dim, n_req, stream);
            case 16: return launch_stream_h<16>(a, p, head_dim, n_req, stream);
            case 32: return launch_stream_h<32>(a, p, head_dim, n_req, stream);
            default: return launch_stream_h<64>(a, p, head_dim, n_req, stream);
        }
    }
    switch (n_heads) {
        case 4: return launch_h<4>(a, p, head_dim, p.split, stream);
        case 8: return launch_h<8>(a, p, head_dim, p.split, stream);
        case 16: return launch_h<16>(a, p, head_dim, p.split, stream);
        case 32: return launch_h<32>(a, p, head_dim, p.split, stream);
        default: return launch_h<64>(a, p, head_dim, p.split, stream);
    }
}

}  // namespace lidx
