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
            const _Float16 *src = a.q + (int64_t)t * a.q_st + (int64_t)head * a.q_sh + kh * (D / 2);
#pragma unroll
            for (int kk = 0; kk < G::KSTEPS; ++kk)
                qa[mb][kk] = ok ? *reinterpret_cast<const half8 *>(src + kk * 8) : half8{};
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
            for (int r = 0; r < 16; ++r) wv[mb][r] = a.w[kh * (H / 2) + mb * 16 + r];
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
                    if (vis[0]) res[i][0] = sum + (float)mv[i][0];
                } else {
#pragma unroll
                    for (int j = 0; j < SLOTS; ++j) {
                        float sum = 0.0f;
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                            for (int rr = 0; rr < 4 * G::G; ++rr)
                                sum = fmaf(relu(acc[mb][4 * G::G * j + rr]), wc[mb * G::HPB + rr], sum);
                        if (vis[j]) res[i][j] = sum + (float)mv[i][j];
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
                if (out_t[j] < row_hi && (!SPLIT || kh == 0))
                    a.score[(int64_t)out_t[j] * a.score_st + s] = res[i][j];
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
    return D == 64 ? launch_hd<H, 64>(a, p, split, stream) : launch_hd<H, 128>(a, p, split, stream);
}

}  // namespace

ScorePlan plan_decode(ScoreArgs &a, int n_heads, int head_dim, int n_requests) {
    ScorePlan p{};
    const int Q = a.q_per_req;
    const bool split = Q == 1 && n_heads >= 32;
    const int hpb = n_heads < 16 ? n_heads : 16;
    const int tpb = split ? 1 : 32 / hpb;
    int ng = 1;
    while (ng < kWaves && ng * tpb < Q) ng *= 2;
    if (split) ng = 1;
    p.nc = kWaves / ng;
    p.nbw = 1;
    p.tile_keys = 32 * p.nc;
    p.rows_per_group = ng * tpb;
    p.split = split;
    a.nc = p.nc;
    a.groups_per_req = (Q + p.rows_per_group - 1) / p.rows_per_group;
    a.n_row_groups = a.groups_per_req * n_requests;
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
    switch (n_heads) {
        case 4: return launch_h<4>(a, p, head_dim, p.split, stream);
        case 8: return launch_h<8>(a, p, head_dim, p.split, stream);
        case 16: return launch_h<16>(a, p, head_dim, p.split, stream);
        case 32: return launch_h<32>(a, p, head_dim, p.split, stream);
        default: return launch_h<64>(a, p, head_dim, p.split, stream);
    }
}

}  // namespace lidx
