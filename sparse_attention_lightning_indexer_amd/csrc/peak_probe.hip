// Achievable-peak probes for gfx950: what the chip sustains for the two
// bounds the indexer kernels are measured against, next to the published
// peaks.  Measurement helpers only; nothing of the indexer's arithmetic.
// Built into its own library, libpeak_probe.so, which only the benchmark and
// its test load; the indexer library does not contain or export it.
//
// C-ABI (all launches asynchronous on `stream`, a hipStream_t; the caller
// times them with events on that stream):
//   int32_t peak_probe_sink_floats(void)
//       floats of the `sink` device buffer both probes take (written only in
//       a case that never occurs).
//   int peak_probe_mfma(int32_t iters, float *sink, double *flops, void *stream)
//       2 workgroups of 256 threads per compute unit, each wave running
//       iters x 128 v_mfma_f32_32x32x16_f16; *flops receives the f16 flops
//       of the launch.  Returns 1 for iters < 1 or a NULL pointer, 4 when the
//       launch fails, else 0.
//   int peak_probe_read(const void *buf, size_t bytes, float *sink, void *stream)
//       one streaming read of `bytes` (a positive multiple of 16) at `buf`
//       (device, 16-byte aligned).  Returns 1 for a bad pointer, alignment or
//       size, 4 when the launch fails, else 0.
//
//   int peak_probe_empty(int32_t blocks, int32_t threads, void *stream)
//       a kernel that does nothing, on `blocks` workgroups of `threads`
//       (1..1024) threads: the fixed cost of one launch.  Returns 1 for bad
//       sizes, 4 when the launch fails, else 0.
//   int peak_probe_rows(const float *rows, int64_t stride, const int32_t *lens,
//                       int32_t n_rows, int32_t row_len, int32_t k, float *val,
//                       int32_t *idx, void *stream)
//       the memory movement of a row-wise selection without the selection:
//       one 1024-thread workgroup per row reads the row's first lens[r]
//       floats (row_len when lens is NULL; clamped to 0..row_len), takes one
//       block-wide maximum and writes k values (the row's first k, capped
//       at the maximum) and k indices.  rows is [n_rows][stride] (device,
//       stride >= row_len), val and idx are [n_rows][k] (device).  Returns 1
//       for bad pointers or sizes (row_len and k at most 16384), 4 when the
//       launch fails, else 0.
//
//  * probe_mfma_kernel: v_mfma_f32_32x32x16_f16 fed the way the score
//    kernels feed it -- A fragments in registers, one 16-byte B fragment per
//    lane read from XOR-swizzled LDS rows per K step, shared by four M-blocks
//    (four independent accumulators), the next two fragments in flight.  Two
//    workgroups of four waves per compute unit (two waves per SIMD).  The
//    operands are pseudo-random f16 values (every mantissa bit in play):
//    the sustained rate depends on the data, and near-constant operands run
//    about a quarter faster than the N(0,1)-like q and keys of real inputs.
//  * probe_read_kernel: a large streaming read, 16 bytes per lane per load,
//    eight workgroups of 256 threads per compute unit.
// Both keep their results live through a store that never happens.
#include "device_common.h"

namespace lidx {
namespace {

constexpr int kProbeMB = 4;      // accumulators fed by one B fragment
constexpr int kProbeBlocks = 4;  // 32-key blocks per LDS tile
constexpr int kProbePF = 2;      // B fragments in flight

// A pseudo-random f16 in [-2, 2) from a 32-bit counter (an integer hash
// whose output bits all depend on every input bit).
__device__ __forceinline__ _Float16 probe_value(uint32_t x) {
    x *= 0x9e3779b1u;
    x ^= x >> 15;
    x *= 0x85ebca77u;
    x ^= x >> 13;
    return (_Float16)((float)(x >> 8) * (4.0f / 16777216.0f) - 2.0f);
}

__global__ void __launch_bounds__(256, 2) probe_mfma_kernel(int iters, float *sink) {
    __shared__ __attribute__((aligned(16))) unsigned char tile[kProbeBlocks * 32 * 256];
    const int lane = threadIdx.x & 63, m = lane & 31, kh = lane >> 5;
    const uint32_t seed = (uint32_t)blockIdx.x * 0x10000u;
    for (int i = threadIdx.x; i < (int)sizeof(tile) / 2; i += 256)
        ((_Float16 *)tile)[i] = probe_value(seed + (uint32_t)i);
    __syncthreads();
    half8 a[kProbeMB][8];
#pragma unroll
    for (int mb = 0; mb < kProbeMB; ++mb)
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                a[mb][kk][e] = probe_value(seed + 0x8000u + (uint32_t)(((mb * 8 + kk) * 64 + lane) * 8 + e));
    f32x16 acc[kProbeMB];
#pragma unroll
    for (int mb = 0; mb < kProbeMB; ++mb) acc[mb] = f32x16{};
    // byte offset of this lane's fragment for K step kk inside a 32-key block
    // (the row stays m, so the swizzle term is the same for every block)
    int off[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) off[kk] = m * 256 + (((kh * 8 + kk) ^ (m & 15)) << 4);
    auto frag = [&](int blk, int kk) {
        return *(const lds_half8 *)(tile + blk * 8192 + off[kk]);
    };
    for (int it = 0; it < iters; ++it) {
        // the tile is not written in the loop: without this the compiler
        // would hoist every fragment read out of it into registers
        asm volatile("" ::: "memory");
#pragma unroll
        for (int blk = 0; blk < kProbeBlocks; ++blk) {
            half8 bq[kProbePF];
#pragma unroll
            for (int p = 0; p < kProbePF; ++p) bq[p] = frag(blk, p);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const half8 b = bq[kk % kProbePF];
                if (kk + kProbePF < 8) bq[kk % kProbePF] = frag(blk, kk + kProbePF);
#pragma unroll
                for (int mb = 0; mb < kProbeMB; ++mb)
                    acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[mb][kk], b, acc[mb], 0, 0, 0);
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int mb = 0; mb < kProbeMB; ++mb) s += acc[mb][lane & 15];
    if (s == 1.2345e-30f) sink[blockIdx.x] = s;
}

__global__ void __launch_bounds__(256) probe_read_kernel(const float4 *p, size_t n, float *sink) {
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
        const float4 v = p[i];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    if (acc.x + acc.y + acc.z + acc.w == 1.2345e-30f) sink[blockIdx.x] = acc.x;
}

__global__ void probe_empty_kernel() {}

constexpr int kRowsE = 16;  // row elements per thread (rows of up to 16384)

__global__ void __launch_bounds__(1024) probe_rows_kernel(const float *rows, int64_t stride, const int32_t *lens,
                                                          int row_len, int k, float *val, int32_t *idx) {
    __shared__ float wmax[16];
    const int r = blockIdx.x, tid = threadIdx.x;
    const int len = lens ? min(max(lens[r], 0), row_len) : row_len;
    const float *p = rows + (int64_t)r * stride;
    float x[kRowsE];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < kRowsE; ++e) {
        const int i = tid + e * 1024;
        x[e] = i < len ? p[i] : -INFINITY;
        mx = fmaxf(mx, x[e]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if ((tid & 63) == 0) wmax[tid >> 6] = mx;
    __syncthreads();
    float bm = wmax[0];
#pragma unroll
    for (int w = 1; w < 16; ++w) bm = fmaxf(bm, wmax[w]);
#pragma unroll
    for (int e = 0; e < kRowsE; ++e) {
        const int j = tid + e * 1024;
        if (j < k) {
            val[(int64_t)r * k + j] = fminf(x[e], bm);
            idx[(int64_t)r * k + j] = j;
        }
    }
}

int cu_count() {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return 256;
    return v;
}

}  // namespace
}  // namespace lidx

extern "C" {

int32_t peak_probe_sink_floats(void) { return 8 * lidx::cu_count(); }

int peak_probe_mfma(int32_t iters, float *sink, double *flops, void *stream) {
    if (iters < 1 || !sink || !flops) return 1;
    const int grid = 2 * lidx::cu_count();
    hipLaunchKernelGGL(lidx::probe_mfma_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters, sink);
    *flops = (double)grid * 4 /*waves*/ * iters * lidx::kProbeBlocks * 8 * lidx::kProbeMB * (32.0 * 32 * 16 * 2);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int peak_probe_read(const void *buf, size_t bytes, float *sink, void *stream) {
    if (!buf || !sink || ((uintptr_t)buf % 16) || bytes % 16 || bytes == 0) return 1;
    const int grid = 8 * lidx::cu_count();
    hipLaunchKernelGGL(lidx::probe_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (const float4 *)buf, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int peak_probe_empty(int32_t blocks, int32_t threads, void *stream) {
    if (blocks < 1 || threads < 1 || threads > 1024) return 1;
    hipLaunchKernelGGL(lidx::probe_empty_kernel, dim3(blocks), dim3(threads), 0, (hipStream_t)stream);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int peak_probe_rows(const float *rows, int64_t stride, const int32_t *lens, int32_t n_rows, int32_t row_len,
                    int32_t k, float *val, int32_t *idx, void *stream) {
    if (!rows || !val || !idx || n_rows < 1 || row_len < 0 || row_len > 1024 * lidx::kRowsE || stride < row_len ||
        k < 1 || k > 1024 * lidx::kRowsE)
        return 1;
    hipLaunchKernelGGL(lidx::probe_rows_kernel, dim3(n_rows), dim3(1024), 0, (hipStream_t)stream, rows, stride,
                       lens, row_len, k, val, idx);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
