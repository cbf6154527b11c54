// Achievable-peak probes for gfx950: what the chip sustains for the two
// bounds the indexer kernels are measured against, next to the published
// peaks.  Measurement helpers only; nothing of the indexer's arithmetic.
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
#include "internal.h"

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

}  // namespace

hipError_t launch_probe_mfma(int iters, float *sink, double *flops, hipStream_t stream) {
    const int grid = 2 * device_cu_count();
    hipLaunchKernelGGL(probe_mfma_kernel, dim3(grid), dim3(256), 0, stream, iters, sink);
    *flops = (double)grid * 4 /*waves*/ * iters * kProbeBlocks * 8 * kProbeMB * (32.0 * 32 * 16 * 2);
    return hipGetLastError();
}

hipError_t launch_probe_read(const void *buf, size_t bytes, float *sink, hipStream_t stream) {
    const int grid = 8 * device_cu_count();
    hipLaunchKernelGGL(probe_read_kernel, dim3(grid), dim3(256), 0, stream, (const float4 *)buf, bytes / 16, sink);
    return hipGetLastError();
}

int probe_sink_floats() { return 8 * device_cu_count(); }

}  // namespace lidx
