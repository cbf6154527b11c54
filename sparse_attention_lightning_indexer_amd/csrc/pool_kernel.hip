// Pooled-key producer for gfx950: the keys the indexer scores.
//
// The llama.cpp b11372 notes ("qwen4exp: compute the indexer score with the
// lightning indexer") run the lightning indexer on the pooled keys, and do
// not say how the keys are pooled.  The reading implemented here is mean
// pooling over consecutive windows: pooled key p of n_keys keys is the
// element-wise mean of keys [p * pool, min((p + 1) * pool, n_keys)), so a
// short last window averages the keys it holds.
//
// Arithmetic: every f16 key element widens exactly to f64, and the sum of at
// most 8192 of them is exact in f64 (f16 values span 2^-24 .. 2^16, 40
// bits, plus 13 bits of carries fit the 53-bit significand); one f64
// division by the window's key count (correctly rounded) and one rounding to
// the nearest f16 (ties to even) follow.  The result is therefore the f16
// nearest the exact mean's f64 rounding, whatever the order of the sum.
//
// HBM-bound: each thread owns one 16-byte chunk (8 elements) of one pooled
// key and streams the window's chunks; the 64 lanes of a wave cover whole
// key rows, so every load instruction reads full 256-byte rows of the window.
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace lidx {
namespace {

constexpr int kPoolThreads = 256;

// Round an f64 to the nearest binary16 (ties to even) straight from f64, with
// no intermediate f32 rounding.  Finite magnitudes below 2^-14 are subnormal
// f16 multiples of 2^-24; at or above 65520 (the halfway point past the
// largest f16, 65504) the result is infinite.
__device__ __forceinline__ unsigned short f64_to_f16_rne(double x) {
    const unsigned long long bits = __builtin_bit_cast(unsigned long long, x);
    const unsigned short sign = (unsigned short)((bits >> 48) & 0x8000u);
    const double a = fabs(x);
    if (a != a) return (unsigned short)(sign | 0x7e00u);         // NaN
    if (a >= 65520.0) return (unsigned short)(sign | 0x7c00u);   // overflow (and inf)
    if (a < 0x1p-14) {
        // subnormal range: the nearest multiple of 2^-24 (rint: ties to even;
        // scaling by a power of two is exact); 1024 * 2^-24 is 2^-14, whose
        // bits (exponent field 1, fraction 0) are the same integer
        return (unsigned short)(sign | (unsigned short)rint(a * 0x1p24));
    }
    int e;
    (void)frexp(a, &e);  // a = f * 2^e, f in [0.5, 1): the unbiased exponent is e - 1
    e -= 1;
    double q = rint(ldexp(a, 10 - e));  // 11 significant bits: q in [1024, 2048]
    if (q >= 2048.0) {                  // rounded up to the next binade
        q = 1024.0;
        e += 1;
    }
    return (unsigned short)(sign | (unsigned short)((e + 15) << 10) | (unsigned short)((int)q - 1024));
}

__global__ void __launch_bounds__(kPoolThreads) pool_keys_kernel(const _Float16 *k, int64_t k_ss, int n_keys, int cpr,
                                                                  int pool, _Float16 *out, int64_t out_ss, int n_pool) {
    const int64_t g = (int64_t)blockIdx.x * kPoolThreads + threadIdx.x;
    const int64_t p = g / cpr;
    const int c = (int)(g - p * cpr);
    if (p >= n_pool) return;
    const int64_t s0 = p * pool;
    const int64_t s1 = min(s0 + pool, (int64_t)n_keys);
    double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    const _Float16 *src = k + s0 * k_ss + c * 8;
    int64_t s = s0;
    // four rows of the window in flight per step
    for (; s + 4 <= s1; s += 4) {
        half8 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const half8 *>(src + (s - s0 + u) * k_ss);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += (double)v[u][e];
    }
    for (; s < s1; ++s) {
        const half8 v = *reinterpret_cast<const half8 *>(src + (s - s0) * k_ss);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += (double)v[e];
    }
    const double cnt = (double)(s1 - s0);
    unsigned short h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = f64_to_f16_rne(acc[e] / cnt);
    uint4 o;
    o.x = h[0] | ((unsigned int)h[1] << 16);
    o.y = h[2] | ((unsigned int)h[3] << 16);
    o.z = h[4] | ((unsigned int)h[5] << 16);
    o.w = h[6] | ((unsigned int)h[7] << 16);
    *reinterpret_cast<uint4 *>(out + p * out_ss + c * 8) = o;
}

}  // namespace

int pooled_count(int n_keys, int pool) { return n_keys <= 0 ? 0 : (int)(((int64_t)n_keys + pool - 1) / pool); }

hipError_t launch_pool(const _Float16 *k, int64_t k_ss, int n_keys, int head_dim, int pool, _Float16 *out,
                       int64_t out_ss, hipStream_t stream) {
    const int n_pool = pooled_count(n_keys, pool);
    if (n_pool == 0) return hipSuccess;
    const int cpr = head_dim / 8;
    const int64_t threads = (int64_t)n_pool * cpr;
    const unsigned grid = (unsigned)((threads + kPoolThreads - 1) / kPoolThreads);
    hipLaunchKernelGGL(pool_keys_kernel, dim3(grid), dim3(kPoolThreads), 0, stream, k, k_ss, n_keys, cpr, pool, out,
                       out_ss, n_pool);
    return hipGetLastError();
}

}  // namespace lidx
