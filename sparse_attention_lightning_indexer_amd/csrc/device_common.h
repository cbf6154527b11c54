// Device helpers shared by the score kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lidx {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Per-head weights are read through the constant address space so that they
// load with scalar instructions and feed the epilogue FMAs as SGPR operands.
typedef const __attribute__((address_space(4))) float const_f32;
typedef const __attribute__((address_space(4))) int32_t const_i32;

// Geometry of one MFMA M-block (32 rows) for a head count H: the rows are
// HPB heads of TPB query rows, arranged so that accumulator register r of a
// lane always holds one head (see the row maps in the kernels).
template <int H, int D>
struct Geo {
    static_assert(H == 4 || H == 8 || (H % 16 == 0 && H <= 64), "head count");
    static_assert(D == 64 || D == 128, "head dim");
    static constexpr int HPB = H < 16 ? H : 16;   // heads per M-block
    static constexpr int TPB = 32 / HPB;          // query rows per M-block
    static constexpr int MBLK = H / HPB;          // M-blocks covering all heads
    static constexpr int G = HPB / 4;             // 4-register groups per row slot
    static constexpr int SLOTS = 4 / G;           // query rows held by one lane
    static constexpr int KSTEPS = D / 16;         // MFMA K steps
    static constexpr int CPR = D / 8;             // 16-byte chunks per key row
    static constexpr int ROWB = 2 * D;            // bytes per key row in LDS
    static constexpr int ROWS_PER_256B = 256 / ROWB;
};

// Swizzled position of a key row's 16-byte chunk in LDS: the chunk index is
// XORed with a function of the row so that the rows read by one 16-lane
// phase land in distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int swz(int n) {
    return (n / Geo<4, D>::ROWS_PER_256B) & (Geo<4, D>::CPR - 1);
}

__device__ __forceinline__ bool half_is_neg_inf(_Float16 h) {
    return __builtin_bit_cast(unsigned short, h) == 0xfc00u;
}

// max(x, 0) as one integer max on the bit pattern: a negative float (or -0)
// is a negative int32 and becomes +0; a non-negative float is unchanged.  One
// v_max_i32 per accumulator (fmaxf would add a NaN-quieting v_max first).
// Inline asm is avoided on purpose: the hazard checks between MFMA results
// and their VALU readers only see compiler-visible instructions.
__device__ __forceinline__ float relu(float x) {
    return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

__device__ __forceinline__ void wait_vmem_all() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Wait until at most n vector-memory operations of this wave are pending.
// Loads complete in issue order, so this waits for everything but the n most
// recent loads.  n is rounded down to an encodable step (waiting longer is
// always safe).
__device__ __forceinline__ void wait_vmem_below(int n) {
#define LIDX_WAIT(N) asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory")
    if (n >= 48) LIDX_WAIT(48);
    else if (n >= 32) LIDX_WAIT(32);
    else if (n >= 24) LIDX_WAIT(24);
    else if (n >= 16) LIDX_WAIT(16);
    else if (n >= 12) LIDX_WAIT(12);
    else if (n >= 8) LIDX_WAIT(8);
    else if (n >= 6) LIDX_WAIT(6);
    else if (n >= 4) LIDX_WAIT(4);
    else if (n >= 3) LIDX_WAIT(3);
    else if (n >= 2) LIDX_WAIT(2);
    else if (n >= 1) LIDX_WAIT(1);
    else LIDX_WAIT(0);
#undef LIDX_WAIT
}

__device__ __forceinline__ void dma16(const void *src, void *lds) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

}  // namespace lidx
