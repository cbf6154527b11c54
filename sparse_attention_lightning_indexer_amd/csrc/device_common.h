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
    static_assert(D == 64 || D == 128 || D == 256, "head dim");
    static constexpr int HPB = H < 16 ? H : 16;   // heads per M-block
    static constexpr int TPB = 32 / HPB;          // query rows per M-block
    static constexpr int MBLK = H / HPB;          // M-blocks covering all heads
    static constexpr int G = HPB / 4;             // 4-register groups per row slot
    static constexpr int SLOTS = 4 / G;           // query rows held by one lane
    static constexpr int KSTEPS = D / 16;         // MFMA K steps
    static constexpr int CPR = D / 8;             // 16-byte chunks per key row
    static constexpr int ROWB = 2 * D;            // bytes per key row in LDS
    static constexpr int ROWS_PER_256B = ROWB < 256 ? 256 / ROWB : 1;
    static constexpr int SWZ_MASK = CPR < 16 ? CPR - 1 : 15;
};

// Swizzled position of a key row's 16-byte chunk in LDS: the chunk index is
// XORed with a function of the row so that the rows read by one 16-lane
// phase land in distinct 16-byte bank groups (the 64 banks span 256 bytes;
// 16 consecutive rows of 128, 256 or 512 bytes then hit 16 different groups).
template <int D>
__device__ __forceinline__ int swz(int n) {
    return (n / Geo<4, D>::ROWS_PER_256B) & Geo<4, D>::SWZ_MASK;
}

// Sixteen zero bytes in device memory: the source of the key chunks past a
// head dimension that is shorter than the compiled tile (its q chunks are
// zero too, so the padded part of every dot product is exactly 0).
static __device__ __attribute__((aligned(16))) const unsigned int kZeroChunk[4] = {0u, 0u, 0u, 0u};

// A value the caller knows to be the same in every lane (an LDS word read at
// a uniform address, say), moved to a scalar register so that the arithmetic
// and branches that depend on it run on the scalar unit.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Head counts below the compiled tile run as the next compiled count: the
// extra heads read a real head's q (any finite values do) and weigh zero, so
// they add exactly nothing to the score.
__device__ __forceinline__ int real_head(int head, int n_heads) { return head < n_heads ? head : n_heads - 1; }
__device__ __forceinline__ float head_weight(const __attribute__((address_space(4))) float *w, int head, int n_heads) {
    const float v = w[real_head(head, n_heads)];
    return head < n_heads ? v : 0.0f;
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

// Wave-level sums, extrema and scans through DPP lane moves (VALU
// operations; a 64-lane shuffle would take an LDS round trip per step).
// Reductions: swap within quads, then mirror within half rows and rows, so
// every lane of a 16-lane row holds the row's value; the four rows are then
// combined from lanes 0, 16, 32 and 48 (a wave-uniform result).
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ int dpp_move(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xf, false);
}
template <typename OP>
__device__ __forceinline__ int row_reduce(int v, int identity, OP op) {
    v = op(v, dpp_move<0xb1>(identity, v));   // quad_perm [1,0,3,2]
    v = op(v, dpp_move<0x4e>(identity, v));   // quad_perm [2,3,0,1]
    v = op(v, dpp_move<0x141>(identity, v));  // row_half_mirror
    v = op(v, dpp_move<0x140>(identity, v));  // row_mirror
    return v;
}
__device__ __forceinline__ int wave_sum(int v) {
    v = row_reduce(v, 0, [](int a, int b) { return a + b; });
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
           __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t u) {
    const int v = row_reduce((int)u, 0, [](int a, int b) { return (int)max((uint32_t)a, (uint32_t)b); });
    return max(max((uint32_t)__builtin_amdgcn_readlane(v, 0), (uint32_t)__builtin_amdgcn_readlane(v, 16)),
               max((uint32_t)__builtin_amdgcn_readlane(v, 32), (uint32_t)__builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t u) {
    const int v = row_reduce((int)u, -1, [](int a, int b) { return (int)min((uint32_t)a, (uint32_t)b); });
    return min(min((uint32_t)__builtin_amdgcn_readlane(v, 0), (uint32_t)__builtin_amdgcn_readlane(v, 16)),
               min((uint32_t)__builtin_amdgcn_readlane(v, 32), (uint32_t)__builtin_amdgcn_readlane(v, 48)));
}
// Inclusive prefix sum inside each 16-lane row (shifts by 1, 2, 4 and 8).
__device__ __forceinline__ int row_incl_scan(int v) {
    v += dpp_move<0x111>(0, v);  // row_shr:1
    v += dpp_move<0x112>(0, v);  // row_shr:2
    v += dpp_move<0x114>(0, v);  // row_shr:4
    v += dpp_move<0x118>(0, v);  // row_shr:8
    return v;
}
// Inclusive prefix sum over the wave's lanes: shifts by 1, 2, 4 and 8 inside
// each 16-lane row, then the end of row 0 (and 2) into row 1 (and 3), then
// the end of row 1 into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += dpp_move<0x111>(0, v);       // row_shr:1
    v += dpp_move<0x112>(0, v);       // row_shr:2
    v += dpp_move<0x114>(0, v);       // row_shr:4
    v += dpp_move<0x118>(0, v);       // row_shr:8
    v += dpp_move<0x142, 0xa>(0, v);  // row_bcast:15
    v += dpp_move<0x143, 0xc>(0, v);  // row_bcast:31
    return v;
}

__device__ __forceinline__ void wait_vmem_all() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// s_waitcnt vmcnt(0) through the builtin: the compiler's own wait insertion
// sees it and knows that every earlier load into registers has completed, so
// it adds no waits of its own before their later uses.
__device__ __forceinline__ void wait_vmem_all_known() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) expcnt(7) lgkmcnt(15)
}

// Workgroup barrier ordering LDS accesses only.  __syncthreads() carries a
// workgroup-scope release fence, and the compiler counts direct-to-LDS loads
// as pending LDS writes under that fence: it would wait for every load in
// flight (vmcnt(0)) at each barrier and drain the load pipelines.  Kernels
// that use this barrier wait for their direct-to-LDS loads explicitly.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Wait until at most n vector-memory operations of this wave are pending.
// Loads complete in issue order, so this waits for everything but the n most
// recent loads.  n is wave-uniform; every count the 6-bit counter can hold
// (0..63) is exact, larger ones wait for 63.
__device__ __forceinline__ void wait_vmem_below(int n) {
#define LIDX_W(N) \
    case N: asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory"); break;
    switch (n < 0 ? 0 : (n > 63 ? 63 : n)) {
        LIDX_W(0) LIDX_W(1) LIDX_W(2) LIDX_W(3) LIDX_W(4) LIDX_W(5) LIDX_W(6) LIDX_W(7)
        LIDX_W(8) LIDX_W(9) LIDX_W(10) LIDX_W(11) LIDX_W(12) LIDX_W(13) LIDX_W(14) LIDX_W(15)
        LIDX_W(16) LIDX_W(17) LIDX_W(18) LIDX_W(19) LIDX_W(20) LIDX_W(21) LIDX_W(22) LIDX_W(23)
        LIDX_W(24) LIDX_W(25) LIDX_W(26) LIDX_W(27) LIDX_W(28) LIDX_W(29) LIDX_W(30) LIDX_W(31)
        LIDX_W(32) LIDX_W(33) LIDX_W(34) LIDX_W(35) LIDX_W(36) LIDX_W(37) LIDX_W(38) LIDX_W(39)
        LIDX_W(40) LIDX_W(41) LIDX_W(42) LIDX_W(43) LIDX_W(44) LIDX_W(45) LIDX_W(46) LIDX_W(47)
        LIDX_W(48) LIDX_W(49) LIDX_W(50) LIDX_W(51) LIDX_W(52) LIDX_W(53) LIDX_W(54) LIDX_W(55)
        LIDX_W(56) LIDX_W(57) LIDX_W(58) LIDX_W(59) LIDX_W(60) LIDX_W(61) LIDX_W(62) LIDX_W(63)
        default: break;
    }
#undef LIDX_W
}

// LDS pointer types with the address space spelled out, so that LDS accesses
// are never lowered to flat accesses (which would also count in vmcnt).
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) int lds_i32;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) half8 lds_half8;

__device__ __forceinline__ void dma16(const void *src, void *lds) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

__device__ __forceinline__ void dma16(const void *src, lds_u8 *lds) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

__device__ __forceinline__ void dma4(const void *src, lds_i32 *lds) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 4, 0, 0);
}

}  // namespace lidx
