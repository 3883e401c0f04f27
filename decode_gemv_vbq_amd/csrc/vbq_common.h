// Shared device helpers for the VBQ1 layout (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "vbq.h"

namespace vbq {

constexpr uint32_t kMagic = 0x31514256u;
constexpr int kGroup = 64;      // weights per group
constexpr int kSlice = 32;      // groups per K-slice
constexpr int kRowPad = 128;    // row record padding, bytes

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

struct __attribute__((aligned(8))) U2 {
    uint32_t v[2];
};
struct __attribute__((aligned(8))) U4 {
    uint32_t v[4];
};

__device__ __forceinline__ uint32_t lo_plane(const uint32_t *wmap, uint64_t rs) { return wmap[2 * rs]; }
__device__ __forceinline__ uint32_t hi_plane(const uint32_t *wmap, uint64_t rs) { return wmap[2 * rs + 1]; }

// Masks of the groups of one row-slice whose width code (log2 b) is c.
struct WidthMasks {
    uint32_t m[4];
};

__device__ __forceinline__ WidthMasks width_masks(uint32_t p0, uint32_t p1, int ng)
{
    uint32_t valid = ng >= 32 ? 0xffffffffu : ((1u << ng) - 1u);
    WidthMasks w;
    w.m[0] = ~p0 & ~p1 & valid;
    w.m[1] = p0 & ~p1 & valid;
    w.m[2] = ~p0 & p1 & valid;
    w.m[3] = p0 & p1 & valid;
    return w;
}

// Element c of a 4-array without dynamic register indexing (no scratch).
template <typename T>
__device__ __forceinline__ T pick4(const T *v, int c)
{
    return c == 0 ? v[0] : c == 1 ? v[1] : c == 2 ? v[2] : v[3];
}

// Byte offset, inside its slice record, of group gi (0..31) of width code c.
__device__ __forceinline__ uint32_t group_offset_in_slice(const WidthMasks &w, int c, int gi)
{
    uint32_t units = 0; // 8-byte units
#pragma unroll
    for (int cc = 0; cc < 4; cc++)
        if (cc < c)
            units += (uint32_t)__popc(w.m[cc]) << cc;
    units += (uint32_t)__popc(pick4(w.m, c) & ((1u << gi) - 1u)) << c;
    return units * 8u;
}

__device__ __forceinline__ int width_code(uint32_t p0, uint32_t p1, int gi)
{
    return (int)((p0 >> gi) & 1u) | (int)(((p1 >> gi) & 1u) << 1);
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane
// (m0 = lds_base, wave-uniform).  Written as asm so the compiler does not tie
// later LDS reads to it with a full vmcnt wait: completion is awaited
// explicitly (wait_vm / wait_vm0) before the barrier that publishes the data.
// The leading s_nop separates the compiler's m0 write from the LDS-DMA load.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds_base)
{
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory");
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// s_waitcnt vmcnt(n) for a run-time n (clamped: a smaller n only waits longer).
__device__ __forceinline__ void wait_vm(int n)
{
    switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    }
}

} // namespace vbq
