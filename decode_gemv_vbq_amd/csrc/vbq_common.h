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

// v from another lane of the same DPP row (ctrl: a DPP control code).
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}

// v of the lane 16 (x16) or 32 (x32) lanes away, by the gfx950 lane swaps
// (VALU, no LDS round trip as a lane shuffle would take): v_permlane16_swap
// of v with itself gives the 16-lane rows (0, 0, 2, 2) and (1, 1, 3, 3),
// v_permlane32_swap gives (0, 1, 0, 1) and (2, 3, 2, 3).
__device__ __forceinline__ float lanes_x16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float lanes_x32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Sum of v over each aligned group of L lanes (L = 8, 16, 32, 64), the same
// value in every lane of the group, in a fixed order: pairs and quads (DPP
// quad permutations), then the two quads of each 8 lanes (row_half_mirror:
// once every lane of a quad holds the quad's sum, the mirrored lane holds the
// other quad's), then the two halves of each 16-lane row (row_mirror), then
// across rows (lanes_x16, lanes_x32).  No lane move goes through LDS.
template <int L>
__device__ __forceinline__ float group_sum(float v)
{
    v += dpp_f<0xB1>(v);  // quad_perm [1, 0, 3, 2]
    v += dpp_f<0x4E>(v);  // quad_perm [2, 3, 0, 1]
    v += dpp_f<0x141>(v); // row_half_mirror
    if (L >= 16)
        v += dpp_f<0x140>(v); // row_mirror
    if (L >= 32)
        v += lanes_x16(v);
    if (L >= 64)
        v += lanes_x32(v);
    return v;
}

} // namespace vbq
