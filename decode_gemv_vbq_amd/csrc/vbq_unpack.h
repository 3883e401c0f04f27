// Code-word unpack and fp16 dot products shared by the GEMV kernels (gfx950).
//
// A b-bit group's 64 codes are stored as two halves (codes 0..31 and 32..63),
// each packed LSB-first into 16-bit units; code word d holds unit d of the
// first half in its low 16 bits and unit d of the second half in its high 16
// bits.  One v_and_or_b32 therefore lifts the same code field of both halves
// into the mantissas of an fp16 pair whose exponent is a "magic" 2^(10-pos):
// each half then equals 2^(10-pos) + q exactly, ready for v_dot2_f32_f16
// against the activation pair (x_p, x_{p+32}).  The magic offsets are removed
// per group with a constant of x (see the correction constants in the kernels).
#pragma once

#include "vbq_common.h"

namespace vbq {

// fp16 bits of 2^(10-pos), in both halves.
__host__ __device__ constexpr uint32_t magic_pair(int pos)
{
    return ((uint32_t)(25 - pos) << 10) | (((uint32_t)(25 - pos) << 10) << 16);
}

// Mantissa position used for pair i (inside its word) of a b-bit group, and
// the right shift applied to the word first.  Shared by the unpack and by the
// correction constants so the two can never disagree.
template <int B>
__host__ __device__ constexpr int pair_pos(int i)
{
    return B == 1 ? (i < 10 ? i : i - 10) : B == 2 ? (i <= 4 ? 2 * i : 2 * i - 10) : B == 4 ? (i <= 1 ? 4 * i : 4 * i - 8) : 0;
}
template <int B>
__host__ __device__ constexpr int pair_shift(int i)
{
    return B == 1 ? (i < 10 ? 0 : 10) : B == 2 ? (i <= 4 ? 0 : 10) : B == 4 ? (i <= 1 ? 0 : 8) : 0;
}

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

// (w & mask) | magic in ONE v_and_or_b32.  Written out because gfx9 VOP3 has no
// literal operand and the compiler otherwise splits it into v_and + v_or with
// literals; here the mask sits in an SGPR and the magic in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(magic));
    return r;
}

// Turn NW code words of a b-bit group into fp16 pairs (2^(10-pos)+q): word d
// gives pairs d*(16/b) .. d*(16/b) + 16/b - 1 of the words' run (for b = 8,
// pairs 2d and 2d+1), so the words of a half or a quarter group give the
// matching half or quarter of the group's 32 pairs.
template <int B, int NW>
__device__ __forceinline__ void unpack_words(const uint32_t *w, uint32_t *h)
{
    if constexpr (B == 8) {
#pragma unroll
        for (int d = 0; d < NW; d++) {
            // bytes [b0, 0x64, b2, 0x64] and [b1, 0x64, b3, 0x64]: 1024 + q
            h[2 * d] = __builtin_amdgcn_perm(0x64646464u, w[d], 0x04020400u);
            h[2 * d + 1] = __builtin_amdgcn_perm(0x64646464u, w[d], 0x04030401u);
        }
    } else {
        constexpr int per = 16 / B;                // pairs per word
        constexpr uint32_t field = (1u << B) - 1u; // one code
#pragma unroll
        for (int d = 0; d < NW; d++) {
#pragma unroll
            for (int i = 0; i < per; i++) {
                const int pos = pair_pos<B>(i);
                const int sh = pair_shift<B>(i);
                const uint32_t mask = (field | (field << 16)) << pos;
                h[d * per + i] = and_or(sh ? (w[d] >> sh) : w[d], mask, magic_pair(pos));
            }
        }
    }
}

// The 2b code words of a whole b-bit group -> its 32 pairs.
template <int B>
__device__ __forceinline__ void unpack_pairs(const uint32_t *w, uint32_t *h)
{
    unpack_words<B, 2 * B>(w, h);
}

} // namespace vbq
