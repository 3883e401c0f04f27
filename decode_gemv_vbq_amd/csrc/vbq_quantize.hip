// Round-to-nearest quantizer: float weights and a width map -> codes and fp16
// scales, the inputs of vbq_pack.
//
// "Variable Bit-width Quantization" (mlsanity.com page, Abstract) gives every
// contiguous group of 64 weights its own width from {1, 2, 4, 8} and stores
// low-bit codes; its scales are learned during training, and the pages give
// no rule that turns float weights into codes.  This library takes the plain
// reading: per group, with c = (2^b - 1) / 2,
//   a   = max_j |w_j|                        (fp32, NaN weights skipped)
//   s   = fp16_rne(a / c)
//   q_j = clamp(rint(w_j / s + c), 0, 2^b - 1)
// each step one IEEE fp32 operation (correctly rounded division, rint rounding
// half to even, fmaxf/fminf for the clamp so a NaN quotient gives 0).
//
// Eight lanes per group, eight weights per lane: a wavefront reads 8 groups
// weights with 16- or 32-byte loads per lane, takes each group's absolute
// maximum over its 8 lanes with DPP moves, and writes 8 codes (8 bytes) per
// lane; the first lane of each group writes its scale.
#include "vbq_host.h"

#include <hip/hip_fp16.h>

using namespace vbq;

namespace {

constexpr int kQT = 256;         // threads per workgroup
constexpr int kQG = kQT / 8;      // groups per workgroup

struct QuantArgs {
    const void *w;
    int ldw;
    int N, G;
    const uint8_t *bits;
    uint8_t *q;
    uint16_t *scales;
    uint32_t *status;
};

template <int kCtrl>
__device__ __forceinline__ float dpp_max(float v)
{
    return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false)));
}

// Weights j0..j0+7 of a row as fp32 (fp16 widened exactly); VEC: one 16-byte
// (fp16) or two 16-byte (fp32) loads, else element loads.
template <bool F16, bool VEC>
__device__ __forceinline__ void load8(const void *w, uint64_t off, float (&v)[8])
{
    if (F16) {
        const __half *p = reinterpret_cast<const __half *>(w) + off;
        if (VEC) {
            const uint4 u = *reinterpret_cast<const uint4 *>(p);
            const uint32_t d[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                v[2 * i] = __half2float(__ushort_as_half((uint16_t)(d[i] & 0xffffu)));
                v[2 * i + 1] = __half2float(__ushort_as_half((uint16_t)(d[i] >> 16)));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; i++)
                v[i] = __half2float(p[i]);
        }
    } else {
        const float *p = reinterpret_cast<const float *>(w) + off;
        if (VEC) {
            const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; i++)
                v[i] = p[i];
        }
    }
}

template <bool F16, bool VEC>
__global__ __launch_bounds__(kQT) void k_quantize(QuantArgs a)
{
    const int sub = threadIdx.x & 7; // lane within the group
    const uint64_t grp = (uint64_t)blockIdx.x * kQG + (threadIdx.x >> 3);
    const bool live = grp < (uint64_t)a.N * (uint64_t)a.G;
    const uint64_t gi = live ? grp : 0; // dead lanes follow group 0 (all lanes join the DPP moves)
    const uint64_t n = gi / (uint64_t)a.G, g = gi % (uint64_t)a.G;
    float v[8];
    load8<F16, VEC>(a.w, n * (uint64_t)a.ldw + 64u * g + 8u * (uint64_t)sub, v);
    const int b = a.bits[gi];
    const bool ok = b == 1 || b == 2 || b == 4 || b == 8;
    // absolute maximum over the group's 64 weights (exact in any order)
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++)
        m = fmaxf(m, fabsf(v[i]));
    m = dpp_max<0xB1>(m);  // quad_perm [1, 0, 3, 2]
    m = dpp_max<0x4E>(m);  // quad_perm [2, 3, 0, 1]
    m = dpp_max<0x141>(m); // row_half_mirror: the other quad of the 8 lanes
    const int bb = ok ? b : 1;
    const float top = (float)((1 << bb) - 1);
    const float c = top * 0.5f;
    const __half sh = __float2half_rn(__fdiv_rn(m, c));
    const float s = __half2float(sh);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float r = rintf(__fadd_rn(__fdiv_rn(v[i], s), c));
        const uint32_t qv = ok ? (uint32_t)fminf(fmaxf(r, 0.0f), top) : 0u;
        if (i < 4)
            lo |= qv << (8 * i);
        else
            hi |= qv << (8 * (i - 4));
    }
    if (!live)
        return;
    *reinterpret_cast<uint2 *>(a.q + 64u * gi + 8u * (uint64_t)sub) = make_uint2(lo, hi);
    if (sub == 0) {
        a.scales[gi] = ok ? __half_as_ushort(sh) : (uint16_t)0;
        if (!ok && a.status)
            atomicOr(a.status, VBQ_STATUS_BITS);
    }
}

} // namespace

extern "C" {

vbq_status vbq_quantize(int N, int K, const void *w, vbq_dtype wt, int ldw, const uint8_t *bits, uint8_t *q,
                        uint16_t *scales, uint32_t *status_word, hipStream_t stream)
{
    if (!w || !bits || !q || !scales)
        return VBQ_ERR_INVALID_ARG;
    if (wt != VBQ_F32 && wt != VBQ_F16)
        return VBQ_ERR_INVALID_ARG;
    if (N < 1 || K < 64 || K % 64 != 0 || ldw < K)
        return VBQ_ERR_SHAPE;
    if ((uintptr_t)w % (wt == VBQ_F32 ? 4 : 2) || (uintptr_t)scales % 2 || (uintptr_t)status_word % 4)
        return VBQ_ERR_ALIGN;
    QuantArgs a{w, ldw, N, K / 64, bits, q, scales, status_word};
    const uint64_t groups = (uint64_t)N * (uint64_t)(K / 64);
    const uint64_t blocks = (groups + kQG - 1) / kQG;
    if (blocks > 0x7fffffffull)
        return VBQ_ERR_SHAPE;
    if ((uintptr_t)q % 8)
        return VBQ_ERR_ALIGN;
    if (status_word)
        VBQ_TRY(zero_words(status_word, 4, stream));
    // vector loads need every lane's 8 weights 16-byte aligned
    const bool vec = (uintptr_t)w % 16 == 0 && ldw % (wt == VBQ_F16 ? 8 : 4) == 0;
    const dim3 grid((unsigned)blocks), block(kQT);
    if (wt == VBQ_F16) {
        if (vec)
            hipLaunchKernelGGL((k_quantize<true, true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((k_quantize<true, false>), grid, block, 0, stream, a);
    } else {
        if (vec)
            hipLaunchKernelGGL((k_quantize<false, true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((k_quantize<false, false>), grid, block, 0, stream, a);
    }
    return launch_status();
}

} // extern "C"
