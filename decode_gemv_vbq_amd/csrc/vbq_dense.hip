// Hand-written dense fp16 GEMV: the on-GPU control the VBQ path is compared
// with ("faster at equal output" against FP16 decode, "Variable Bit-width
// Quantization" page, Abstract).  Same HBM-bound shape as the VBQ kernel: one
// wavefront per pair of rows, 16-byte loads per lane (1 KiB per wavefront
// instruction), v_dot2_f32_f16 with fp32 accumulation, a butterfly reduction
// across the 64 lanes.
#include "vbq_common.h"
#include "vbq_host.h"

using namespace vbq;

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWave = 2;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

template <int MT>
__global__ __launch_bounds__(kThreads) void k_dense_f16(int N, int K, int M, const uint16_t *__restrict__ w,
                                                        const uint16_t *__restrict__ x, int ldx, void *__restrict__ y,
                                                        int ldy, int yt)
{
    const int lane = threadIdx.x & 63;
    const int wave = (blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int n0 = wave * kRowsPerWave;
    if (n0 >= N)
        return;
    float acc[kRowsPerWave][MT];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; r++)
#pragma unroll
        for (int m = 0; m < MT; m++)
            acc[r][m] = 0.f;
    const uint16_t *wr[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; r++)
        wr[r] = w + (uint64_t)min(n0 + r, N - 1) * K;
    for (int k = lane * 8; k < K; k += 64 * 8) {
        U4 wv[kRowsPerWave];
#pragma unroll
        for (int r = 0; r < kRowsPerWave; r++)
            wv[r] = *reinterpret_cast<const U4 *>(wr[r] + k);
#pragma unroll
        for (int m = 0; m < MT; m++) {
            if (m < M) {
                U4 xv = *reinterpret_cast<const U4 *>(x + (uint64_t)m * ldx + k);
#pragma unroll
                for (int r = 0; r < kRowsPerWave; r++)
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        acc[r][m] = dot2(wv[r].v[j], xv.v[j], acc[r][m]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < kRowsPerWave; r++)
#pragma unroll
        for (int m = 0; m < MT; m++) {
            float v = acc[r][m];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1)
                v += __shfl_xor(v, off, 64);
            acc[r][m] = v;
        }
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < kRowsPerWave; r++) {
            int n = n0 + r;
            if (n >= N)
                continue;
#pragma unroll
            for (int m = 0; m < MT; m++) {
                if (m >= M)
                    continue;
                if (yt == VBQ_F16)
                    reinterpret_cast<__half *>(y)[(uint64_t)m * ldy + n] = __float2half_rn(acc[r][m]);
                else
                    reinterpret_cast<float *>(y)[(uint64_t)m * ldy + n] = acc[r][m];
            }
        }
    }
}

template <int MT>
vbq_status launch(int N, int K, int M, const uint16_t *w, const uint16_t *x, int ldx, void *y, int ldy, int yt,
                  hipStream_t stream)
{
    uint64_t waves = ((uint64_t)N + kRowsPerWave - 1) / kRowsPerWave;
    unsigned blocks = (unsigned)((waves * 64 + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(k_dense_f16<MT>, dim3(blocks), dim3(kThreads), 0, stream, N, K, M, w, x, ldx, y, ldy, yt);
    return launch_status();
}

} // namespace

extern "C" vbq_status vbq_dense_f16_gemv(int N, int K, int M, const uint16_t *w16, const uint16_t *x, int ldx,
                                         void *y, int ldy, vbq_dtype yt, hipStream_t stream)
{
    if (!w16 || !x || !y)
        return VBQ_ERR_INVALID_ARG;
    if (yt != VBQ_F32 && yt != VBQ_F16)
        return VBQ_ERR_INVALID_ARG;
    if (N < 1 || K < 8 || K % 8 || ldx < K || ldx % 8 || ldy < N)
        return VBQ_ERR_SHAPE;
    if (M < 1 || M > 16)
        return VBQ_ERR_BATCH;
    if ((uintptr_t)w16 % 16 || (uintptr_t)x % 16 || (uintptr_t)y % (yt == VBQ_F32 ? 4 : 2))
        return VBQ_ERR_ALIGN;
    int t = (int)yt;
    if (M == 1)
        return launch<1>(N, K, M, w16, x, ldx, y, ldy, t, stream);
    if (M <= 4)
        return launch<4>(N, K, M, w16, x, ldx, y, ldy, t, stream);
    return launch<16>(N, K, M, w16, x, ldx, y, ldy, t, stream);
}
