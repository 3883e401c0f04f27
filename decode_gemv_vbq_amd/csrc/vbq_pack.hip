// Packing (q, widths, scales) -> VBQ1 blob, and the blob -> dense dequant.
//
// Offline steps of the path; plain, bounds-checked kernels.  Each group of 64
// weights ("Variable Bit-width Quantization" page, Abstract) is handled by one
// thread; rows are located through row_off (128-byte units), slices through
// slice_off, groups inside a slice through the width bit planes.
#include <stdio.h>
#include <string.h>

#include "vbq_common.h"
#include "vbq_host.h"

using namespace vbq;

namespace {

// Header bytes 0..95 mirror vbq_layout; 96..255 are zero (blob pre-zeroed).
__global__ void k_write_header(uint8_t *blob, vbq_layout L)
{
    const uint32_t *src = reinterpret_cast<const uint32_t *>(&L);
    int i = threadIdx.x;
    if (i < (int)(sizeof(vbq_layout) / 4))
        reinterpret_cast<uint32_t *>(blob)[i] = src[i];
}

// units[n] = ceil(sum_g 8*b / 128); total code bytes; width validation.
__global__ void k_row_units(int N, int G, const uint8_t *__restrict__ bits, uint32_t *__restrict__ units,
                            unsigned long long *__restrict__ code_bytes, uint32_t *__restrict__ status)
{
    int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N)
        return;
    const uint8_t *b = bits + (uint64_t)n * G;
    uint32_t bytes = 0;
    bool bad = false;
    for (int g = 0; g < G; g++) {
        uint32_t w = b[g];
        bool ok = w == 1 || w == 2 || w == 4 || w == 8;
        bad |= !ok;
        bytes += ok ? 8u * w : 0u;
    }
    units[n] = (bytes + 127u) / 128u;
    if (code_bytes)
        atomicAdd(code_bytes, (unsigned long long)bytes);
    if (bad)
        atomicOr(status, VBQ_STATUS_BITS);
}

// In-place exclusive scan: d[0..N-1] in, d[0..N] out.  One block of 1024.
__global__ __launch_bounds__(1024) void k_scan_excl(uint32_t *d, int N)
{
    __shared__ uint32_t s[1024];
    __shared__ uint32_t carry;
    int tid = threadIdx.x;
    if (tid == 0)
        carry = 0;
    __syncthreads();
    for (int base = 0; base < N; base += 1024) {
        int i = base + tid;
        uint32_t v = i < N ? d[i] : 0u;
        s[tid] = v;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            uint32_t t = tid >= off ? s[tid - off] : 0u;
            __syncthreads();
            s[tid] += t;
            __syncthreads();
        }
        uint32_t incl = s[tid];
        uint32_t c = carry;
        if (i < N)
            d[i] = c + incl - v;
        __syncthreads();
        if (tid == 1023)
            carry = c + incl;
        __syncthreads();
    }
    if (tid == 0)
        d[N] = carry;
}

// Per row: width bit planes and slice offsets; checks the record fits.
__global__ void k_pack_meta(vbq_layout L, const uint8_t *__restrict__ bits, uint8_t *__restrict__ blob,
                            uint32_t *__restrict__ status)
{
    int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= (int)L.N)
        return;
    const uint32_t *row_off = reinterpret_cast<const uint32_t *>(blob + L.off_row_off);
    uint32_t *slice_off = reinterpret_cast<uint32_t *>(blob + L.off_slice_off);
    uint32_t *wmap = reinterpret_cast<uint32_t *>(blob + L.off_wmap);
    const uint8_t *b = bits + (uint64_t)n * L.G;
    uint32_t pos = 0;
    for (uint32_t t = 0; t < L.nS; t++) {
        uint32_t p0 = 0, p1 = 0;
        uint32_t g0 = 32 * t, g1 = min(L.G, g0 + 32);
        slice_off[(uint64_t)n * L.nS + t] = pos;
        for (uint32_t g = g0; g < g1; g++) {
            uint32_t w = b[g];
            uint32_t c = w == 2 ? 1u : w == 4 ? 2u : w == 8 ? 3u : 0u;
            p0 |= (c & 1u) << (g - g0);
            p1 |= (c >> 1) << (g - g0);
            pos += (w == 1 || w == 2 || w == 4 || w == 8) ? 8u * w : 0u;
        }
        wmap[2 * ((uint64_t)n * L.nS + t)] = p0;
        wmap[2 * ((uint64_t)n * L.nS + t) + 1] = p1;
    }
    uint64_t start = 128ull * row_off[n], end = 128ull * row_off[n + 1];
    if (start + pos > end || L.off_codes + end > L.total_bytes)
        atomicOr(status, VBQ_STATUS_LAYOUT);
}

__global__ void k_copy_u16(const uint16_t *__restrict__ src, uint16_t *__restrict__ dst, uint64_t count)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (uint64_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

// Encode the 64 codes of one b-bit group into its 2b little-endian words.
template <int B>
__device__ __forceinline__ bool encode_group(const uint8_t *__restrict__ q, uint32_t *__restrict__ out)
{
    constexpr int per_unit = 16 / B; // codes per 16-bit unit
    constexpr uint32_t maxq = (1u << B) - 1u;
    uint8_t c[64];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        U4 v = *reinterpret_cast<const U4 *>(q + 16 * k);
#pragma unroll
        for (int j = 0; j < 16; j++)
            c[16 * k + j] = (uint8_t)(v.v[j / 4] >> (8 * (j % 4)));
    }
    bool ok = true;
#pragma unroll
    for (int j = 0; j < 64; j++)
        ok &= c[j] <= maxq;
#pragma unroll
    for (int d = 0; d < 2 * B; d++) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < per_unit; i++) {
            lo |= ((uint32_t)c[d * per_unit + i] & maxq) << (i * B);
            hi |= ((uint32_t)c[32 + d * per_unit + i] & maxq) << (i * B);
        }
        out[d] = lo | (hi << 16);
    }
    return ok;
}

// One thread per group: locate it in its row record and write its codes.
__global__ void k_pack_codes(vbq_layout L, const uint8_t *__restrict__ q, const uint8_t *__restrict__ bits,
                             uint8_t *__restrict__ blob, uint32_t *__restrict__ status)
{
    uint64_t gid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (uint64_t)L.N * L.G)
        return;
    uint64_t n = gid / L.G;
    uint32_t g = (uint32_t)(gid % L.G), t = g / 32, gi = g % 32;
    uint32_t w = bits[gid];
    if (!(w == 1 || w == 2 || w == 4 || w == 8))
        return; // reported by k_row_units
    const uint32_t *row_off = reinterpret_cast<const uint32_t *>(blob + L.off_row_off);
    const uint32_t *slice_off = reinterpret_cast<const uint32_t *>(blob + L.off_slice_off);
    const uint32_t *wmap = reinterpret_cast<const uint32_t *>(blob + L.off_wmap);
    uint64_t rs = n * L.nS + t;
    int ng = (int)min(32u, L.G - 32 * t);
    WidthMasks m = width_masks(wmap[2 * rs], wmap[2 * rs + 1], ng);
    int c = w == 1 ? 0 : w == 2 ? 1 : w == 4 ? 2 : 3;
    uint64_t dst = L.off_codes + 128ull * row_off[n] + slice_off[rs] + group_offset_in_slice(m, c, (int)gi);
    uint64_t row_end = L.off_codes + 128ull * row_off[n + 1];
    if (dst + 8ull * w > row_end || row_end > L.total_bytes) {
        atomicOr(status, VBQ_STATUS_LAYOUT);
        return;
    }
    uint32_t *out = reinterpret_cast<uint32_t *>(blob + dst);
    const uint8_t *src = q + n * L.K + 64ull * g;
    bool ok;
    switch (c) {
    case 0: ok = encode_group<1>(src, out); break;
    case 1: ok = encode_group<2>(src, out); break;
    case 2: ok = encode_group<4>(src, out); break;
    default: ok = encode_group<8>(src, out); break;
    }
    if (!ok)
        atomicOr(status, VBQ_STATUS_CODES);
}

// Decode one b-bit group and write its 64 dequantized weights.
template <int B, typename T>
__device__ __forceinline__ void dequant_group(const uint32_t *__restrict__ src, float s, T *__restrict__ dst)
{
    // w = s * (q - c) must be one exact product: no contraction into an fma
    // (s*q - s*c loses the sign of zero products) and no fused f16 rounding.
#pragma clang fp contract(off)
    constexpr int per_unit = 16 / B;
    constexpr uint32_t maxq = (1u << B) - 1u;
    const float center = 0.5f * (float)maxq;
    uint32_t wd[2 * B];
#pragma unroll
    for (int d = 0; d < 2 * B; d += 2) {
        U2 v = *reinterpret_cast<const U2 *>(src + d);
        wd[d] = v.v[0];
        wd[d + 1] = v.v[1];
    }
    float out[64];
#pragma unroll
    for (int d = 0; d < 2 * B; d++)
#pragma unroll
        for (int i = 0; i < per_unit; i++) {
            out[d * per_unit + i] = s * ((float)((wd[d] >> (i * B)) & maxq) - center);
            out[32 + d * per_unit + i] = s * ((float)((wd[d] >> (16 + i * B)) & maxq) - center);
        }
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int j = 0; j < 64; j += 4)
            *reinterpret_cast<float4 *>(dst + j) = make_float4(out[j], out[j + 1], out[j + 2], out[j + 3]);
    } else {
#pragma unroll
        for (int j = 0; j < 64; j += 8) {
            U4 v;
#pragma unroll
            for (int k = 0; k < 4; k++) {
                // keep the exact fp32 product: the compiler would otherwise fold
                // product + rounding into v_fma_mix, whose "+ 0" flips -0 to +0
                float p0 = out[j + 2 * k], p1 = out[j + 2 * k + 1];
                asm volatile("" : "+v"(p0), "+v"(p1));
                uint32_t a = __half_as_ushort(__float2half_rn(p0));
                uint32_t b = __half_as_ushort(__float2half_rn(p1));
                v.v[k] = a | (b << 16);
            }
            *reinterpret_cast<U4 *>(dst + j) = v;
        }
    }
}

template <typename T>
__global__ void k_dequant(vbq_layout L, const uint8_t *__restrict__ blob, T *__restrict__ w)
{
    uint64_t gid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (uint64_t)L.N * L.G)
        return;
    uint64_t n = gid / L.G;
    uint32_t g = (uint32_t)(gid % L.G), t = g / 32, gi = g % 32;
    const uint32_t *row_off = reinterpret_cast<const uint32_t *>(blob + L.off_row_off);
    const uint32_t *slice_off = reinterpret_cast<const uint32_t *>(blob + L.off_slice_off);
    const uint32_t *wmap = reinterpret_cast<const uint32_t *>(blob + L.off_wmap);
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(blob + L.off_scales);
    uint64_t rs = n * L.nS + t;
    uint32_t p0 = wmap[2 * rs], p1 = wmap[2 * rs + 1];
    int ng = (int)min(32u, L.G - 32 * t);
    WidthMasks m = width_masks(p0, p1, ng);
    int c = width_code(p0, p1, (int)gi);
    uint64_t off = L.off_codes + 128ull * row_off[n] + slice_off[rs] + group_offset_in_slice(m, c, (int)gi);
    if (off + (8ull << c) > L.total_bytes)
        return; // a blob whose tables point outside itself: nothing to read
    const uint32_t *src = reinterpret_cast<const uint32_t *>(blob + off);
    float s = __half2float(__ushort_as_half(scales[gid]));
    T *dst = w + n * L.K + 64ull * g;
    switch (c) {
    case 0: dequant_group<1>(src, s, dst); break;
    case 1: dequant_group<2>(src, s, dst); break;
    case 2: dequant_group<4>(src, s, dst); break;
    default: dequant_group<8>(src, s, dst); break;
    }
}

unsigned blocks_for(uint64_t items, unsigned threads) { return (unsigned)((items + threads - 1) / threads); }

} // namespace

extern "C" {

size_t vbq_pack_plan_workspace(int N)
{
    if (N < 1)
        return 0;
    return align_up(4ull * ((uint64_t)N + 1), 256) + 256;
}

vbq_status vbq_pack_plan(int N, int K, const uint8_t *bits, vbq_layout *L, void *ws, size_t ws_bytes,
                         hipStream_t stream)
{
    if (!bits || !L || !ws)
        return VBQ_ERR_INVALID_ARG;
    VBQ_TRY(vbq_layout_init(N, K, L));
    if (ws_bytes < vbq_pack_plan_workspace(N))
        return VBQ_ERR_WORKSPACE;
    if ((uintptr_t)ws % 8)
        return VBQ_ERR_ALIGN;
    uint8_t *w = (uint8_t *)ws;
    uint32_t *units = (uint32_t *)w;
    uint8_t *tail = w + align_up(4ull * ((uint64_t)N + 1), 256);
    unsigned long long *code_bytes = (unsigned long long *)tail;
    uint32_t *status = (uint32_t *)(tail + 8);
    VBQ_TRY(zero_words(tail, 16, stream));
    hipLaunchKernelGGL(k_row_units, dim3(blocks_for(N, 256)), dim3(256), 0, stream, N, (int)L->G, bits, units,
                       code_bytes, status);
    VBQ_TRY(launch_status());
    hipLaunchKernelGGL(k_scan_excl, dim3(1), dim3(1024), 0, stream, units, N);
    VBQ_TRY(launch_status());
    uint32_t total_units = 0;
    uint64_t host_tail[2] = {0, 0};
    VBQ_TRY(hip_status(hipMemcpyAsync(&total_units, units + N, 4, hipMemcpyDeviceToHost, stream)));
    VBQ_TRY(hip_status(hipMemcpyAsync(host_tail, tail, 16, hipMemcpyDeviceToHost, stream)));
    VBQ_TRY(hip_status(hipStreamSynchronize(stream)));
    if ((uint32_t)host_tail[1] & VBQ_STATUS_BITS)
        return VBQ_ERR_BITS;
    L->code_bytes = host_tail[0];
    L->code_bytes_padded = 128ull * total_units;
    L->total_bytes = L->off_codes + L->code_bytes_padded;
    if (L->code_bytes_padded / 8 >= (1ull << 32))
        return VBQ_ERR_SHAPE;
    return VBQ_OK;
}

vbq_status vbq_pack(const vbq_layout *L, const uint8_t *q, const uint8_t *bits, const uint16_t *scales, void *blob,
                    uint32_t *status_word, hipStream_t stream)
{
    if (!q || !bits || !scales || !blob || !status_word)
        return VBQ_ERR_INVALID_ARG;
    VBQ_TRY(check_layout(L));
    if ((uintptr_t)blob % 256 || (uintptr_t)q % 16 || (uintptr_t)scales % 2 || (uintptr_t)status_word % 4)
        return VBQ_ERR_ALIGN;
    const vbq_layout Lv = *L;
    uint8_t *b = (uint8_t *)blob;
    int N = (int)Lv.N;
    VBQ_TRY(zero_words(status_word, 4, stream));
    VBQ_TRY(zero_words(b, Lv.total_bytes, stream));
    hipLaunchKernelGGL(k_write_header, dim3(1), dim3(64), 0, stream, b, Lv);
    VBQ_TRY(launch_status());
    // row_off: per-row units into row_off[0..N-1], then the in-place scan
    uint32_t *row_off = (uint32_t *)(b + Lv.off_row_off);
    hipLaunchKernelGGL(k_row_units, dim3(blocks_for(N, 256)), dim3(256), 0, stream, N, (int)Lv.G, bits, row_off,
                       (unsigned long long *)nullptr, status_word);
    VBQ_TRY(launch_status());
    hipLaunchKernelGGL(k_scan_excl, dim3(1), dim3(1024), 0, stream, row_off, N);
    VBQ_TRY(launch_status());
    hipLaunchKernelGGL(k_pack_meta, dim3(blocks_for(N, 256)), dim3(256), 0, stream, Lv, bits, b, status_word);
    VBQ_TRY(launch_status());
    uint64_t ns = (uint64_t)Lv.N * Lv.G;
    hipLaunchKernelGGL(k_copy_u16, dim3(blocks_for(ns, 256) < 8192 ? blocks_for(ns, 256) : 8192), dim3(256), 0, stream,
                       scales, (uint16_t *)(b + Lv.off_scales), ns);
    VBQ_TRY(launch_status());
    hipLaunchKernelGGL(k_pack_codes, dim3(blocks_for(ns, 256)), dim3(256), 0, stream, Lv, q, bits, b, status_word);
    return launch_status();
}

vbq_status vbq_status_check(const uint32_t *status_word, uint32_t *raw, hipStream_t stream)
{
    if (!status_word)
        return VBQ_ERR_INVALID_ARG;
    uint32_t v = 0;
    VBQ_TRY(hip_status(hipMemcpyAsync(&v, status_word, 4, hipMemcpyDeviceToHost, stream)));
    VBQ_TRY(hip_status(hipStreamSynchronize(stream)));
    if (raw)
        *raw = v;
    if (v & VBQ_STATUS_BITS)
        return VBQ_ERR_BITS;
    if (v & VBQ_STATUS_CODES)
        return VBQ_ERR_CODE_RANGE;
    if (v & VBQ_STATUS_LAYOUT)
        return VBQ_ERR_LAYOUT;
    if (v & VBQ_STATUS_PLAN)
        return VBQ_ERR_SHAPE;
    return VBQ_OK;
}

vbq_status vbq_dequant(const vbq_layout *L, const void *blob, void *w, vbq_dtype wt, hipStream_t stream)
{
    if (!blob || !w)
        return VBQ_ERR_INVALID_ARG;
    if (wt != VBQ_F32 && wt != VBQ_F16)
        return VBQ_ERR_INVALID_ARG;
    VBQ_TRY(check_layout(L));
    if ((uintptr_t)blob % 256 || (uintptr_t)w % 16)
        return VBQ_ERR_ALIGN;
    uint64_t groups = (uint64_t)L->N * L->G;
    if (wt == VBQ_F32)
        hipLaunchKernelGGL(k_dequant<float>, dim3(blocks_for(groups, 256)), dim3(256), 0, stream, *L,
                           (const uint8_t *)blob, (float *)w);
    else
        hipLaunchKernelGGL(k_dequant<uint16_t>, dim3(blocks_for(groups, 256)), dim3(256), 0, stream, *L,
                           (const uint8_t *)blob, (uint16_t *)w);
    return launch_status();
}

} // extern "C"
