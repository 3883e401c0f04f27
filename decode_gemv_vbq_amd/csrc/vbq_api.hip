// C-ABI plumbing of libvbq.so: version, status text, layout geometry,
// workspace helpers.  The compute entry points live beside their kernels.
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>

#include "vbq_common.h"
#include "vbq_host.h"

namespace vbq {

static thread_local char g_last_error[256];

vbq_status hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return VBQ_OK;
    snprintf(g_last_error, sizeof g_last_error, "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
    return VBQ_ERR_HIP;
}

vbq_status check_layout(const vbq_layout *L)
{
    if (!L)
        return VBQ_ERR_INVALID_ARG;
    if (L->magic != kMagic || L->version != 1)
        return VBQ_ERR_LAYOUT;
    if (L->N < 1 || L->K < 64 || L->K % 64 || L->G != L->K / 64 || L->S != 32 || L->nS != (L->G + 31) / 32 ||
        L->row_pad != 128)
        return VBQ_ERR_LAYOUT;
    vbq_layout ref;
    if (vbq_layout_init((int)L->N, (int)L->K, &ref) != VBQ_OK)
        return VBQ_ERR_LAYOUT;
    if (L->off_row_off != ref.off_row_off || L->off_slice_off != ref.off_slice_off || L->off_wmap != ref.off_wmap ||
        L->off_scales != ref.off_scales || L->off_codes != ref.off_codes)
        return VBQ_ERR_LAYOUT;
    if (L->code_bytes_padded % 128 || L->total_bytes != L->off_codes + L->code_bytes_padded ||
        L->code_bytes > L->code_bytes_padded || L->code_bytes < 8ull * L->N * L->G ||
        L->code_bytes > 64ull * L->N * L->G)
        return VBQ_ERR_LAYOUT;
    // codes are addressed in 8-byte units with 32-bit indices in the GEMV
    if (L->code_bytes_padded / 8 >= (1ull << 32))
        return VBQ_ERR_LAYOUT;
    return VBQ_OK;
}

} // namespace vbq

using namespace vbq;

extern "C" {

const char *vbq_version(void) { return "vbq 0.1.0 (VBQ1 layout, gfx950)"; }

const char *vbq_status_string(vbq_status st)
{
    switch (st) {
    case VBQ_OK: return "ok";
    case VBQ_ERR_INVALID_ARG: return "invalid argument";
    case VBQ_ERR_SHAPE: return "bad shape (N >= 1, K >= 64, K % 64 == 0, leading dimensions)";
    case VBQ_ERR_BATCH: return "batch M outside [1, 16]";
    case VBQ_ERR_BITS: return "bit-width outside {1, 2, 4, 8}";
    case VBQ_ERR_CODE_RANGE: return "code above 2^b - 1";
    case VBQ_ERR_ALIGN: return "misaligned pointer";
    case VBQ_ERR_WORKSPACE: return "workspace missing or too small";
    case VBQ_ERR_LAYOUT: return "bad or inconsistent VBQ1 layout";
    case VBQ_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *vbq_last_error(void) { return g_last_error; }

vbq_status vbq_layout_init(int N, int K, vbq_layout *L)
{
    if (!L)
        return VBQ_ERR_INVALID_ARG;
    if (N < 1 || K < 64 || K % 64)
        return VBQ_ERR_SHAPE;
    memset(L, 0, sizeof *L);
    uint64_t G = (uint64_t)K / 64, nS = (G + 31) / 32;
    L->magic = kMagic;
    L->version = 1;
    L->N = (uint32_t)N;
    L->K = (uint32_t)K;
    L->G = (uint32_t)G;
    L->S = 32;
    L->nS = (uint32_t)nS;
    L->row_pad = 128;
    L->off_row_off = 256;
    L->off_slice_off = align_up(L->off_row_off + 4ull * ((uint64_t)N + 1), 256);
    L->off_wmap = align_up(L->off_slice_off + 4ull * (uint64_t)N * nS, 256);
    L->off_scales = align_up(L->off_wmap + 8ull * (uint64_t)N * nS, 256);
    L->off_codes = align_up(L->off_scales + 2ull * (uint64_t)N * G, 256);
    return VBQ_OK;
}

vbq_status vbq_layout_from_header(const void *header, vbq_layout *L)
{
    if (!header || !L)
        return VBQ_ERR_INVALID_ARG;
    memcpy(L, header, sizeof *L);
    const uint8_t *h = (const uint8_t *)header;
    for (int i = (int)sizeof(vbq_layout); i < 256; i++)
        if (h[i])
            return VBQ_ERR_LAYOUT;
    return check_layout(L);
}

} // extern "C"

namespace {

__global__ void k_zero_u32(uint32_t *p, uint64_t nwords)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += (uint64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

} // namespace

namespace vbq {

int current_device_cus()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    return cus;
}

vbq_status dynamic_lds_once(const void *fn, int bytes)
{
    static std::mutex mu;
    static std::map<std::pair<const void *, int>, int> done;  // (kernel, device) -> bytes set
    int dev = 0;
    VBQ_TRY(hip_status(hipGetDevice(&dev)));
    std::lock_guard<std::mutex> lock(mu);
    auto it = done.find({fn, dev});
    if (it != done.end() && it->second >= bytes)
        return VBQ_OK;
    VBQ_TRY(hip_status(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes)));
    done[{fn, dev}] = bytes;
    return VBQ_OK;
}

vbq_status zero_words(void *p, uint64_t bytes, hipStream_t stream)
{
    uint64_t words = bytes / 4;
    if (!words)
        return VBQ_OK;
    uint64_t blocks = (words + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)blocks), dim3(256), 0, stream, (uint32_t *)p, words);
    return launch_status();
}

} // namespace vbq

extern "C" vbq_status vbq_workspace_clear(void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (!ws_bytes)
        return VBQ_OK;
    if (!ws)
        return VBQ_ERR_INVALID_ARG;
    if ((uintptr_t)ws % 4 || ws_bytes % 4)
        return VBQ_ERR_ALIGN;
    return zero_words(ws, ws_bytes, stream);
}
