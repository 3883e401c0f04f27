// vbq_gemv_planned_argmax_noalloc: the greedy-decode argmax of
// vbq_gemv_planned_argmax with its state (the per-token keys and the ticket
// counter the launch's workgroups merge through) in a file-scope device array
// of this library instead of a caller workspace, for callers that cannot
// allocate device memory.
//
// Host code never passes the array's name to a kernel: its address on each
// device comes from hipGetSymbolAddress, taken once per device (with that
// device current) at the first call there, and kept.  Every call on a device
// shares that device's array: a call leaves keys and counter zero for the
// next one, and calls that overlap on one device (different streams) race.
#include <mutex>

#include "vbq_host.h"

using namespace vbq;

namespace {

// 16 keys (u64) and the ticket counter (u32), rounded up to 256 bytes.
constexpr int kScratchBytes = 256;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

// This device's address of `scratch`, cleared once (a fill kernel on
// `stream`, so the first call may be captured in a graph); null on error.
vbq_status scratch_ptr(hipStream_t stream, void **out)
{
    static std::mutex mu;
    static void *ptr[kMaxDevices] = {};
    int dev = 0;
    VBQ_TRY(hip_status(hipGetDevice(&dev)));
    if (dev < 0 || dev >= kMaxDevices)
        return VBQ_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void *p = nullptr;
        VBQ_TRY(hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))));
        if (!p)
            return VBQ_ERR_HIP;
        VBQ_TRY(zero_words(p, kScratchBytes, stream));
        ptr[dev] = p;
    }
    *out = ptr[dev];
    return VBQ_OK;
}

} // namespace

extern "C" vbq_status vbq_gemv_planned_argmax_noalloc(const vbq_plan *P, const void *plan, int M, const uint16_t *x,
                                                      int ldx, int32_t *index, float *value, hipStream_t stream)
{
    if (!P || !plan || !x || !index || !value)
        return VBQ_ERR_INVALID_ARG;
    if (M < 1 || M > 16)
        return VBQ_ERR_BATCH; // the array holds the keys of at most 16 tokens
    if ((uintptr_t)index % 4 || (uintptr_t)value % 4)
        return VBQ_ERR_ALIGN;
    void *state = nullptr;
    VBQ_TRY(scratch_ptr(stream, &state));
    return planned_argmax(P, plan, M, x, ldx, state, index, value, stream);
}
