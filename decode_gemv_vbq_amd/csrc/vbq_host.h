// Host-side helpers shared by the C-ABI translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vbq.h"

namespace vbq {

// Record a HIP error for vbq_last_error(); returns VBQ_ERR_HIP, or VBQ_OK.
vbq_status hip_status(hipError_t e);

// hip_status(hipGetLastError()) after a launch.
inline vbq_status launch_status() { return hip_status(hipGetLastError()); }

// Host check of a layout struct: magic, version and geometry.
vbq_status check_layout(const vbq_layout *L);

// Zero `bytes` (multiple of 4) at p with a fill kernel (graph-capture safe).
vbq_status zero_words(void *p, uint64_t bytes, hipStream_t stream);

inline uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// Compute units of the current device, queried on every call (so a process
// that drives several devices gets each one's count); 256 if the query fails.
int current_device_cus();

// hipFuncSetAttribute(fn, MaxDynamicSharedMemorySize, bytes) once per kernel
// and device; thread-safe.
vbq_status dynamic_lds_once(const void *fn, int bytes);

// One GEMV request after host-side validation.
struct GemvCall {
    const vbq_layout *L;
    const void *blob;
    int M;
    const uint16_t *x;
    int ldx;
    void *y;
    int ldy;
    vbq_dtype yt;
    hipStream_t stream;
};

// Launches the streaming kernel when it applies (M <= 2 and every row record
// fits one LDS sub-unit); returns false, launching nothing, when it does not.
bool stream_gemv(const GemvCall &g, vbq_status *st);
// Whether the streaming kernel takes a matrix of layout L at M tokens (host only).
bool stream_applies(const vbq_layout *L, int M);

// One matrix of a shared-activation launch.
struct StreamItem {
    const vbq_layout *L;
    const void *blob;
    void *y;
    int ldy;
};

// One streaming launch for up to 4 matrices with the same K that read the same
// x; false (nothing launched) when the streaming kernel does not apply.
bool stream_gemv_shared(const StreamItem *items, int n, int M, const uint16_t *x, int ldx, vbq_dtype yt,
                        hipStream_t stream, vbq_status *st);

// The matrix-core batched GEMV (vbq_mfma.hip): used for M >= kMfmaMinTokens,
// and for M <= 2 where the streaming kernel does not apply, when x is 16-byte
// aligned, ldx % 8 == 0 and the blob and x fit 32-bit buffer offsets
// (mfma_applies checks those conditions for any 1 <= M <= kMaxBatch).
constexpr int kMfmaMinTokens = 3;
constexpr int kMaxBatch = 32; // vbq_gemv_batched: more than 16 tokens only on the matrix cores
bool mfma_applies(const vbq_layout *L, int M, const uint16_t *x, int ldx);
// Workspace bytes for the K split the current device would use at M tokens.
size_t mfma_workspace(const vbq_layout *L, int M);
// Launch on g.stream; splits K only when ws (4-byte aligned) holds the partial sums.
vbq_status mfma_gemv(const GemvCall &g, void *ws, size_t ws_bytes);

// Every check vbq_gemv_planned_shared makes, for every launch it would
// enqueue; launches nothing.
vbq_status planned_shared_check(const vbq_planned_item *items, int n, int M, const uint16_t *x, int ldx,
                                vbq_dtype yt);

// The argmax launches of vbq_gemv_planned_argmax for M (1..16) tokens of a
// checked plan: keys and the ticket counter at `state` (16 u64 keys, then a
// u32 counter; zero before the call, left zero after it), results to
// index[M] and value[M].  Checks plan, x and M-dependent shapes; launches
// nothing on error.
vbq_status planned_argmax(const vbq_plan *P, const void *plan, int M, const uint16_t *x, int ldx, void *state,
                          int32_t *index, float *value, hipStream_t stream);

// Whether two plans can share one launch (same K and M, and one LDS carve-up
// holds both blocks' partial sums).
bool planned_can_share(const vbq_plan *a, const vbq_plan *b);

} // namespace vbq

#define VBQ_TRY(expr)                                                                                                 \
    do {                                                                                                              \
        vbq_status _st = (expr);                                                                                      \
        if (_st != VBQ_OK)                                                                                            \
            return _st;                                                                                               \
    } while (0)
