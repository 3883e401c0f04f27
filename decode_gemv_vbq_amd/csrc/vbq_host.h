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

// Every check vbq_gemv_planned_shared makes, for every launch it would
// enqueue; launches nothing.
vbq_status planned_shared_check(const vbq_planned_item *items, int n, int M, const uint16_t *x, int ldx,
                                vbq_dtype yt);

// vbq_gemv_planned_shared whose last launch also fetches, into each
// workgroup's free ring slot, the first tile that workgroup's counterpart in
// the following launch (the items `next`, checked plans; null: none) reads.
vbq_status planned_shared_launch(const vbq_planned_item *items, int n, int M, const uint16_t *x, int ldx,
                                 vbq_dtype yt, hipStream_t stream, const vbq_planned_item *next, int nnext);

} // namespace vbq

#define VBQ_TRY(expr)                                                                                                 \
    do {                                                                                                              \
        vbq_status _st = (expr);                                                                                      \
        if (_st != VBQ_OK)                                                                                            \
            return _st;                                                                                               \
    } while (0)
