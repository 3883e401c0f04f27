// Decode-step executors: the GEMVs of one step enqueued stage by stage.
//
// Autoregressive decode runs a model's projections one after another, each
// reading activations computed by the previous stage ("Variable Bit-width
// Quantization", mlsanity.com page, Abstract: the quantized models are decoded
// with fused dequantize-and-multiply kernels, a memory-bound workload).  The
// executors take the step as an array of GEMVs tagged with their stage and
// enqueue them on one stream in stage order, so the stream orders each stage
// after the one before.  Inside a stage, GEMVs that read the same activations
// with the same K (the gate and up projections of an MLP block) share one
// launch.  Every item is checked before the first launch.
//
// There is no persistent tier: on MI355X a grid-wide dependency carried
// through memory inside one cooperative kernel (every workgroup publishes its
// slice of the outputs, every workgroup waits for all of them and reads the
// whole vector back) costs 4.4 to 5.2 us per stage however it is signalled
// (one counter or per-workgroup flags, agent or system scope), and about
// 60 us with release/acquire fences, which write back and invalidate the L2;
// a kernel node of a replayed HIP graph costs about 1.9 us.  Stages therefore
// stay separate launches and a caller that wants the launch floor captures
// the step in a graph.
#include <vector>

#include "vbq_host.h"

using namespace vbq;

namespace {

constexpr int kMaxStage = 1024; // items per stage

bool elem_aligned(const void *p, vbq_dtype t) { return (uintptr_t)p % (t == VBQ_F32 ? 4 : 2) == 0; }

vbq_status check_common(const void *items, int n, int M, vbq_dtype yt)
{
    if (!items || n < 1)
        return VBQ_ERR_INVALID_ARG;
    if (yt != VBQ_F32 && yt != VBQ_F16)
        return VBQ_ERR_INVALID_ARG;
    if (M < 1 || M > 16)
        return VBQ_ERR_BATCH;
    return VBQ_OK;
}

// Stages must be non-decreasing and a stage holds at most kMaxStage items.
template <typename Item>
vbq_status check_stages(const Item *items, int n)
{
    for (int i = 1, i0 = 0; i < n; i++) {
        if (items[i].stage < items[i - 1].stage)
            return VBQ_ERR_INVALID_ARG;
        if (items[i].stage != items[i - 1].stage)
            i0 = i;
        if (i - i0 >= kMaxStage)
            return VBQ_ERR_INVALID_ARG;
    }
    return VBQ_OK;
}

// Calls group(idx, k) for each launch of the step, in order: stages in order,
// and inside a stage, items in order, each opening a group that takes the
// later items of its stage that `compatible` admits, up to VBQ_MAX_SHARED.
template <typename Item, typename Compatible, typename Group>
vbq_status for_each_group(const Item *items, int n, Compatible compatible, Group group)
{
    for (int i0 = 0; i0 < n;) {
        int i1 = i0 + 1;
        while (i1 < n && items[i1].stage == items[i0].stage)
            i1++;
        bool taken[kMaxStage] = {};
        for (int i = i0; i < i1; i++) {
            if (taken[i - i0])
                continue;
            int idx[VBQ_MAX_SHARED];
            int k = 0;
            idx[k++] = i;
            for (int j = i + 1; j < i1 && k < VBQ_MAX_SHARED; j++)
                if (!taken[j - i0] && compatible(items[i], items[j])) {
                    idx[k++] = j;
                    taken[j - i0] = true;
                }
            VBQ_TRY(group(idx, k));
        }
        i0 = i1;
    }
    return VBQ_OK;
}

} // namespace

extern "C" {

vbq_status vbq_gemv_seq(const vbq_seq_item *items, int n, int M, vbq_dtype yt, void *ws, size_t ws_bytes,
                        hipStream_t stream)
{
    VBQ_TRY(check_common(items, n, M, yt));
    for (int i = 0; i < n; i++) {
        const vbq_seq_item &it = items[i];
        if (!it.L || !it.blob || !it.x || !it.y)
            return VBQ_ERR_INVALID_ARG;
        VBQ_TRY(check_layout(it.L));
        if (it.ldx < (int)it.L->K || it.ldy < (int)it.L->N)
            return VBQ_ERR_SHAPE;
        if ((uintptr_t)it.blob % 256 || (uintptr_t)it.x % 2 || !elem_aligned(it.y, yt))
            return VBQ_ERR_ALIGN;
    }
    VBQ_TRY(check_stages(items, n));
    auto compatible = [](const vbq_seq_item &a, const vbq_seq_item &b) {
        return a.x == b.x && a.ldx == b.ldx && a.L->K == b.L->K;
    };
    return for_each_group(items, n, compatible, [&](const int *idx, int k) {
        const vbq_seq_item &a = items[idx[0]];
        if (k == 1)
            return vbq_gemv_batched(a.L, a.blob, M, a.x, a.ldx, a.y, a.ldy, yt, ws, ws_bytes, stream);
        vbq_gemv_item sh[VBQ_MAX_SHARED];
        for (int j = 0; j < k; j++) {
            const vbq_seq_item &b = items[idx[j]];
            sh[j] = vbq_gemv_item{b.L, b.blob, b.y, b.ldy};
        }
        return vbq_gemv_shared(sh, k, M, a.x, a.ldx, yt, stream);
    });
}

vbq_status vbq_gemv_planned_seq(const vbq_planned_seq_item *items, int n, int M, vbq_dtype yt, hipStream_t stream)
{
    VBQ_TRY(check_common(items, n, M, yt));
    for (int i = 0; i < n; i++) {
        const vbq_planned_seq_item &it = items[i];
        if (!it.P || !it.plan || !it.x || !it.y)
            return VBQ_ERR_INVALID_ARG;
    }
    VBQ_TRY(check_stages(items, n));
    // two plans share a launch only where one LDS carve-up serves both
    auto compatible = [](const vbq_planned_seq_item &a, const vbq_planned_seq_item &b) {
        return a.x == b.x && a.ldx == b.ldx && planned_can_share(a.P, b.P);
    };
    // the launches in order, every one checked before the first is enqueued
    struct Launch {
        vbq_planned_item it[VBQ_MAX_SHARED];
        int n;
        const uint16_t *x;
        int ldx;
    };
    std::vector<Launch> launches;
    VBQ_TRY(for_each_group(items, n, compatible, [&](const int *idx, int k) {
        Launch l;
        l.n = k;
        l.x = items[idx[0]].x;
        l.ldx = items[idx[0]].ldx;
        for (int j = 0; j < k; j++) {
            const vbq_planned_seq_item &b = items[idx[j]];
            l.it[j] = vbq_planned_item{b.P, b.plan, b.y, b.ldy};
        }
        launches.push_back(l);
        return planned_shared_check(l.it, k, M, l.x, l.ldx, yt);
    }));
    for (const Launch &l : launches)
        VBQ_TRY(vbq_gemv_planned_shared(l.it, l.n, M, l.x, l.ldx, yt, stream));
    return VBQ_OK;
}

} // extern "C"
