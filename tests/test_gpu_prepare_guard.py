"""A plan sized for one blob, written from another of the same shape with wider
groups, must report VBQ_STATUS_PLAN and write nothing past its buffer (the
prepared GEMV plan and the GEMM plan)."""
import ctypes

import numpy as np
import pytest

from decode_gemv_vbq_amd import workload as wl
from tests.gpu_util import upload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GUARD = 1 << 16


def vbq():
    import decode_gemv_vbq_amd as v
    v.lib()
    return v


def blob_of(v, N, K, mix, seed):
    spec = wl.MatrixSpec("g", N, K, mix, layer=seed)
    q, bits, s, x = wl.draw_matrix(spec, 92, M=1)
    dq, db, ds, _ = upload(q, bits, s, x, torch)
    return v.pack(dq, db, ds)


def guarded(nbytes):
    """A 256-byte aligned view of nbytes followed by GUARD bytes of 0x5A."""
    raw = torch.full((nbytes + GUARD + 256,), 0x5A, dtype=torch.uint8, device="cuda")
    off = (-raw.data_ptr()) % 256
    return raw, raw[off:off + nbytes], raw[off + nbytes:off + nbytes + GUARD]


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("N,K", [(300, 64 * 40), (1000, 64 * 64)])
def test_prepared_plan_rejects_wider_blob(N, K):
    v = vbq()
    blob_a, L_a = blob_of(v, N, K, {1: 1.0}, 1)
    blob_b, L_b = blob_of(v, N, K, {8: 1.0}, 2)
    P = v.plan_init(L_a, blob_a)
    raw, plan, guard = guarded(P.total_bytes)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    rc = v.lib().vbq_prepare(ctypes.byref(P), ctypes.byref(L_b), ctypes.c_void_p(blob_b.data_ptr()),
                             ctypes.c_void_p(plan.data_ptr()), ctypes.c_void_p(status.data_ptr()), stream())
    torch.cuda.synchronize()
    assert v.STATUS[rc] == "VBQ_OK"
    assert int(status.item()) & v.STATUS_PLAN
    assert bool((guard == 0x5A).all())
    with pytest.raises(v.VbqError):
        v.status_check(status)
    # the blob it was sized for still prepares cleanly
    status.zero_()
    rc = v.lib().vbq_prepare(ctypes.byref(P), ctypes.byref(L_a), ctypes.c_void_p(blob_a.data_ptr()),
                             ctypes.c_void_p(plan.data_ptr()), ctypes.c_void_p(status.data_ptr()), stream())
    torch.cuda.synchronize()
    assert v.STATUS[rc] == "VBQ_OK" and int(status.item()) == 0
    assert bool((guard == 0x5A).all())


@pytest.mark.parametrize("N,K", [(300, 64 * 40), (130, 64 * 96)])
def test_gemm_plan_rejects_wider_blob(N, K):
    v = vbq()
    blob_a, L_a = blob_of(v, N, K, {1: 1.0}, 3)
    blob_b, L_b = blob_of(v, N, K, {8: 1.0}, 4)
    GP = v.gemm_plan_init(L_a, blob_a)
    raw, buf, guard = guarded(GP.total_bytes)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    rc = v.lib().vbq_gemm_prepare(ctypes.byref(GP), ctypes.byref(L_b), ctypes.c_void_p(blob_b.data_ptr()),
                                  ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(status.data_ptr()), stream())
    torch.cuda.synchronize()
    assert v.STATUS[rc] == "VBQ_OK"
    assert int(status.item()) & v.STATUS_PLAN
    assert bool((guard == 0x5A).all())
    status.zero_()
    rc = v.lib().vbq_gemm_prepare(ctypes.byref(GP), ctypes.byref(L_a), ctypes.c_void_p(blob_a.data_ptr()),
                                  ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(status.data_ptr()), stream())
    torch.cuda.synchronize()
    assert v.STATUS[rc] == "VBQ_OK" and int(status.item()) == 0
    assert bool((guard == 0x5A).all())
