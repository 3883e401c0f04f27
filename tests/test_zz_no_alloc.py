"""GPU check of vbq_gemv_planned_argmax_noalloc (no workspace: the library's
own device array holds the argmax state) against vbq_gemv_planned_argmax with
a caller workspace, on two calls in a row, the second with a smaller input:
index and value must be identical (the same launches over the same plan)."""
import pytest

from decode_gemv_vbq_amd import workload as wl
from tests.gpu_util import upload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def prepared(v, N, K, M, seed):
    spec = wl.MatrixSpec("head", N, K, wl.MIX_HEAD, layer=seed)
    q, bits, s, x = wl.draw_matrix(spec, 95, M=M, outliers=0.0)
    dq, db, ds, dx = upload(q, bits, s, x, torch)
    blob, L = v.pack(dq, db, ds)
    plan, P = v.prepare(L, blob, M=min(2, M))
    return P, plan, dx


def test_noalloc_argmax_matches_workspace_argmax_twice():
    import decode_gemv_vbq_amd as v
    v.lib()
    ws = v.argmax_workspace()
    for N, K, M, seed in [(6000, 2048, 5, 1), (700, 1024, 2, 2)]:  # the second call is smaller
        P, plan, dx = prepared(v, N, K, M, seed)
        i_ws, v_ws = v.gemv_planned_argmax(P, plan, dx, ws=ws)
        i_ws, v_ws = i_ws.clone(), v_ws.clone()
        i_na, v_na = v.gemv_planned_argmax_noalloc(P, plan, dx)
        torch.cuda.synchronize()
        assert torch.equal(i_na, i_ws), (N, M, i_na, i_ws)
        assert torch.equal(v_na.view(torch.int32), v_ws.view(torch.int32)), (N, M, v_na, v_ws)
        assert 0 <= int(i_na.min()) and int(i_na.max()) < N
