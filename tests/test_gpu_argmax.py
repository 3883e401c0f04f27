"""GPU checks of the greedy-decode epilogue vbq_gemv_planned_argmax.

Several rows can be correct when two outputs lie within the GEMV tolerance of
each other, so the index is checked for validity against the oracle (its
oracle value is within the two outputs' bounds of the oracle maximum) and for
uniqueness against the GPU's own fp32 outputs (vbq_gemv_planned, bit for bit:
the returned value is that row's output and the index is the first maximal
row).  Engineered cases with a clear winner or exact ties check the index
itself against the oracle.
"""
import numpy as np
import pytest

import oracle
from decode_gemv_vbq_amd import workload as wl
from tests.gpu_util import upload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def vbq():
    import decode_gemv_vbq_amd as v
    v.lib()
    return v


def draw(N, K, seed, M):
    spec = wl.MatrixSpec("head", N, K, wl.MIX_HEAD, layer=seed)
    return wl.draw_matrix(spec, 93, M=M, outliers=0.0)


def run(v, q, bits, s, x, wgs=0):
    dq, db, ds, dx = upload(q, bits, s, x, torch)
    blob, L = v.pack(dq, db, ds)
    plan, P = v.prepare(L, blob, M=min(2, dx.shape[0]), wgs=wgs)
    ws = v.argmax_workspace()
    idx, val = v.gemv_planned_argmax(P, plan, dx, ws=ws)
    y = v.gemv_planned(P, plan, dx, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return idx.cpu().numpy().copy(), val.cpu().numpy().copy(), y.cpu().numpy(), (P, plan, dx, ws)


@pytest.mark.parametrize("N,K,M,wgs", [(5000, 2048, 1, 0), (3001, 1024, 2, 0), (4096, 4096, 3, 3), (777, 640, 16, 0)])
def test_argmax_valid_and_consistent(N, K, M, wgs):
    v = vbq()
    q, bits, s, x = draw(N, K, N + M, M)
    idx, val, y, _ = run(v, q, bits, s, x, wgs=wgs)
    y_ref, bound = oracle.gemv(q, bits, s, x)
    for m in range(M):
        i = int(idx[m])
        assert 0 <= i < N
        assert val[m].tobytes() == y[m, i].tobytes()          # the row's own fp32 output
        assert i == int(np.argmax(y[m]))                      # first maximal row of the GPU outputs
        r = int(np.argmax(y_ref[m]))
        assert y_ref[m, i] >= y_ref[m, r] - 1e-3 * (bound[m, i] + bound[m, r]), (m, i, r)


def test_argmax_clear_winner_and_ties():
    v = vbq()
    N, K, M = 2048, 2048, 1
    q, bits, s, x = draw(N, K, 5, M)
    # row 1234 gets scales of 64 with the sign that makes its output positive:
    # it then exceeds every other output by far more than the tolerance
    y0, _ = oracle.gemv(q, bits, s, x)
    s = s.copy()
    s[1234] = (np.float16(64.0) * (1 if y0[0, 1234] * s[1234].view(np.float16).astype(np.float64)[0] >= 0 else -1)
               * np.sign(s[1234].view(np.float16).astype(np.float64))).astype(np.float16).view(np.uint16)
    idx, val, y, _ = run(v, q, bits, s, x)
    y_ref, _ = oracle.gemv(q, bits, s, x)
    assert list(idx) == [int(np.argmax(y_ref[m])) for m in range(M)]
    # an exact copy of the winner at a lower row: the tie goes to the smaller row
    q2, bits2, s2 = q.copy(), bits.copy(), s.copy()
    win = int(idx[0])
    q2[100], bits2[100], s2[100] = q2[win], bits2[win], s2[win]
    idx2, val2, y2, _ = run(v, q2, bits2, s2, x)
    assert idx2[0] == 100 and val2[0].tobytes() == val[0].tobytes()


def test_argmax_workspace_reuse_and_reset():
    v = vbq()
    N, K, M = 3000, 1024, 5
    q, bits, s, x = draw(N, K, 8, M)
    idx, val, y, (P, plan, dx, ws) = run(v, q, bits, s, x, wgs=7)
    for _ in range(3):
        i2, v2 = v.gemv_planned_argmax(P, plan, dx, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(i2.cpu().numpy(), idx) and v2.cpu().numpy().tobytes() == val.tobytes()
    wsn = ws.cpu().numpy()
    assert not wsn[:36].any()  # keys and counter are zero between calls
