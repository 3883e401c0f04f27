"""GPU checks of the SwiGLU epilogue vbq_gemv_planned_swiglu on interleaved
(gate, up) matrices against the oracle: h = silu(g) * u from the oracle GEMV's
fp64 outputs.  The bound follows from the GEMV's: with tol_g, tol_u the GEMV
tolerances of the two rows (1e-3 * sum |w||x|) and |silu'| <= 1.1,
|h - h_ref| <= 1.1 |u| tol_g + (|silu(g)| + 1.1 tol_g) tol_u + 1e-6 |h_ref|
(fp32 evaluation of the activation), plus 2^-11 |h_ref| for fp16 outputs."""
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


def interleaved(Np, K, seed, M):
    g = wl.draw_matrix(wl.MatrixSpec("gate", Np, K, wl.MIX_BASE, layer=seed), 95, M=M)
    u = wl.draw_matrix(wl.MatrixSpec("up", Np, K, wl.MIX_BASE, layer=seed), 96, M=M)
    q = np.empty((2 * Np, K), np.uint8)
    bits = np.empty((2 * Np, K // 64), np.uint8)
    s = np.empty((2 * Np, K // 64), np.uint16)
    for dst, src in ((q, 0), (bits, 1), (s, 2)):
        dst[0::2], dst[1::2] = g[src], u[src]
    return q, bits, s, g[3]


@pytest.mark.parametrize("Np,K,M,wgs", [(1536, 2048, 1, 0), (700, 1024, 2, 0), (2048, 4096, 5, 7), (33, 640, 1, 0)])
@pytest.mark.parametrize("yt", ["f16", "f32"])
def test_swiglu_against_oracle(Np, K, M, wgs, yt):
    v = vbq()
    q, bits, s, x = interleaved(Np, K, Np + K, M)
    dq, db, ds, dx = upload(q, bits, s, x, torch)
    blob, L = v.pack(dq, db, ds)
    plan, P = v.prepare(L, blob, M=min(2, M), wgs=wgs)
    assert P.rows % 2 == 0
    h = v.gemv_planned_swiglu(P, plan, dx, out_dtype=torch.float16 if yt == "f16" else torch.float32)
    torch.cuda.synchronize()
    y_ref, bound = oracle.gemv(q, bits, s, x)
    g, u = y_ref[:, 0::2], y_ref[:, 1::2]
    tg, tu = 1e-3 * bound[:, 0::2], 1e-3 * bound[:, 1::2]
    h_ref = oracle.swiglu(g, u)
    sg = np.abs(oracle.swiglu(g, np.ones_like(g)))
    tol = 1.1 * np.abs(u) * tg + (sg + 1.1 * tg) * tu + 1e-6 * np.abs(h_ref)
    if yt == "f16":
        tol += 2.0 ** -11 * np.abs(h_ref)
    err = np.abs(h.float().cpu().numpy().astype(np.float64) - h_ref)
    assert np.all(err <= tol), f"worst err/tol {np.max(err / np.maximum(tol, 1e-300)):.3g}"


def test_swiglu_rejects_odd_rows():
    v = vbq()
    q, bits, s, x = interleaved(64, 128, 3, 1)
    dq, db, ds, dx = upload(q[:127], bits[:127], s[:127], x, torch)
    blob, L = v.pack(dq, db, ds)
    plan, P = v.prepare(L, blob, M=1)
    with pytest.raises(v.VbqError) as e:
        v.gemv_planned_swiglu(P, plan, dx)
    assert e.value.name == "VBQ_ERR_SHAPE"
