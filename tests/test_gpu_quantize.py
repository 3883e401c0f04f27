"""GPU parity of vbq_quantize against the oracle's quantizer: codes and fp16
scales bit for bit (the rule decides integers in fp32 on both sides), for fp32
and fp16 weights, strided rows, special values, a bad width, and quantize ->
pack -> planned GEMV end to end against the oracle GEMV of the same codes."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import to_dev, within_bound

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

WIDTHS = np.array([1, 2, 4, 8], np.uint8)


def vbq():
    import decode_gemv_vbq_amd as v
    v.lib()
    return v


def weights(N, K, seed, special=True):
    r = np.random.default_rng(seed)
    w = (r.standard_normal((N, K)) * np.exp(2 * r.standard_normal((N, K // 64)).repeat(64, 1))).astype(np.float32)
    if special and N >= 8 and K >= 128:
        w[0, :64] = 0.0
        w[1, 3] = -0.0
        w[2, 7] = np.nan
        w[3, 70] = np.inf
        w[4, 9] = -np.inf
        w[5, :64] *= 1e30
        w[6, 64:128] *= 1e-12
    return w


@pytest.mark.parametrize("N,K", [(1, 64), (8, 128), (37, 2048 + 640), (300, 4096)])
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_quantize_bit_exact(N, K, dtype):
    v = vbq()
    r = np.random.default_rng(N + K)
    bits = r.choice(WIDTHS, (N, K // 64))
    w = weights(N, K, N * 7 + K)
    if dtype == "f16":
        with np.errstate(over="ignore"):
            w = w.astype(np.float16)
    q_ref, s_ref = oracle.quantize(w, bits)
    dw = to_dev(w, torch)
    q, s = v.quantize(dw, to_dev(bits, torch))
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy().view(np.uint16), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


def test_quantize_strided_rows_and_bad_width():
    v = vbq()
    N, K = 16, 1024
    r = np.random.default_rng(9)
    bits = r.choice(WIDTHS, (N, K // 64))
    w = weights(N, K, 10, special=False)
    big = torch.zeros((N, K + 192), dtype=torch.float32, device="cuda")
    big[:, :K] = to_dev(w, torch)
    status = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    q, s = v.quantize(big[:, :K], to_dev(bits, torch), status=status)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize(w, bits)
    assert np.array_equal(q.cpu().numpy(), q_ref) and np.array_equal(s.cpu().numpy().view(np.uint16), s_ref)
    assert int(status.item()) == 0  # cleared, no bad width
    bits_bad = bits.copy()
    bits_bad[3, 5] = 3
    q, s = v.quantize(big[:, :K], to_dev(bits_bad, torch), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & v.STATUS_BITS
    qn, sn = q.cpu().numpy(), s.cpu().numpy().view(np.uint16)
    assert not qn[3, 320:384].any() and sn[3, 5] == 0
    keep = np.ones((N, K // 64), bool)
    keep[3, 5] = False
    assert np.array_equal(sn[keep], s_ref[keep])


def test_quantize_pack_gemv_end_to_end():
    v = vbq()
    N, K = 512, 4096
    r = np.random.default_rng(11)
    bits = r.choice(WIDTHS, (N, K // 64), p=[0.69, 0.15, 0.12, 0.04])
    w = weights(N, K, 12, special=False)
    x = r.standard_normal((2, K)).astype(np.float16).view(np.uint16)
    dq, ds = v.quantize(to_dev(w, torch), to_dev(bits, torch))
    blob, L = v.pack(dq, to_dev(bits, torch), ds.view(torch.float16))
    plan, P = v.prepare(L, blob, M=2)
    y = v.gemv_planned(P, plan, to_dev(x.view(np.int16), torch, torch.float16), out_dtype=torch.float32)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize(w, bits)
    y_ref, bound = oracle.gemv(q_ref, bits, s_ref, x)
    ok, worst, idx = within_bound(y.cpu().numpy(), y_ref, bound)
    assert ok, f"worst err/bound {worst:.3g} at {idx}"
