"""GPU parity of the matrix-core batched GEMV (vbq_gemv_batched with 3 <= M <= 32,
x 16-byte aligned, ldx % 8 == 0; one or two token tiles of 16) against the CPU oracle.

* |y - y_ref| <= 1e-3 * sum|w||x| per output over ragged shapes (N not a
  multiple of the 16-row tile or the 128-row block, G not a multiple of the
  8-group chunk or the 32-group slice), every width mix, outlier channels,
  fp16 and fp32 outputs, with and without a K split.
* x = e_k gives column k of the dequantized matrix bit for bit (every k-slot
  position of a group, several groups and slices).
* A token's output does not depend on the batch it runs in (bit for bit), and
  repeated calls are bit-identical, split or not.
"""
import numpy as np
import pytest

import oracle
from decode_gemv_vbq_amd import workload as wl
from tests.gpu_util import upload, within_bound

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def vbq():
    import decode_gemv_vbq_amd as v
    v.lib()
    return v


def draw(N, K, mix=None, seed=0, M=1, cluster=1, outliers=0.0):
    spec = wl.MatrixSpec("m", N, K, mix or wl.MIX_BASE, layer=seed, cluster=cluster)
    return wl.draw_matrix(spec, 91, M=M, outliers=outliers)


def packed(v, q, bits, s, x):
    dq, db, ds, dx = upload(q, bits, s, x, torch)
    blob, L = v.pack(dq, db, ds)
    return blob, L, dx


def check(y, q, bits, s, x, what):
    y_ref, bound = oracle.gemv(q, bits, s, x)
    ok, worst, idx = within_bound(y.float().cpu().numpy(), y_ref, bound)
    assert ok, f"{what}: worst err/bound={worst:.3g} at {idx}"
    return worst


SHAPES = [(1, 64), (17, 128), (129, 64 * 13), (130, 2112), (333, 64 * 150), (1000, 5632), (48, 8192 + 64)]


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("M", [3, 16, 17, 32])
def test_mfma_parity_shapes(N, K, M):
    v = vbq()
    q, bits, s, x = draw(N, K, seed=N + M, M=M, outliers=0.01)
    blob, L, dx = packed(v, q, bits, s, x)
    for yt in (torch.float32, torch.float16):
        y = v.gemv_batched(L, blob, dx, out_dtype=yt, ws=v.workspace(L, M))
        torch.cuda.synchronize()
        check(y, q, bits, s, x, f"N={N} K={K} M={M} {yt}")


@pytest.mark.parametrize("mix", ["u1", "u2", "u4", "u8", "wide", "head"])
@pytest.mark.parametrize("M", [8, 24])
def test_mfma_width_mixes(mix, M):
    v = vbq()
    m = {"u1": {1: 1.0}, "u2": {2: 1.0}, "u4": wl.MIX_U4, "u8": wl.MIX_U8, "wide": wl.MIX_WIDE,
         "head": wl.MIX_HEAD}[mix]
    q, bits, s, x = draw(300, 64 * 45, m, seed=12, M=M, outliers=0.01)
    blob, L, dx = packed(v, q, bits, s, x)
    y = v.gemv_batched(L, blob, dx, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check(y, q, bits, s, x, mix)


@pytest.mark.parametrize("M", list(range(3, 33)))
def test_mfma_every_batch_size(M):
    v = vbq()
    q, bits, s, x = draw(200, 64 * 70, seed=100 + M, M=M, cluster=8, outliers=0.01)
    blob, L, dx = packed(v, q, bits, s, x)
    y = v.gemv_batched(L, blob, dx, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check(y, q, bits, s, x, f"M={M}")


@pytest.mark.parametrize("M", [16, 32])
def test_mfma_split_k_and_determinism(M):
    """A matrix with few row blocks and a long K splits K when the workspace
    allows it; split and unsplit results both meet the bound, and each is
    bit-identical across calls."""
    v = vbq()
    N, K = 200, 64 * 300
    q, bits, s, x = draw(N, K, seed=61, M=M, outliers=0.01)
    blob, L, dx = packed(v, q, bits, s, x)
    ws = v.workspace(L, M)
    assert ws is not None and v.workspace_size(L, M) >= 2 * M * N * 4  # this shape splits
    ys = v.gemv_batched(L, blob, dx, out_dtype=torch.float32, ws=ws)
    ys2 = v.gemv_batched(L, blob, dx, out_dtype=torch.float32, ws=ws)
    small = torch.zeros(16, dtype=torch.uint8, device="cuda")  # too small for the partial sums: one workgroup per row block
    y1 = v.gemv_batched(L, blob, dx, out_dtype=torch.float32, ws=small)
    y12 = v.gemv_batched(L, blob, dx, out_dtype=torch.float32, ws=small)
    torch.cuda.synchronize()
    assert torch.equal(ys, ys2) and torch.equal(y1, y12)
    assert torch.equal(ys, y1)  # the K segments are added in the same order either way
    check(ys, q, bits, s, x, "split")
    check(y1, q, bits, s, x, "unsplit")


def test_mfma_token_independent_of_batch():
    """A token's outputs are the same bit for bit in a batch of 32 (two tiles),
    of 16 or of 3, wherever it sits in the batch."""
    v = vbq()
    N, K = 150, 64 * 67
    q, bits, s, x = draw(N, K, seed=71, M=32, outliers=0.01)
    blob, L, dx = packed(v, q, bits, s, x)
    y16 = v.gemv_batched(L, blob, dx, out_dtype=torch.float32)
    check(y16, q, bits, s, x, "M=32")
    for lo, hi in ((0, 3), (5, 9), (13, 16), (14, 20), (16, 32), (3, 29), (0, 17)):
        part = torch.empty((hi - lo, K), dtype=torch.float16, device="cuda")
        part.copy_(dx[lo:hi])
        yp = v.gemv_batched(L, blob, part, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(yp, y16[lo:hi]), (lo, hi)


def test_mfma_unit_vectors_give_dequant_columns():
    v = vbq()
    N, K = 97, 64 * 75
    q, bits, s, _ = draw(N, K, mix=wl.MIX_WIDE, seed=81)
    blob, L, _ = packed(v, q, bits, s, np.zeros((1, K), np.uint16))
    w = v.dequant(L, blob, torch.float32)
    ks = list(range(64)) + [64, 100, 2047, 2048, 2111, 4000, K - 1]
    for i0 in range(0, len(ks), 32):
        kk = ks[i0:i0 + 32]
        if len(kk) < 3:
            kk = kk + ks[:3 - len(kk)]
        X = torch.zeros((len(kk), K), dtype=torch.float16, device="cuda")
        for i, k in enumerate(kk):
            X[i, k] = 1.0
        Y = v.gemv_batched(L, blob, X, out_dtype=torch.float32)
        torch.cuda.synchronize()
        for i, k in enumerate(kk):
            assert torch.equal(Y[i], w[:, k]), f"column {k}"


def test_mfma_special_scales():
    v = vbq()
    N, K, M = 40, 64 * 70, 4
    q, bits, s, x = draw(N, K, seed=22, M=M)
    s = s.copy()
    s[0, :] = 0x0000           # +0
    s[1, :] = 0x8000           # -0
    s[2, 3] = 0x0001           # smallest subnormal
    s[3, :] = 0x03FF           # largest subnormal
    s[4, :] = 0xAC00           # negative
    s[5, 7] = 0x7C00           # +inf
    s[6, 40] = 0xFC00          # -inf
    s[7, 65] = 0x7E00          # NaN
    s[8, :] = 0x7BFF           # largest finite
    blob, L, dx = packed(v, q, bits, s, x)
    for yt in (torch.float32, torch.float16):
        y = v.gemv_batched(L, blob, dx, out_dtype=yt)
        torch.cuda.synchronize()
        y_ref, bound = oracle.gemv(q, bits, s, x)
        if yt == torch.float16:
            bound = np.where(np.abs(y_ref) > 65504, np.inf, bound)
        ok, worst, idx = within_bound(y.float().cpu().numpy(), y_ref, bound)
        assert ok, f"{yt}: worst err/bound={worst:.3g} at {idx}"
        assert bool((y[:, :2] == 0).all())


@pytest.mark.parametrize("M", [5, 20])
def test_mfma_strided_rows(M):
    """Row strides: ldx % 8 == 0 takes the matrix cores, other strides the
    vector kernels (M <= 16; more tokens are refused); results are in bound and
    only [M][N] is written."""
    v = vbq()
    N, K = 70, 2048 + 64
    q, bits, s, x = draw(N, K, seed=52, M=M)
    blob, L, dx = packed(v, q, bits, s, x)
    for pad in (64, 40, 3):
        if M > 16 and pad % 8:
            xs = torch.zeros((M, K + pad), dtype=torch.float16, device="cuda")
            with pytest.raises(v.VbqError, match="ALIGN"):
                v.gemv_batched(L, blob, xs[:, :K])
            continue
        xs = torch.zeros((M, K + pad), dtype=torch.float16, device="cuda")
        xs[:, :K] = dx
        out = torch.full((M, N + 10), float("nan"), dtype=torch.float32, device="cuda")
        v.gemv_batched(L, blob, xs[:, :K], out=out[:, :N])
        torch.cuda.synchronize()
        check(out[:, :N], q, bits, s, x, f"ldx={K + pad}")
        assert bool(torch.isnan(out[:, N:]).all())


@pytest.mark.parametrize("M", [16, 32])
def test_mfma_graph_replays_match_eager(M):
    """The split launch and its partial-sum kernel captured in a HIP graph:
    every replay (with eager work and synchronisation between replays) gives
    the eager result bit for bit."""
    v = vbq()
    N, K = 200, 64 * 300
    q, bits, s, x = draw(N, K, seed=33 + M, M=M, outliers=0.01)
    blob, L, dx = packed(v, q, bits, s, x)
    ws = v.workspace(L, M)
    assert ws is not None
    eager = v.gemv_batched(L, blob, dx, out_dtype=torch.float32, ws=ws)
    out = torch.empty_like(eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        v.gemv_batched(L, blob, dx, out=out, ws=ws)
    for r in range(3):
        out.fill_(float("nan"))
        other = v.gemv_batched(L, blob, dx[:3].contiguous(), out_dtype=torch.float32, ws=ws)  # eager work between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r}"
        assert torch.equal(other, eager[:3])
    check(eager, q, bits, s, x, f"M={M}")
