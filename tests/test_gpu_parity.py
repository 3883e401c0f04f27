"""GPU parity of libvbq against the CPU oracle (same seeded inputs).

* vbq_pack and vbq_dequant: bit-exact, whole blob / whole matrix.
* vbq_gemv / vbq_gemv_batched: |y - y_ref| <= 1e-3 * sum|w||x| per output,
  at sizes spanning several row tiles, several K-slices and ragged tails.
* Invariants: x = e_k gives column k of the dequantized matrix bit-exactly,
  repeated runs are bit-identical, a matrix in a shared launch gives the bits
  it gives alone; a token of a batch of 3+ (matrix cores) and the same token
  alone (streaming kernel) add in different orders and are each held to the
  bound.
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


SHAPES = [
    # (N, K) spanning: one group; G not a multiple of 32; one full slice;
    # several slices with a ragged last slice; N not a multiple of the tile.
    (1, 64), (3, 128), (768, 768), (37, 2048), (200, 2112), (130, 4096 + 640), (64, 8192), (1000, 5632),
]


def draw(N, K, mix=None, seed=0, M=1, cluster=1, outliers=0.0):
    spec = wl.MatrixSpec("t", N, K, mix or wl.MIX_BASE, layer=seed, cluster=cluster)
    return wl.draw_matrix(spec, 90, M=M, outliers=outliers)


@pytest.mark.parametrize("N,K", SHAPES)
def test_pack_bitexact(N, K):
    v = vbq()
    q, bits, s, x = draw(N, K, seed=N)
    ref = oracle.pack(q, bits, s)
    dq, db, ds, _ = upload(q, bits, s, x, torch)
    L = v.pack_plan(db, K)
    assert L.total_bytes == ref.size
    blob, L = v.pack(dq, db, ds, L)
    got = blob.cpu().numpy()
    assert np.array_equal(got, ref), f"first diff at byte {int(np.argmax(got != ref))}"
    # the header read back from the device blob gives the same layout
    assert v.layout_of(blob).as_dict() == L.as_dict()


@pytest.mark.parametrize("mix", ["base", "u8", "u1", "wide"])
def test_pack_bitexact_mixes(mix):
    v = vbq()
    m = {"base": wl.MIX_BASE, "u8": wl.MIX_U8, "u1": {1: 1.0}, "wide": wl.MIX_WIDE}[mix]
    q, bits, s, x = draw(70, 3008, m, seed=7)
    dq, db, ds, _ = upload(q, bits, s, x, torch)
    blob, _ = v.pack(dq, db, ds)
    assert np.array_equal(blob.cpu().numpy(), oracle.pack(q, bits, s))


def test_pack_reports_bad_inputs():
    v = vbq()
    q, bits, s, x = draw(8, 256, seed=3)
    dq, db, ds, _ = upload(q, bits, s, x, torch)
    L = v.pack_plan(db, 256)
    bad = bits.copy()
    bad[2, 1] = 3
    with pytest.raises(v.VbqError) as e:
        v.pack_plan(upload(q, bad, s, x, torch)[1], 256)
    assert e.value.name == "VBQ_ERR_BITS"
    qb = q.copy()
    g = int(np.argmax(bits[0] < 8))
    qb[0, 64 * g] = 255 if bits[0, g] < 8 else qb[0, 64 * g]
    with pytest.raises(v.VbqError) as e:
        v.pack(upload(qb, bits, s, x, torch)[0], db, ds, L)
    assert e.value.name == "VBQ_ERR_CODE_RANGE"
    # widths that no longer match the plan: rejected, and nothing written out of bounds
    wider = bits.copy()
    wider[:, :] = 8
    guard = torch.full((4096,), 0x5A, dtype=torch.uint8, device="cuda")
    with pytest.raises(v.VbqError) as e:
        v.pack(dq, upload(q, wider, s, x, torch)[1], ds, L)
    assert e.value.name == "VBQ_ERR_LAYOUT"
    assert bool((guard == 0x5A).all())


@pytest.mark.parametrize("N,K", SHAPES[:6])
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_dequant_bitexact(N, K, dtype):
    v = vbq()
    q, bits, s, x = draw(N, K, seed=N + 1)
    dq, db, ds, _ = upload(q, bits, s, x, torch)
    blob, L = v.pack(dq, db, ds)
    if dtype == "f32":
        got = v.dequant(L, blob, torch.float32).cpu().numpy()
        ref = oracle.dequant(q, bits, s)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    else:
        got = v.dequant(L, blob, torch.float16).cpu().numpy().view(np.uint16)
        ref = oracle.dequant(q, bits, s, dtype=np.float16)
        assert np.array_equal(got, ref)


def test_dequant_special_scales_bitexact():
    v = vbq()
    N, K = 16, 64 * 40
    q, bits, s, x = draw(N, K, seed=5)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0xBC00, 0x7BFF, 0xFBFF], np.uint16)
    s = s.copy()
    s[:, :len(specials)] = specials
    dq, db, ds, _ = upload(q, bits, s, x, torch)
    blob, L = v.pack(dq, db, ds)
    got = v.dequant(L, blob, torch.float32).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), oracle.dequant(q, bits, s).view(np.uint32))
    got16 = v.dequant(L, blob, torch.float16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got16, oracle.dequant(q, bits, s, dtype=np.float16))


def run_gemv(v, q, bits, s, x, yt="f16"):
    dq, db, ds, dx = upload(q, bits, s, x, torch)
    blob, L = v.pack(dq, db, ds)
    out_dtype = torch.float16 if yt == "f16" else torch.float32
    if dx.shape[0] == 1:
        y = v.gemv(L, blob, dx[0], out_dtype=out_dtype)[None]
    else:
        y = v.gemv_batched(L, blob, dx, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), blob, L


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("yt", ["f16", "f32"])
def test_gemv_parity(N, K, yt):
    v = vbq()
    q, bits, s, x = draw(N, K, seed=N + 2)
    y, _, _ = run_gemv(v, q, bits, s, x, yt)
    y_ref, bound = oracle.gemv(q, bits, s, x)
    ok, worst, idx = within_bound(y, y_ref, bound)
    assert ok, f"N={N} K={K} worst err/bound={worst:.3g} at {idx}"


@pytest.mark.parametrize("M", [2, 3, 4, 7, 8, 13, 16])
def test_gemv_batched_parity(M):
    v = vbq()
    q, bits, s, x = draw(150, 4096 + 192, seed=M, M=M, outliers=0.01)
    y, _, _ = run_gemv(v, q, bits, s, x, "f32")
    y_ref, bound = oracle.gemv(q, bits, s, x)
    ok, worst, idx = within_bound(y, y_ref, bound)
    assert ok, f"M={M} worst err/bound={worst:.3g} at {idx}"


@pytest.mark.parametrize("mix", ["u1", "u2", "u4", "u8", "wide", "head"])
def test_gemv_parity_width_mixes(mix):
    v = vbq()
    m = {"u1": {1: 1.0}, "u2": {2: 1.0}, "u4": wl.MIX_U4, "u8": wl.MIX_U8, "wide": wl.MIX_WIDE,
         "head": wl.MIX_HEAD}[mix]
    q, bits, s, x = draw(300, 2048 + 1024, m, seed=11, M=3)
    y, _, _ = run_gemv(v, q, bits, s, x, "f32")
    y_ref, bound = oracle.gemv(q, bits, s, x)
    ok, worst, idx = within_bound(y, y_ref, bound)
    assert ok, f"{mix} worst err/bound={worst:.3g} at {idx}"


def test_gemv_clustered_outliers():
    v = vbq()
    q, bits, s, x = draw(256, 8192, seed=4, M=4, cluster=8, outliers=0.01)
    y, _, _ = run_gemv(v, q, bits, s, x, "f32")
    y_ref, bound = oracle.gemv(q, bits, s, x)
    ok, worst, idx = within_bound(y, y_ref, bound)
    assert ok, f"worst err/bound={worst:.3g}"


def test_gemv_special_scales():
    v = vbq()
    N, K = 40, 64 * 70
    q, bits, s, x = draw(N, K, seed=21)
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
    for yt in ("f32", "f16"):
        y, _, _ = run_gemv(v, q, bits, s, x, yt)
        y_ref, bound = oracle.gemv(q, bits, s, x)
        if yt == "f16":
            # fp16 output overflows where the exact value exceeds the fp16 range
            big = np.abs(y_ref) > 65504
            bound = np.where(big, np.inf, bound)
        ok, worst, idx = within_bound(y, y_ref, bound)
        assert ok, f"{yt}: worst err/bound={worst:.3g} at {idx}"
        assert np.all(y[0, :2] == 0)


def test_gemv_unit_vectors_give_dequant_columns():
    v = vbq()
    N, K = 97, 64 * 75
    q, bits, s, _ = draw(N, K, seed=31)
    dq, db, ds, _ = upload(q, bits, s, np.zeros((1, K), np.uint16), torch)
    blob, L = v.pack(dq, db, ds)
    w = v.dequant(L, blob, torch.float32)
    ks = [0, 1, 31, 32, 63, 64, 2047, 2048, 2111, K - 1]
    X = torch.zeros((len(ks), K), dtype=torch.float16, device="cuda")
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    Y = v.gemv_batched(L, blob, X, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for i, k in enumerate(ks):
        assert torch.equal(Y[i], w[:, k]), f"column {k}"


def test_gemv_deterministic_and_batch_consistent():
    v = vbq()
    N, K, M = 333, 64 * 150, 5
    q, bits, s, x = draw(N, K, seed=41, M=M)
    dq, db, ds, dx = upload(q, bits, s, x, torch)
    blob, L = v.pack(dq, db, ds)
    ws = v.workspace(L, 16)
    y1 = v.gemv_batched(L, blob, dx, out_dtype=torch.float32, ws=ws)
    y2 = v.gemv_batched(L, blob, dx, out_dtype=torch.float32, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    y_ref, bound = oracle.gemv(q, bits, s, x)
    for m in range(M):
        ym = v.gemv(L, blob, dx[m].contiguous(), out_dtype=torch.float32, ws=ws)
        torch.cuda.synchronize()
        # a single-token call may sum in another order (other tile plan): both meet the bound
        ok, worst, _ = within_bound(ym.cpu().numpy()[None], y_ref[m:m + 1], bound[m:m + 1])
        assert ok, f"token {m}: {worst:.3g}"
        ym2 = v.gemv(L, blob, dx[m].contiguous(), out_dtype=torch.float32, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(ym, ym2)


def test_gemv_strided_batch():
    v = vbq()
    N, K, M = 64, 2048 + 64, 3
    q, bits, s, x = draw(N, K, seed=51, M=M)
    dq, db, ds, dx = upload(q, bits, s, x, torch)
    blob, L = v.pack(dq, db, ds)
    xs = torch.zeros((M, K + 40), dtype=torch.float16, device="cuda")
    xs[:, :K] = dx
    out = torch.full((M, N + 10), float("nan"), dtype=torch.float32, device="cuda")
    v.gemv_batched(L, blob, xs[:, :K], out=out[:, :N])
    torch.cuda.synchronize()
    y_ref, bound = oracle.gemv(q, bits, s, x)
    ok, worst, _ = within_bound(out[:, :N].cpu().numpy(), y_ref, bound)
    assert ok, worst
    assert bool(torch.isnan(out[:, N:]).all())   # nothing written past ldy's used part


@pytest.mark.parametrize("N,K,M", [(1, 64, 1), (257, 2048, 1), (100, 5632, 4), (64, 8192, 16)])
def test_dense_control_parity(N, K, M):
    v = vbq()
    q, bits, s, x = draw(N, K, seed=61, M=M)
    w16 = oracle.dequant(q, bits, s, dtype=np.float16)
    dw = torch.from_numpy(w16.view(np.int16)).view(torch.float16).cuda()
    dx = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.float16).cuda()
    y = v.dense_f16_gemv(dw, dx, out_dtype=torch.float32)
    torch.cuda.synchronize()
    y_ref, bound = oracle.dense_gemv(w16, x)
    ok, worst, _ = within_bound(y.cpu().numpy(), y_ref, bound)
    assert ok, worst


@pytest.mark.parametrize("Ns,K,M,yt", [((5632, 5632), 2048, 1, "f16"), ((300, 77, 1000), 4096, 1, "f32"),
                                        ((640, 33, 200, 129), 2112, 2, "f16"), ((96, 64), 768, 4, "f32")])
def test_gemv_shared_parity_and_equal_to_single(Ns, K, M, yt):
    """Matrices that share x in one launch: each output within the bound of
    the oracle, and bit-identical to the same matrix run alone (the per-row
    summation order does not depend on the launch)."""
    v = vbq()
    out_dtype = torch.float16 if yt == "f16" else torch.float32
    spec0 = wl.MatrixSpec("t", Ns[0], K, wl.MIX_BASE, layer=K)
    x = wl.draw_x(spec0, 91, M, outliers=0.01)
    dx = torch.from_numpy(x.view(np.int16)).cuda().view(torch.float16)
    mats, host = [], []
    for i, N in enumerate(Ns):
        spec = wl.MatrixSpec("t", N, K, wl.MIX_WIDE if i % 2 else wl.MIX_BASE, layer=i + 3)
        bits = wl.draw_bits(spec, 91)
        q = wl.draw_codes(spec, 91, bits)
        s = wl.draw_scales(spec, 91)
        dq, db, ds, _ = upload(q, bits, s, x, torch)
        blob, L = v.pack(dq, db, ds)
        mats.append((L, blob))
        host.append((q, bits, s))
    outs = v.gemv_shared(mats, dx, out_dtype=out_dtype)
    torch.cuda.synchronize()
    for (L, blob), (q, bits, s), y in zip(mats, host, outs):
        got = y.float().cpu().numpy().astype(np.float64)
        y_ref, bound = oracle.gemv(q, bits, s, x)
        ok, worst, where = within_bound(got, y_ref, bound)
        assert ok, (Ns, L.N, worst, where)
        alone = v.gemv_batched(L, blob, dx, out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(alone, y)


@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("align", [True, False])
def test_gemv_long_k_one_or_two_tokens(M, align):
    """K above what the streaming kernel stages (16256): one or two tokens run
    on the matrix cores when x is 16-byte aligned (with or without a
    workspace, the same bits), else on the vector fallback; both in bound."""
    v = vbq()
    N, K = 150, 64 * 448
    q, bits, s, x = draw(N, K, seed=90 + M, M=M, outliers=0.01)
    dq, db, ds, dx = upload(q, bits, s, x, torch)
    blob, L = v.pack(dq, db, ds)
    if not align:  # rows at an odd 8-byte offset: not 16-byte aligned
        xs = torch.zeros(M * K + 4, dtype=torch.float16, device="cuda")
        xs[4:].view(M, K).copy_(dx)
        dx = xs[4:].view(M, K)
    assert (dx.data_ptr() % 16 == 0) == align
    ws = v.workspace(L, M)
    assert ws is not None  # a long K on few row blocks: the matrix cores' K split wants partial sums
    ys = []
    for w in (ws, torch.zeros(16, dtype=torch.uint8, device="cuda")):
        if M == 1 and align:
            ys.append(v.gemv(L, blob, dx[0], out_dtype=torch.float32, ws=w)[None])
        else:
            ys.append(v.gemv_batched(L, blob, dx, out_dtype=torch.float32, ws=w))
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1])
    y_ref, bound = oracle.gemv(q, bits, s, x)
    ok, worst, idx = within_bound(ys[0].cpu().numpy().astype(np.float64), y_ref, bound)
    assert ok, f"M={M} align={align} worst err/bound={worst:.3g} at {idx}"
