"""GPU parity of the prepared-plan GEMV (vbq_plan_init / vbq_prepare /
vbq_gemv_planned[_shared]) against the CPU oracle, on the same seeded inputs.

* |y - y_ref| <= 1e-3 * sum|w||x| per output, at shapes that span one group,
  ragged K-slices, large row blocks (small block counts, up to the LDS limit)
  and every width mix.
* Invariants: x = e_k gives column k of vbq_dequant bit-exactly; repeated runs
  are bit-identical; a matrix in a shared launch gives the same bits as alone.
* The plan buffer itself: pass records and width bytes read back on the host
  must hold every group of the matrix exactly once, in the documented order.
"""
import numpy as np
import pytest

import oracle
from decode_gemv_vbq_amd import workload as wl
from tests import mini_oracle
from tests.gpu_util import upload, within_bound

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def vbq():
    import decode_gemv_vbq_amd as v
    v.lib()
    return v


def draw(N, K, mix=None, seed=0, M=1, cluster=1, outliers=0.0):
    spec = wl.MatrixSpec("t", N, K, mix or wl.MIX_BASE, layer=seed, cluster=cluster)
    return wl.draw_matrix(spec, 92, M=M, outliers=outliers)


def planned(v, q, bits, s, x, M=None, wgs=0, yt="f32"):
    dq, db, ds, dx = upload(q, bits, s, x, torch)
    blob, L = v.pack(dq, db, ds)
    plan, P = v.prepare(L, blob, M=M or dx.shape[0], wgs=wgs)
    out_dtype = torch.float16 if yt == "f16" else torch.float32
    y = v.gemv_planned(P, plan, dx, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), (blob, L, plan, P, dx)


# (N, K, wgs): one group; G below one slice; ragged slices; large blocks (wgs
# 1..3 put hundreds of rows in one block, up to the LDS limit, beyond which the
# block count grows); K = 28672 (G = 448)
CASES = [
    (1, 64, 0), (3, 128, 0), (768, 768, 0), (37, 2048, 0), (200, 2112, 0), (130, 4096 + 640, 0),
    (1000, 5632, 0), (300, 4096, 1), (257, 2048, 3), (64, 28672, 0), (9, 28672, 2), (2000, 64, 1),
]


@pytest.mark.parametrize("N,K,wgs", CASES)
@pytest.mark.parametrize("yt", ["f16", "f32"])
def test_planned_parity(N, K, wgs, yt):
    v = vbq()
    q, bits, s, x = draw(N, K, seed=N + 7)
    y, _ = planned(v, q, bits, s, x, wgs=wgs, yt=yt)
    y_ref, bound = oracle.gemv(q, bits, s, x)
    ok, worst, idx = within_bound(y, y_ref, bound)
    assert ok, f"N={N} K={K} wgs={wgs} worst err/bound={worst:.3g} at {idx}"


@pytest.mark.parametrize("mix", ["u1", "u2", "u4", "u8", "wide", "head"])
def test_planned_width_mixes_two_tokens(mix):
    v = vbq()
    m = {"u1": {1: 1.0}, "u2": {2: 1.0}, "u4": wl.MIX_U4, "u8": wl.MIX_U8, "wide": wl.MIX_WIDE,
         "head": wl.MIX_HEAD}[mix]
    q, bits, s, x = draw(300, 2048 + 1024, m, seed=13, M=2, outliers=0.01)
    for wgs in (0, 2):
        y, _ = planned(v, q, bits, s, x, wgs=wgs)
        y_ref, bound = oracle.gemv(q, bits, s, x)
        ok, worst, idx = within_bound(y, y_ref, bound)
        assert ok, f"{mix} wgs={wgs} worst err/bound={worst:.3g} at {idx}"


def test_planned_special_scales():
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
        y, _ = planned(v, q, bits, s, x, wgs=3, yt=yt)
        y_ref, bound = oracle.gemv(q, bits, s, x)
        if yt == "f16":
            big = np.abs(y_ref) > 65504
            bound = np.where(big, np.inf, bound)
        ok, worst, idx = within_bound(y, y_ref, bound)
        assert ok, f"{yt}: worst err/bound={worst:.3g} at {idx}"
        assert np.all(y[0, :2] == 0)


def test_planned_unit_vectors_give_dequant_columns():
    v = vbq()
    N, K = 97, 64 * 75
    q, bits, s, _ = draw(N, K, seed=31)
    dq, db, ds, _ = upload(q, bits, s, np.zeros((1, K), np.uint16), torch)
    blob, L = v.pack(dq, db, ds)
    w = v.dequant(L, blob, torch.float32)
    plan, P = v.prepare(L, blob, M=2, wgs=5)
    ks = [0, 1, 31, 32, 63, 64, 2047, 2048, 2111, K - 1]
    for i in range(0, len(ks), 2):
        X = torch.zeros((2, K), dtype=torch.float16, device="cuda")
        X[0, ks[i]] = 1.0
        X[1, ks[i + 1]] = 1.0
        Y = v.gemv_planned(P, plan, X, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(Y[0], w[:, ks[i]]), f"column {ks[i]}"
        assert torch.equal(Y[1], w[:, ks[i + 1]]), f"column {ks[i + 1]}"


def test_planned_deterministic_strided_and_token_consistent():
    v = vbq()
    N, K, M = 333, 64 * 150, 2
    q, bits, s, x = draw(N, K, seed=41, M=M)
    dq, db, ds, dx = upload(q, bits, s, x, torch)
    blob, L = v.pack(dq, db, ds)
    plan, P = v.prepare(L, blob, M=2)
    xs = torch.zeros((M, K + 40), dtype=torch.float16, device="cuda")
    xs[:, :K] = dx
    out = torch.full((M, N + 10), float("nan"), dtype=torch.float32, device="cuda")
    v.gemv_planned(P, plan, xs[:, :K], out=out[:, :N])
    y2 = v.gemv_planned(P, plan, dx, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out[:, :N], y2)
    assert bool(torch.isnan(out[:, N:]).all())  # nothing written past the used part of each row
    y_ref, bound = oracle.gemv(q, bits, s, x)
    ok, worst, _ = within_bound(y2.cpu().numpy(), y_ref, bound)
    assert ok, worst
    for m in range(M):  # one token alone: the same plan sums in the same order
        ym = v.gemv_planned(P, plan, dx[m].contiguous(), out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(ym, y2[m])


@pytest.mark.parametrize("M,Mp", [(3, 2), (4, 1), (7, 2), (16, 2)])
def test_planned_many_tokens(M, Mp):
    """M above what one launch holds: token chunks over the same plan, each
    token bit-identical to its single-token run and within the bound."""
    v = vbq()
    N, K = 150, 4096 + 192
    q, bits, s, x = draw(N, K, seed=M, M=M, outliers=0.01)
    dq, db, ds, dx = upload(q, bits, s, x, torch)
    blob, L = v.pack(dq, db, ds)
    plan, P = v.prepare(L, blob, M=Mp)
    y = v.gemv_planned(P, plan, dx, out_dtype=torch.float32)
    torch.cuda.synchronize()
    y_ref, bound = oracle.gemv(q, bits, s, x)
    ok, worst, idx = within_bound(y.cpu().numpy(), y_ref, bound)
    assert ok, f"M={M} worst err/bound={worst:.3g} at {idx}"
    for m in (0, M - 1):
        ym = v.gemv_planned(P, plan, dx[m].contiguous(), out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(ym, y[m])


@pytest.mark.parametrize("Ns,K,M,yt", [((5632, 5632), 2048, 1, "f16"), ((300, 77, 1000), 4096, 1, "f32"),
                                        ((640, 33, 200, 129), 2112, 2, "f16"),
                                        # two same-shape matrices, one token: the preloaded two-record kernel;
                                        # two shapes: the argument records
                                        ((3000, 3000), 4096 + 640, 1, "f32"), ((1000, 998), 4096, 1, "f32")])
def test_planned_shared_parity_and_equal_to_single(Ns, K, M, yt):
    v = vbq()
    out_dtype = torch.float16 if yt == "f16" else torch.float32
    spec0 = wl.MatrixSpec("t", Ns[0], K, wl.MIX_BASE, layer=K)
    x = wl.draw_x(spec0, 93, M, outliers=0.01)
    dx = torch.from_numpy(x.view(np.int16)).cuda().view(torch.float16)
    plans, host = [], []
    rows = -(-max(Ns) // 64)  # about the same rows per block for every matrix
    for i, N in enumerate(Ns):
        spec = wl.MatrixSpec("t", N, K, wl.MIX_WIDE if i % 2 else wl.MIX_BASE, layer=i + 3)
        bits = wl.draw_bits(spec, 93)
        q = wl.draw_codes(spec, 93, bits)
        s = wl.draw_scales(spec, 93)
        dq, db, ds, _ = upload(q, bits, s, x, torch)
        blob, L = v.pack(dq, db, ds)
        plan, P = v.prepare(L, blob, M=2, wgs=-(-N // rows))
        plans.append((P, plan))
        host.append((q, bits, s))
    outs = v.gemv_planned_shared(plans, dx, out_dtype=out_dtype)
    torch.cuda.synchronize()
    for (P, plan), (q, bits, s), y in zip(plans, host, outs):
        got = y.float().cpu().numpy().astype(np.float64)
        y_ref, bound = oracle.gemv(q, bits, s, x)
        ok, worst, where = within_bound(got, y_ref, bound)
        assert ok, (Ns, P.N, worst, where)
        alone = v.gemv_planned(P, plan, dx, out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(alone, y)


@pytest.mark.parametrize("N,K,wgs", [(300, 4096, 1), (1000, 5632, 7), (5, 64, 0), (64, 28672, 3), (1, 128, 0)])
def test_plan_passes_cover_every_group_once(N, K, wgs):
    """Host read-back of the plan: per block, the width bytes list the passes
    (widths 1, 2, 4, 8 in order) for each wavefront; every group of the block
    sits in exactly one pass of its width, with the blob's code record (the
    independent numpy packer's bytes for its codes), its scale and its
    position; (column, row) ascend within a width; empty places hold zero
    codes, scale 0 and the spare position; the word area holds each group's
    word once per lane that works on the group (all 512 bytes used)."""
    v = vbq()
    q, bits, s, x = draw(N, K, seed=5)
    _, (blob, L, plan, P, _) = planned(v, q, bits, s, x, wgs=wgs)
    buf = plan.cpu().numpy()
    G = K // 64
    # the documented position stride: from 32 rows on, padded to 64 / L mod 32
    L = 64 if G > 256 else 32 if G > 128 else 16 if G > 64 else 8
    S = max(P.rows, 2) if P.rows < 32 else P.rows + (64 // L - P.rows) % 32
    assert P.psum == (S * G + 1 + 3) // 4 * 4
    seen = np.zeros((N, G), np.int32)
    assert P.region_bytes == (P.passes * 1536 + 16 * P.per_wave + 255) // 256 * 256
    for b in range(P.wgs):
        n0 = b * P.rows
        R = min(P.rows, N - n0)
        base = b * P.region_bytes
        meta = buf[base + P.passes * 1536:base + P.passes * 1536 + 16 * P.per_wave].reshape(16, P.per_wave)
        width_byte = np.zeros(16 * P.per_wave, np.uint8)
        for w in range(16):
            for j in range(P.per_wave):
                width_byte[w + 16 * j] = meta[w, j]
        npass = int(np.argmin(width_byte != 0))
        assert npass >= 1 and not width_byte[npass:].any() and npass <= P.passes
        assert np.all(np.diff(width_byte[:npass].astype(int)) >= 0)  # widths 1, 2, 4, 8 in order
        last = {}
        for p in range(npass):
            c = int(width_byte[p]) - 1
            wbits, per = 1 << c, 128 >> c
            rec = buf[base + p * 1536:base + (p + 1) * 1536]
            # group k's word repeated in the 2^c slots k 2^c .. (k + 1) 2^c - 1
            slots = rec[1024:1536].view(np.uint32).reshape(per, 1 << c)
            assert np.all(slots == slots[:, :1])
            words = slots[:, 0]
            for k in range(per):
                e = int(words[k]) >> 16
                code = rec[k * 8 * wbits:(k + 1) * 8 * wbits]
                if e == S * G:  # an empty place
                    assert int(words[k]) & 0xFFFF == 0 and not code.any()
                    continue
                col, row = e // S, e % S
                assert row < R and col < G
                n = n0 + row
                assert int(bits[n, col]) == wbits
                assert int(words[k]) & 0xFFFF == int(s[n, col])
                assert code.tobytes() == mini_oracle.group_bytes(q[n, 64 * col:64 * col + 64], wbits)
                key = (col, row)
                assert last.get(c, (-1, -1)) < key  # (column, row) ascend within a width
                last[c] = key
                seen[n, col] += 1
    assert np.all(seen == 1)
