"""GPU parity of the prefill GEMM (vbq_gemm_plan_init / vbq_gemm_prepare /
vbq_gemm) against the CPU oracle, on the same seeded inputs.

* |y - y_ref| <= 1e-3 * sum|w||x| + 2^-24 * sum|x| per output (the GEMM feeds
  the matrix cores fp16(s * (q - c)); the second term is the fp16 subnormal
  spacing), at shapes that span one chunk, odd group counts (a last chunk of
  one group), ragged row blocks and token blocks, K-splits and every width mix.
* x = e_k gives fp16(w[:, k]) bit-exactly (the dequantized weight of column k,
  as vbq_dequant rounds it): this pins the k-slot order and the fp16 rounding.
* Repeated calls are bit-identical; strided x / y are honoured.
* The plan buffer read back on the host describes every group of the matrix
  once, with the blob's code record and scale.
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
    spec = wl.MatrixSpec("t", N, K, mix or wl.MIX_BASE, layer=seed, cluster=cluster)
    return wl.draw_matrix(spec, 93, M=M, outliers=outliers)


def gemm_bound(bound, x):
    """1e-3 * sum|w||x| + 2^-24 * sum|x| per output (x: fp16 bits [M][K])."""
    ax = np.abs(np.atleast_2d(x).view(np.float16).astype(np.float64)).sum(axis=1)
    return 1e-3 * bound + 2.0 ** -24 * ax[:, None]


def run_gemm(v, q, bits, s, x, yt="f32"):
    dq, db, ds, dx = upload(q, bits, s, x, torch)
    blob, L = v.pack(dq, db, ds)
    buf, GP = v.gemm_prepare(L, blob)
    out_dtype = torch.float16 if yt == "f16" else torch.float32
    y = v.gemm(GP, buf, dx, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), (blob, L, buf, GP, dx)


def check(y, q, bits, s, x, what, f16_out=False):
    y_ref, bound = oracle.gemv(q, bits, s, x)
    b = gemm_bound(bound, x)
    if f16_out:  # one more rounding of the output to fp16
        b = b + np.abs(y_ref) * 2.0 ** -11 + 2.0 ** -25
        b = np.where(np.abs(y_ref) > 65504, np.inf, b)
    ok, worst, idx = within_bound(y, y_ref, b, rel=1.0)
    assert ok, f"{what}: worst err/bound={worst:.3g} at {idx}"
    return worst


# (N, K, M): one chunk; one group (a chunk of one group); odd G; ragged row
# blocks; one, two and five token blocks of each tile height; K-splits (few
# row blocks, many chunks); K = 28672
CASES = [
    (1, 64, 17), (3, 128, 33), (128, 128, 32), (130, 192, 40), (257, 64 * 9, 65), (300, 448, 129),
    (256, 4096, 64), (1000, 5632, 100), (129, 28672, 20), (64, 2048, 1), (2000, 64, 17), (77, 64 * 33, 300),
]


@pytest.mark.parametrize("N,K,M", CASES)
def test_gemm_parity(N, K, M):
    v = vbq()
    q, bits, s, x = draw(N, K, seed=N + K + M, M=M, outliers=0.01)
    y, _ = run_gemm(v, q, bits, s, x)
    worst = check(y, q, bits, s, x, f"N={N} K={K} M={M}")
    print(f"N={N} K={K} M={M}: worst err/bound {worst:.2e}")


@pytest.mark.parametrize("mix", ["u1", "u2", "u4", "u8", "wide", "head"])
def test_gemm_width_mixes(mix):
    v = vbq()
    m = {"u1": {1: 1.0}, "u2": {2: 1.0}, "u4": wl.MIX_U4, "u8": wl.MIX_U8, "wide": wl.MIX_WIDE,
         "head": wl.MIX_HEAD}[mix]
    for M in (24, 100):
        q, bits, s, x = draw(300, 64 * 37, m, seed=17, M=M, cluster=8 if mix == "wide" else 1)
        y, (_, _, _, GP, _) = run_gemm(v, q, bits, s, x)
        check(y, q, bits, s, x, f"{mix} M={M} slot={GP.slot_bytes}")


def test_gemm_f16_output_and_strides():
    v = vbq()
    N, K, M = 333, 64 * 41, 70
    q, bits, s, x = draw(N, K, seed=5, M=M)
    dq, db, ds, dx = upload(q, bits, s, x, torch)
    blob, L = v.pack(dq, db, ds)
    buf, GP = v.gemm_prepare(L, blob)
    xs = torch.zeros((M, K + 24), dtype=torch.float16, device="cuda")
    xs[:, :K] = dx
    out = torch.full((M, N + 10), float("nan"), dtype=torch.float32, device="cuda")
    v.gemm(GP, buf, xs[:, :K], out=out[:, :N])
    y16 = v.gemm(GP, buf, dx, out_dtype=torch.float16)
    y2 = v.gemm(GP, buf, dx, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out[:, :N], y2)
    assert bool(torch.isnan(out[:, N:]).all())  # nothing written past the used part of each row
    assert torch.equal(y16, y2.half())           # the same fp32 sums, rounded once
    check(y2.cpu().numpy().astype(np.float64), q, bits, s, x, "strided")


def test_gemm_unit_vectors_give_fp16_dequant_columns():
    v = vbq()
    N, K = 200, 64 * 75
    q, bits, s, _ = draw(N, K, seed=31)
    dq, db, ds, _ = upload(q, bits, s, np.zeros((1, K), np.uint16), torch)
    blob, L = v.pack(dq, db, ds)
    w16 = v.dequant(L, blob, torch.float16)
    buf, GP = v.gemm_prepare(L, blob)
    ks = [0, 1, 31, 32, 33, 63, 64, 95, 96, 127, 128, 2047, 2048, 2111, K - 65, K - 64, K - 33, K - 1]
    X = torch.zeros((len(ks), K), dtype=torch.float16, device="cuda")
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    Y = v.gemm(GP, buf, X, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for i, k in enumerate(ks):
        assert torch.equal(Y[i], w16[:, k].float()), f"column {k}"


def test_gemm_special_scales():
    v = vbq()
    N, K, M = 40, 64 * 70, 20
    q, bits, s, x = draw(N, K, seed=21, M=M)
    s = s.copy()
    s[0, :] = 0x0000           # +0
    s[1, :] = 0x8000           # -0
    s[2, 3] = 0x0001           # smallest subnormal
    s[3, :] = 0x03FF           # largest subnormal
    s[4, :] = 0xAC00           # negative
    s[5, 7] = 0x7C00           # +inf
    s[6, 40] = 0xFC00          # -inf
    s[7, 65] = 0x7E00          # NaN
    s[8, :] = 0x5800           # 128: the largest weights stay inside the fp16 range
    y, _ = run_gemm(v, q, bits, s, x)
    check(y, q, bits, s, x, "special scales")
    assert np.all(y[:, :2] == 0)


def test_gemm_weights_beyond_fp16_range_give_nonfinite_outputs():
    v = vbq()
    N, K, M = 8, 128, 17
    q, bits, s, x = draw(N, K, seed=3, M=M)
    bits = bits.copy()
    q = q.copy()
    s = s.copy()
    bits[0, 0] = 8
    q[0, :64] = 255                  # q - c = 127.5
    s[0, 0] = 0x7BFF                 # 65504: w = 8.35e6, beyond fp16
    x = x.copy()
    x[:, 0] = 0x3C00                 # x = 1 on that column
    y, _ = run_gemm(v, q, bits, s, x)
    assert not np.isfinite(y[:, 0]).any()
    check(y[:, 1:], q[1:], bits[1:], s[1:], x, "other rows")


def test_gemm_deterministic():
    v = vbq()
    N, K, M = 129, 28672, 40       # K-split launch
    q, bits, s, x = draw(N, K, seed=9, M=M)
    y, (blob, L, buf, GP, dx) = run_gemm(v, q, bits, s, x)
    ws = v.gemm_workspace(GP, M)
    for _ in range(3):
        y2 = v.gemm(GP, buf, dx, out_dtype=torch.float32, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(y2.cpu().numpy().astype(np.float64), y)
    check(y, q, bits, s, x, "K-split")


def test_gemm_plan_buffer_describes_every_group_once():
    v = vbq()
    N, K = 300, 64 * 9
    q, bits, s, x = draw(N, K, wl.MIX_WIDE, seed=11)
    dq, db, ds, _ = upload(q, bits, s, x, torch)
    blob, L = v.pack(dq, db, ds)
    buf, GP = v.gemm_prepare(L, blob)
    torch.cuda.synchronize()
    B = buf.cpu().numpy()
    ref = oracle.pack(q, bits, s)
    h = oracle.header(ref)
    assert np.array_equal(blob.cpu().numpy(), ref)
    G = K // 64
    table = B[:GP.table_bytes].view(np.uint32)
    nt = GP.nb * GP.kc
    seen = np.zeros((N, G), np.int32)
    # the blob's code record of every group, from the oracle's own packer
    rec = {}
    for n in range(N):
        for g in range(G):
            b = int(bits[n, g])
            one = np.zeros((1, 64), np.uint8)
            one[0] = q[n, 64 * g:64 * g + 64]
            blob1 = oracle.pack(one, np.array([[b]], np.uint8), np.array([[0]], np.uint16))
            h1 = oracle.header(blob1)
            rec[n, g] = blob1[h1["off_codes"]:h1["off_codes"] + 8 * b]
    assert h["N"] == N
    for i in range(GP.nb):
        for j in range(GP.kc):
            t0 = 16 * int(table[i * GP.kc + j])
            t1 = 16 * int(table[i * GP.kc + j + 1])
            hd = B[t0:t0 + 16].view(np.uint32)
            cnt = [int(hd[0] & 0xFFFF), int(hd[0] >> 16), int(hd[1] & 0xFFFF), int(hd[1] >> 16)]  # 8,4,2,1 bits
            assert int(hd[2]) == t1 - t0
            se_off = int(hd[3])
            words = B[t0 + se_off:t0 + se_off + 4 * sum(cnt)].view(np.uint32)
            off = t0 + 16
            slot = 0
            for w, c in zip((8, 4, 2, 1), cnt):
                for _ in range(c):
                    pos = int(words[slot] >> 16)
                    r, gl = pos & 127, pos >> 7
                    n, g = 128 * i + r, 2 * j + gl
                    assert bits[n, g] == w
                    assert int(words[slot] & 0xFFFF) == int(s[n, g])
                    assert np.array_equal(B[off:off + 8 * w], rec[n, g])
                    seen[n, g] += 1
                    off += 8 * w
                    slot += 1
            assert off == t0 + se_off
    assert np.all(seen == 1)
    assert int(table[nt]) * 16 + GP.slot_bytes == GP.total_bytes
