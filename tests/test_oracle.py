"""Pins for the CPU oracle: each test ties it to something other than itself.

* fp16 decoding: exhaustively against numpy's float16 (an independent library).
* fp16 rounding: against numpy's float64 -> float16 conversion.
* packing: byte strings derived by hand from the layout rules (tests/golden).
* dequant: closed forms of w = s * (q - (2^b - 1)/2) per width, antisymmetry,
  exactness in fp32.
* GEMV: brute force in exact rational arithmetic on tiny inputs, closed forms
  for x = 1 and unit vectors, exact linearity, and the all-8-bit / all-4-bit
  special cases (textbook symmetric uniform quantization) against numpy's
  float64 matmul.

Group size 64 and widths {1,2,4,8}: "Variable Bit-width Quantization" page,
Abstract.  Dequant rule, scale format and layout are the build's readings.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from decode_gemv_vbq_amd import workload as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f16(v):
    return np.array(v, dtype=np.float16).view(np.uint16)


# ------------------------------------------------------------------ fp16

def test_f16_decode_exhaustive():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_f16_round_matches_numpy():
    r = np.random.default_rng(7)
    vals = np.concatenate([
        r.normal(0, 1, 4000),
        r.normal(0, 1e-5, 2000),           # subnormal range
        r.normal(0, 3e4, 2000),            # near overflow
        np.ldexp(r.integers(1, 4096, 2000).astype(np.float64), r.integers(-30, 8, 2000)),
    ])
    # exact ties: midpoints between neighbouring fp16 values
    h = np.arange(0x0001, 0x7bff, 37, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    vals = np.concatenate([vals, (lo + hi) / 2, -(lo + hi) / 2, [65504.0, 65519.99, 65520.0, 1e6, -0.0, 0.0]])
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f64_to_f16(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


# -------------------------------------------------------------- packing

def _golden_group_rows():
    rows = []
    with open(os.path.join(GOLDEN, "group_codes.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            b, rule, hexs = line.split()
            rows.append((int(b), rule, bytes.fromhex(hexs)))
    return rows


def _codes_for(rule):
    j = np.arange(64)
    return {
        "alt": j % 2, "firsthalf": (j < 32).astype(int), "only16": (j == 16).astype(int),
        "only33": (j == 33).astype(int), "mod4": j % 4, "mod16": j % 16, "iota": j,
    }[rule].astype(np.uint8)


@pytest.mark.parametrize("b,rule,expect", _golden_group_rows())
def test_group_encoding_golden(b, rule, expect):
    q = _codes_for(rule).reshape(1, 64)
    bits = np.array([[b]], np.uint8)
    blob = oracle.pack(q, bits, f16([[1.0]]))
    h = oracle.header(blob)
    got = blob[h["off_codes"]:h["off_codes"] + 8 * b].tobytes()
    assert got == expect
    # padding of the 128-byte row record is zero
    assert not blob[h["off_codes"] + 8 * b:h["total_bytes"]].any()


def test_blob_golden_1x128():
    total = None
    expect = None
    with open(os.path.join(GOLDEN, "blob_1x128.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            if parts[0] == "total":
                total = int(parts[1])
                expect = np.zeros(total, np.uint8)
                continue
            off = int(parts[0])
            data = bytes.fromhex("".join(parts[1:]))
            expect[off:off + len(data)] = np.frombuffer(data, np.uint8)
    q = np.zeros((1, 128), np.uint8)
    q[0, :64] = np.arange(64)
    q[0, 64:] = 1
    bits = np.array([[8, 1]], np.uint8)
    blob = oracle.pack(q, bits, np.array([[0x3C00, 0x4000]], np.uint16))
    assert blob.size == total
    assert np.array_equal(blob, expect)


def _adversarial_cases():
    r = np.random.default_rng(11)
    cases = []
    for N, K in [(1, 64), (1, 128), (3, 768), (5, 2112), (4, 4096), (7, 2048 + 64 * 5)]:
        G = K // 64
        for kind in ("random", "allmax", "alternate", "all8", "all1"):
            if kind == "random":
                bits = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, G))
            elif kind == "alternate":
                bits = np.tile(np.array([1, 8, 2, 4], np.uint8), (N, (G + 3) // 4))[:, :G]
            elif kind == "all8":
                bits = np.full((N, G), 8, np.uint8)
            elif kind == "all1":
                bits = np.full((N, G), 1, np.uint8)
            else:
                bits = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, G))
            mx = (np.left_shift(1, bits.astype(np.int32)) - 1).astype(np.uint8)
            if kind == "allmax":
                q = np.repeat(mx, 64, axis=1)
            else:
                q = (r.integers(0, 256, (N, K)) & np.repeat(mx, 64, axis=1)).astype(np.uint8)
            s = r.integers(0, 65536, (N, G)).astype(np.uint16)  # any bit pattern, NaNs included
            cases.append((kind, q, bits, s))
    return cases


@pytest.mark.parametrize("case", _adversarial_cases(), ids=lambda c: f"{c[0]}-{c[1].shape}")
def test_pack_unpack_roundtrip(case):
    _, q, bits, s = case
    blob = oracle.pack(q, bits, s)
    q2, b2, s2 = oracle.unpack(blob)
    assert np.array_equal(q, q2) and np.array_equal(bits, b2) and np.array_equal(s, s2)
    h = oracle.header(blob)
    N, K = q.shape
    assert h["code_bytes"] == int(8 * bits.astype(np.int64).sum())
    # row records are 128-byte multiples and rows are ordered
    row_off = blob[h["off_row_off"]:h["off_row_off"] + 4 * (N + 1)].view(np.uint32)
    assert row_off[0] == 0 and np.all(np.diff(row_off.astype(np.int64)) >= 1)
    assert h["total_bytes"] == h["off_codes"] + 128 * int(row_off[-1])
    for off in ("off_row_off", "off_slice_off", "off_wmap", "off_scales", "off_codes"):
        assert h[off] % 256 == 0


def test_pack_rejects_bad_inputs():
    q = np.zeros((1, 64), np.uint8)
    with pytest.raises(oracle.OracleError) as e:
        oracle.pack(q, np.array([[3]], np.uint8), f16([[1.0]]))
    assert e.value.rc == -2
    q[0, 5] = 2
    with pytest.raises(oracle.OracleError) as e:
        oracle.pack(q, np.array([[1]], np.uint8), f16([[1.0]]))
    assert e.value.rc == -3
    with pytest.raises(oracle.OracleError):
        oracle.pack(np.zeros((1, 96), np.uint8), np.array([[1]], np.uint8), f16([[1.0]]))


# -------------------------------------------------------------- dequant

@pytest.mark.parametrize("b,expect", [
    (1, [-0.5, 0.5]),
    (2, [-1.5, -0.5, 0.5, 1.5]),
    (4, [q - 7.5 for q in range(16)]),
    (8, [q - 127.5 for q in range(256)]),
])
def test_dequant_closed_forms(b, expect):
    levels = len(expect)
    q = (np.arange(64) % levels).astype(np.uint8).reshape(1, 64)
    for s in (1.0, 0.5, -3.0, 0.0183):
        w = oracle.dequant(q, np.array([[b]], np.uint8), f16([[s]]))
        sv = float(np.float16(s))
        assert np.array_equal(w[0], np.array([sv * expect[k % levels] for k in range(64)], np.float32))
    # the page-specified 8-bit extremes at s = 1
    if b == 8:
        q8 = np.array([[127, 128, 0, 255] + [0] * 60], np.uint8)
        w = oracle.dequant(q8, np.array([[8]], np.uint8), f16([[1.0]]))
        assert list(w[0, :4]) == [-0.5, 0.5, -127.5, 127.5]


def test_dequant_invariants_and_special_scales():
    r = np.random.default_rng(3)
    N, K = 16, 512
    bits = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, K // 64))
    mx = np.repeat((np.left_shift(1, bits.astype(np.int32)) - 1), 64, axis=1)
    q = (r.integers(0, 256, (N, K)) & mx).astype(np.uint8)
    s = np.exp(r.normal(-4, 0.5, (N, K // 64))).astype(np.float16).view(np.uint16)
    w = oracle.dequant(q, bits, s).astype(np.float64)
    wa = oracle.dequant((mx - q).astype(np.uint8), bits, s).astype(np.float64)
    assert np.array_equal(w, -wa)                                   # antisymmetry
    sv = np.repeat(s.view(np.float16).astype(np.float64), 64, axis=1)
    odd = 2 * w / sv
    assert np.array_equal(odd, np.round(odd)) and np.all(np.abs(odd) % 2 == 1)
    assert np.all(np.abs(odd) <= mx)
    # special scales: zeros keep their sign, inf gives inf (no zero level), NaN propagates
    q1 = np.zeros((1, 64 * 6), np.uint8)
    q1[0, ::2] = 1
    b1 = np.ones((1, 6), np.uint8)
    sp = np.array([[0x0000, 0x8000, 0x7C00, 0xFC00, 0x7E00, 0x0001]], np.uint16)
    w = oracle.dequant(q1, b1, sp)
    g = w.reshape(6, 64)
    # q = 1 on even positions: +0 * (+1/2) = +0, +0 * (-1/2) = -0; the -0 scale flips both
    assert np.all(g[0] == 0) and np.array_equal(np.signbit(g[0]), np.tile([False, True], 32))
    assert np.array_equal(np.signbit(g[1]), np.tile([True, False], 32))
    assert np.all(np.isinf(g[2])) and np.all(np.isinf(g[3])) and np.all(np.isnan(g[4]))
    assert np.array_equal(np.abs(g[5]), np.full(64, 2.0 ** -25, np.float32))  # subnormal fp16 scale
    w16 = oracle.dequant(q1, b1, sp, dtype=np.float16)
    assert np.array_equal(w16, w.astype(np.float16).view(np.uint16))


def test_dequant_f16_is_rne_of_f32():
    r = np.random.default_rng(5)
    bits = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(8, 8))
    q = (r.integers(0, 256, (8, 512)) & np.repeat(np.left_shift(1, bits.astype(np.int32)) - 1, 64, 1)).astype(np.uint8)
    s = r.integers(0, 0x7C00, (8, 8)).astype(np.uint16)   # finite positive patterns, subnormals included
    w32 = oracle.dequant(q, bits, s)
    w16 = oracle.dequant(q, bits, s, dtype=np.float16)
    assert np.array_equal(w16, w32.astype(np.float16).view(np.uint16))


# -------------------------------------------------------------- GEMV

def _frac_gemv(q, bits, s, x):
    """Exact rational y and bound on tiny inputs (brute force)."""
    N, K = q.shape
    ys, bs = [], []
    for n in range(N):
        acc = Fraction(0)
        mag = Fraction(0)
        for k in range(K):
            b = int(bits[n, k // 64])
            sv = Fraction(float(np.uint16(s[n, k // 64]).view(np.float16)))
            w = sv * (Fraction(int(q[n, k])) - Fraction(2 ** b - 1, 2))
            xv = Fraction(float(np.uint16(x[k]).view(np.float16)))
            acc += w * xv
            mag += abs(w) * abs(xv)
        ys.append(acc)
        bs.append(mag)
    return ys, bs


@pytest.mark.parametrize("K", [64, 128, 256])
def test_gemv_brute_force_fraction(K):
    r = np.random.default_rng(K)
    N = 4
    bits = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, K // 64))
    bits[0, 0] = 1
    bits[-1, -1] = 8
    q = (r.integers(0, 256, (N, K)) & np.repeat(np.left_shift(1, bits.astype(np.int32)) - 1, 64, 1)).astype(np.uint8)
    s = np.exp(r.normal(-4, 0.5, (N, K // 64))).astype(np.float16).view(np.uint16)
    x = r.normal(0, 1, K).astype(np.float16).view(np.uint16)
    y, bound = oracle.gemv(q, bits, s, x)
    ey, eb = _frac_gemv(q, bits, s, x)
    for n in range(N):
        assert abs(Fraction(y[0, n]) - ey[n]) <= abs(ey[n]) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)
        assert abs(Fraction(bound[0, n]) - eb[n]) <= eb[n] * Fraction(1, 2 ** 50)


def test_gemv_golden_values():
    # 1x64, b=1, all q=1, s=0.5, x=1 -> 64 * 0.5 * 0.5 = 16
    y, b = oracle.gemv(np.ones((1, 64), np.uint8), np.array([[1]], np.uint8), f16([[0.5]]), f16(np.ones(64)))
    assert y[0, 0] == 16.0 and b[0, 0] == 16.0
    # 1x128, g0 (b=1, q=0, s=1), g1 (b=8, q=255, s=1), x=1 -> -32 + 8160
    q = np.zeros((1, 128), np.uint8)
    q[0, 64:] = 255
    y, b = oracle.gemv(q, np.array([[1, 8]], np.uint8), f16([[1.0, 1.0]]), f16(np.ones(128)))
    assert y[0, 0] == 8128.0 and b[0, 0] == 8192.0


def test_gemv_closed_form_ones_and_unit_vectors():
    r = np.random.default_rng(9)
    N, K = 6, 640
    bits = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, K // 64))
    mx = np.repeat(np.left_shift(1, bits.astype(np.int64)) - 1, 64, 1)
    q = (r.integers(0, 256, (N, K)) & mx).astype(np.uint8)
    s = np.exp(r.normal(-4, 0.5, (N, K // 64))).astype(np.float16).view(np.uint16)
    y, _ = oracle.gemv(q, bits, s, f16(np.ones(K)))
    sv = s.view(np.float16).astype(np.float64)
    qsum = q.astype(np.int64).reshape(N, K // 64, 64).sum(-1)
    expect = (sv * (qsum - 32 * (np.left_shift(1, bits.astype(np.int64)) - 1))).sum(-1)
    assert np.allclose(y[0], expect, rtol=1e-14, atol=0)
    # a 1-bit row with x = 1 gives s * (popcount - 32)
    b1 = np.ones((1, 1), np.uint8)
    q1 = (r.integers(0, 2, (1, 64))).astype(np.uint8)
    y1, _ = oracle.gemv(q1, b1, f16([[0.25]]), f16(np.ones(64)))
    assert y1[0, 0] == 0.25 * (int(q1.sum()) - 32)
    # x = e_k gives column k of the dequantized matrix, exactly
    w = oracle.dequant(q, bits, s).astype(np.float64)
    for k in (0, 63, 64, 300, K - 1):
        e = np.zeros(K)
        e[k] = 1.0
        yk, _ = oracle.gemv(q, bits, s, f16(e))
        assert np.array_equal(yk[0], w[:, k])


def test_gemv_linearity_exact():
    r = np.random.default_rng(13)
    N, K = 5, 384
    bits = r.choice(np.array([1, 2, 4, 8], np.uint8), size=(N, K // 64))
    q = (r.integers(0, 256, (N, K)) & np.repeat(np.left_shift(1, bits.astype(np.int32)) - 1, 64, 1)).astype(np.uint8)
    s = np.exp(r.normal(-4, 0.5, (N, K // 64))).astype(np.float16).view(np.uint16)
    x = r.normal(0, 1, (2, K)).astype(np.float16)
    y, b = oracle.gemv(q, bits, s, x.view(np.uint16))
    y2, b2 = oracle.gemv(q, bits, s, (x * np.float16(4)).view(np.uint16))
    assert np.array_equal(y2, 4 * y) and np.array_equal(b2, 4 * b)
    yn, _ = oracle.gemv(q, bits, s, (-x).view(np.uint16))
    assert np.array_equal(yn, -y)


@pytest.mark.parametrize("b", [4, 8])
def test_gemv_uniform_quantization_matches_library_matmul(b):
    """All groups at one width is textbook symmetric uniform quantization."""
    r = np.random.default_rng(b)
    N, K, M = 32, 1024, 3
    q = r.integers(0, 2 ** b, (N, K)).astype(np.uint8)
    bits = np.full((N, K // 64), b, np.uint8)
    s = np.exp(r.normal(-4, 0.5, (N, K // 64))).astype(np.float16)
    x = r.normal(0, 1, (M, K)).astype(np.float16)
    w = np.repeat(s.astype(np.float64), 64, axis=1) * (q.astype(np.float64) - (2 ** b - 1) / 2)
    ref = x.astype(np.float64) @ w.T
    y, bound = oracle.gemv(q, bits, s.view(np.uint16), x.view(np.uint16))
    mag = np.abs(x.astype(np.float64)) @ np.abs(w).T
    assert np.all(np.abs(y - ref) <= 1e-12 * mag)
    assert np.allclose(bound, np.abs(x.astype(np.float64)) @ np.abs(w).T, rtol=1e-13)


def test_gemv_blob_equals_gemv():
    spec = wl.MatrixSpec("t", 24, 2048 + 320, wl.MIX_BASE)
    q, bits, s, x = wl.draw_matrix(spec, 99, M=3)
    y1, b1 = oracle.gemv(q, bits, s, x)
    y2, b2 = oracle.gemv_blob(oracle.pack(q, bits, s), x)
    assert np.array_equal(y1, y2) and np.array_equal(b1, b2)


def test_dense_gemv_matches_vbq_on_dequantized_weights():
    spec = wl.MatrixSpec("t", 16, 512, wl.MIX_BASE)
    q, bits, s, x = wl.draw_matrix(spec, 98, M=2)
    w32 = oracle.dequant(q, bits, s)
    w16 = w32.astype(np.float16)
    exact16 = np.array_equal(w16.astype(np.float32), w32)
    yd, bd = oracle.dense_gemv(w16.view(np.uint16), x)
    yv, bv = oracle.gemv(q, bits, s, x)
    if exact16:
        assert np.array_equal(yd, yv)
    assert np.all(np.abs(yd - yv) <= 2 ** -10 * bv)


def test_workload_statistics():
    """The synthetic draws follow the stated mixtures (sanity of the generator)."""
    spec = wl.MatrixSpec("t", 4096, 2048, wl.MIX_BASE)
    bits = wl.draw_bits(spec, 1)
    frac = {w: float((bits == w).mean()) for w in (1, 2, 4, 8)}
    for w, p in wl.MIX_BASE.items():
        assert abs(frac[w] - p) < 0.01
    cl = wl.MatrixSpec("c", 64, 8192, wl.MIX_BASE, cluster=8)
    bc = wl.draw_bits(cl, 1)
    assert np.all(bc.reshape(64, -1, 8) == bc.reshape(64, -1, 8)[:, :, :1])
    q = wl.draw_codes(spec, 1, bits)
    assert np.all(q <= np.repeat(np.left_shift(1, bits.astype(np.int32)) - 1, 64, 1))
    x = wl.draw_x(wl.MatrixSpec("x", 1, 8192, wl.MIX_BASE), 1, 2, outliers=0.01)
    big = (np.abs(x.view(np.float16).astype(np.float64)) > 8).any(0).sum()
    assert 40 <= big <= 82
