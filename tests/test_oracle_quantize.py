"""Pins of the oracle's round-to-nearest quantizer (oracle.quantize).

The pages learn VBQ's scales in training and give no rule for turning float
weights into codes; the quantizer is the plain reading (per group of 64, with
c = (2^b - 1)/2: s = fp16(max|w| / c), q = clamp(rint(w/s + c), 0, 2^b - 1),
each step one IEEE fp32 operation).  It is pinned here by
  * hand-derived worked examples, one per width;
  * exact recovery: weights that are themselves s*(q - c) for a power-of-two s,
    with an extreme code in every group, quantize back to the same q and s;
  * the round-to-nearest bound |w - s(q - c)| <= s/2 for weights inside the
    representable range;
  * a second implementation written here with numpy's own fp32 operations,
    which must agree bit for bit, special values included.
"""
import numpy as np
import pytest

import oracle

WIDTHS = np.array([1, 2, 4, 8], np.uint8)


def np_quantize(w, bits):
    """Independent fp32 statement of the rule with numpy's IEEE operations."""
    w32 = np.asarray(w, dtype=np.float32)
    N, K = w32.shape
    G = K // 64
    wg = w32.reshape(N, G, 64)
    b = bits.astype(np.int64)
    top = ((1 << b) - 1).astype(np.float32)
    c = top / np.float32(2)
    with np.errstate(all="ignore"):
        a = np.fmax(np.float32(0), np.fmax.reduce(np.abs(wg), axis=2))
        s16 = (a / c).astype(np.float32).astype(np.float16)
        s = s16.astype(np.float32)
        u = (wg / s[..., None]).astype(np.float32) + c[..., None]
        q = np.fmin(np.fmax(np.rint(u), np.float32(0)), top[..., None])
    return q.astype(np.uint8).reshape(N, K), s16.view(np.uint16)


def test_worked_examples():
    # b=1: weights +-1 -> a = 1, s = 1/0.5 = 2 (0x4000), w/s + 0.5 = 0 or 1
    w = np.tile(np.array([-1, 1], np.float32), 32)[None]
    q, s = oracle.quantize(w, np.array([[1]], np.uint8))
    assert s[0, 0] == 0x4000 and list(q[0, :4]) == [0, 1, 0, 1]
    # b=2: weights -3, -1, 1, 3 -> s = 3/1.5 = 2, codes 0..3
    w = np.tile(np.array([-3, -1, 1, 3], np.float32), 16)[None]
    q, s = oracle.quantize(w, np.array([[2]], np.uint8))
    assert s[0, 0] == 0x4000 and list(q[0, :4]) == [0, 1, 2, 3]
    # b=4: 0.25*(j - 7.5) for j = 0..15 -> a = 1.875, s = 0.25 (0x3400), codes j
    w = np.tile(0.25 * (np.arange(16, dtype=np.float32) - 7.5), 4)[None]
    q, s = oracle.quantize(w, np.array([[4]], np.uint8))
    assert s[0, 0] == 0x3400 and list(q[0, :16]) == list(range(16))
    # b=8: j - 127.5 for j = 0..63 -> a = 127.5, s = 1 (0x3c00), codes j
    w = (np.arange(64, dtype=np.float32) - 127.5)[None]
    q, s = oracle.quantize(w, np.array([[8]], np.uint8))
    assert s[0, 0] == 0x3C00 and list(q[0]) == list(range(64))
    # values halfway between two levels round to the even code:
    # b=2, s = 2: w = 0 -> 1.5 -> 2; w = 2 -> 2.5 -> 2 (not 3); w = -2 -> 0.5 -> 0
    w = np.zeros((1, 64), np.float32)
    w[0, 0], w[0, 1], w[0, 2], w[0, 3] = 3.0, 0.0, 2.0, -2.0
    q, s = oracle.quantize(w, np.array([[2]], np.uint8))
    assert s[0, 0] == 0x4000 and list(q[0, :4]) == [3, 2, 2, 0]
    # an all-zero group: s = 0 and every quotient 0/0 is NaN -> q = 0
    q, s = oracle.quantize(np.zeros((1, 64), np.float32), np.array([[4]], np.uint8))
    assert s[0, 0] == 0 and not q.any()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_recovery_of_representable_weights(seed):
    r = np.random.default_rng(seed)
    N, G = 24, 10
    bits = r.choice(WIDTHS, (N, G))
    top = (1 << bits.astype(np.int64)) - 1
    q = (r.integers(0, 256, (N, G, 64)) % (top[..., None] + 1)).astype(np.uint8)
    # an extreme code in every group makes max|w| = s*c exactly
    q[:, :, 5] = np.where(r.random((N, G)) < 0.5, 0, top).astype(np.uint8)
    e = r.integers(-12, 6, (N, G))
    s16 = np.ldexp(np.ones((N, G)), e).astype(np.float16)
    q = q.reshape(N, G * 64)
    w = oracle.dequant(q, bits, s16.view(np.uint16))
    q2, s2 = oracle.quantize(w, bits)
    assert np.array_equal(s2, s16.view(np.uint16))
    assert np.array_equal(q2, q)


@pytest.mark.parametrize("seed", [3, 4])
def test_round_to_nearest_bound(seed):
    r = np.random.default_rng(seed)
    N, G = 16, 8
    bits = r.choice(WIDTHS, (N, G))
    w = (r.standard_normal((N, G * 64)) * np.exp(r.standard_normal((N, 1)))).astype(np.float32)
    q, s = oracle.quantize(w, bits)
    top = (1 << bits.astype(np.int64)) - 1
    assert np.all(q.reshape(N, G, 64) <= top[..., None])
    sf = s.view(np.float16).astype(np.float64)
    c = top / 2.0
    wq = sf[..., None] * (q.reshape(N, G, 64).astype(np.float64) - c[..., None])
    err = np.abs(w.reshape(N, G, 64).astype(np.float64) - wq)
    # s is a rounded a/c, so the grid reaches max|w| only up to fp16 rounding:
    # values beyond s*c are clamped to the end level
    a = np.abs(w.reshape(N, G, 64)).max(axis=2)
    slack = np.maximum(a - sf * c, 0)[..., None]
    assert np.all(err <= sf[..., None] * (0.5 + 2 ** -20) + slack)


@pytest.mark.parametrize("seed", [5, 6, 7])
def test_matches_independent_numpy_statement(seed):
    r = np.random.default_rng(seed)
    N, G = 20, 12
    bits = r.choice(WIDTHS, (N, G))
    w = (r.standard_normal((N, G * 64)) * np.exp(3 * r.standard_normal((N, G * 64)))).astype(np.float32)
    # special values: zeros of both signs, an all-zero group, NaN, +-inf, huge,
    # tiny (fp16 scale underflow), fp16-representable
    w[0, :64] = 0.0
    w[1, 3] = -0.0
    w[2, 7] = np.nan
    w[3, 70] = np.inf
    w[4, 9] = -np.inf
    w[5, :64] *= 1e30
    w[6, 64:128] *= 1e-12
    w[7] = w[7].astype(np.float16).astype(np.float32)
    q, s = oracle.quantize(w, bits)
    q2, s2 = np_quantize(w, bits)
    assert np.array_equal(s, s2)
    assert np.array_equal(q, q2)
    # fp16 input is widened exactly
    with np.errstate(over="ignore"):
        w16 = w.astype(np.float16)
    q, s = oracle.quantize(w16, bits)
    q2, s2 = np_quantize(w16.astype(np.float32), bits)
    assert np.array_equal(s, s2) and np.array_equal(q, q2)


def test_rejects_bad_shapes_and_widths():
    with pytest.raises(oracle.OracleError):
        oracle.quantize(np.zeros((2, 96), np.float32), np.ones((2, 1), np.uint8))
    with pytest.raises(oracle.OracleError):
        oracle.quantize(np.zeros((1, 64), np.float32), np.array([[3]], np.uint8))
