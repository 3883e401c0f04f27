"""The C oracle against the independent numpy statement in tests/mini_oracle.py: the
packed blob byte for byte, the fp32 dequant exactly, the GEMV to fp64 rounding, on
random matrices up to 256 x 512 with every width (several 32-group slices, a ragged
last slice, one group)."""
import numpy as np
import pytest

import oracle
from tests import mini_oracle

WIDTHS = np.array([1, 2, 4, 8], np.uint8)


def draw(N, K, seed, mix=None):
    r = np.random.default_rng(seed)
    G = K // 64
    bits = r.choice(WIDTHS, (N, G), p=mix)
    top = (1 << bits.astype(np.int64)) - 1
    q = (r.integers(0, 256, (N, G, 64)) % (top[..., None] + 1)).astype(np.uint8).reshape(N, K)
    s = (np.exp(r.normal(-4, 0.5, (N, G))) * r.choice([-1, 1], (N, G))).astype(np.float16).view(np.uint16)
    x = r.standard_normal((3, K)).astype(np.float16).view(np.uint16)
    return q, bits, s, x


@pytest.mark.parametrize("N,K,seed", [(1, 64, 0), (4, 128, 1), (17, 64 * 33, 2), (64, 512, 3), (256, 512, 4),
                                      (9, 64 * 70, 5), (33, 64 * 96, 6)])
def test_pack_dequant_gemv_agree(N, K, seed):
    q, bits, s, x = draw(N, K, seed)
    blob = oracle.pack(q, bits, s)
    assert np.array_equal(blob, mini_oracle.pack(q, bits, s))
    w = oracle.dequant(q, bits, s).astype(np.float64)
    assert np.array_equal(w, mini_oracle.dequant(q, bits, s))
    y, _ = oracle.gemv(q, bits, s, x)
    y2 = mini_oracle.gemv(q, bits, s, x)
    scale = np.abs(np.atleast_2d(x).view(np.float16).astype(np.float64)) @ np.abs(w).T
    assert np.all(np.abs(y - y2) <= 1e-12 * scale + 1e-300)


@pytest.mark.parametrize("mix", [[1, 0, 0, 0], [0, 0, 0, 1], [0.25, 0.25, 0.25, 0.25]])
def test_pack_agrees_for_uniform_and_even_mixes(mix):
    q, bits, s, _ = draw(40, 64 * 40, 7, mix)
    assert np.array_equal(oracle.pack(q, bits, s), mini_oracle.pack(q, bits, s))
