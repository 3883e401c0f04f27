"""CPU checks of the byte accounting behind bench.py's GB/s figures.

The metric counts, per GEMV, the packed code bytes (sum of 8*b over the groups, row
padding excluded), fp16 scales, the offset tables the kernels read, and the activations.
Here the layout sizes come from the oracle's own packer (independent of the library) and
the counts are compared with direct sums over the width map.
"""
import types

import numpy as np
import pytest

import oracle
from decode_gemv_vbq_amd import accounting as acc

WIDTHS = np.array([1, 2, 4, 8], np.uint8)


def layout_ns(N, K, bits):
    h = oracle.layout(N, K, bits)
    return types.SimpleNamespace(N=N, K=K, G=K // 64, nS=h["nS"], code_bytes=h["code_bytes"],
                                 code_bytes_padded=h["code_bytes_padded"])


@pytest.mark.parametrize("N,K,seed", [(1, 64, 0), (7, 2048 + 64, 1), (64, 4096, 2), (33, 64 * 33, 3)])
def test_read_bytes_match_direct_sums(N, K, seed):
    r = np.random.default_rng(seed)
    bits = r.choice(WIDTHS, (N, K // 64))
    L = layout_ns(N, K, bits)
    codes = int((8 * bits.astype(np.int64)).sum())
    assert L.code_bytes == codes
    # each row's code record padded to 128 bytes
    rows = (8 * bits.astype(np.int64)).sum(axis=1)
    assert L.code_bytes_padded == int(((rows + 127) // 128 * 128).sum())
    nS = -(-(K // 64) // 32)
    for M in (1, 16):
        want = codes + 2 * N * (K // 64) + 4 * (N + 1) + 4 * N * nS + 8 * N * nS + 2 * M * K
        assert acc.vbq_read_bytes(L, M) == want
        assert acc.vbq_layout_bytes(L, M) - acc.vbq_read_bytes(L, M) == L.code_bytes_padded - codes
    assert acc.dense_read_bytes(N, K, 3) == 2 * N * K + 6 * K
    assert acc.write_bytes(N, 4) == 8 * N


def test_bench_refuses_more_than_one_gpu(capsys):
    import bench
    with pytest.raises(SystemExit) as e:
        bench.main(["--gpus", "2"])
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().out


@pytest.mark.parametrize("name", ["linear768", "mlp1b", "decode1b", "decode9b"])
def test_cold_copies_stream_past_the_memory_side_cache(name):
    """A workload below the 256 MB memory-side cache runs as copies in turn that
    stream at least 512 MB of codes and scales per step; larger ones run once."""
    import bench
    from decode_gemv_vbq_amd import workload as wl
    W = wl.workload(name)
    c = bench.cold_copies(W)
    packed = sum(sp.N * sp.K * sum(b * f for b, f in sp.mix.items()) / 8 + 2 * sp.N * sp.G for sp in W.mats)
    if packed >= 256e6:
        assert c == 1
    else:
        assert c > 1 and c * packed >= 512e6 and (c - 1) * packed < 512e6
