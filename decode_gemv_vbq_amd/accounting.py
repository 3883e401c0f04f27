"""Byte accounting of one VBQ GEMV (what the metric counts as algorithmic bytes).

Algorithmic bytes read per GEMV over an N x K VBQ1 matrix with M tokens:
  packed codes (sum of 8*b over groups, row padding excluded)
  + fp16 scales (2*N*G)
  + offset tables the kernel reads (row_off 4*(N+1), slice_off 4*N*nS,
    width bit planes 8*N*nS)
  + activations (2*M*K)
Output writes (2*M*N for fp16 y) are reported apart.  The dense fp16 control
reads 2*N*K weight bytes + 2*M*K activation bytes.
"""
from __future__ import annotations


def vbq_read_bytes(L, M: int = 1) -> int:
    N, K, G, nS = L.N, L.K, L.G, L.nS
    return int(L.code_bytes + 2 * N * G + 4 * (N + 1) + 4 * N * nS + 8 * N * nS + 2 * M * K)


def vbq_layout_bytes(L, M: int = 1) -> int:
    """Same with the 128-byte row padding of the code records included."""
    return vbq_read_bytes(L, M) - int(L.code_bytes) + int(L.code_bytes_padded)


def dense_read_bytes(N: int, K: int, M: int = 1) -> int:
    return 2 * N * K + 2 * M * K


def write_bytes(N: int, M: int = 1, out_bytes: int = 2) -> int:
    return out_bytes * M * N
