"""CPU oracle for the VBQ decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library and its Python binding
never import, link or call it, and it imports nothing from them.

The arithmetic lives in ``vbq_oracle.c`` (plain C, scalar loops, fp64), whose
header states the method it follows ("Variable Bit-width Quantization" page,
Abstract: per-group widths in {1,2,4,8} over contiguous 64-weight groups) and
the readings the build fixes (dequant rule, scale format, packed layout).  This
module only marshals numpy arrays to it through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vbq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ERRORS = {0: "ok", -1: "shape", -2: "bits", -3: "code range", -4: "layout", -5: "size"}


class OracleError(RuntimeError):
    def __init__(self, rc: int, what: str):
        super().__init__(f"oracle {what}: error {rc} ({ERRORS.get(rc, '?')})")
        self.rc = rc


def build() -> str:
    """Compile the oracle with gcc (no HIP); returns the library path."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        u64 = ctypes.c_uint64
        L.vbqo_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.vbqo_f16_to_f64.restype = ctypes.c_double
        L.vbqo_f64_to_f16_rne.argtypes = [ctypes.c_double]
        L.vbqo_f64_to_f16_rne.restype = ctypes.c_uint16
        L.vbqo_layout.argtypes = [i, i, P, P]
        L.vbqo_pack.argtypes = [i, i, P, P, P, P, u64]
        L.vbqo_header.argtypes = [P, u64, P]
        L.vbqo_quantize.argtypes = [i, i, P, i, P, P, P]
        L.vbqo_unpack.argtypes = [P, u64, P, P, P]
        L.vbqo_dequant_f32.argtypes = [i, i, P, P, P, P]
        L.vbqo_dequant_f16.argtypes = [i, i, P, P, P, P]
        L.vbqo_gemv.argtypes = [i, i, i, P, P, P, P, i, P, P]
        L.vbqo_gemv_blob.argtypes = [P, u64, i, P, i, P, P]
        L.vbqo_dense_gemv.argtypes = [i, i, i, P, P, i, P, P]
        for f in ("vbqo_layout", "vbqo_pack", "vbqo_header", "vbqo_unpack", "vbqo_dequant_f32",
                  "vbqo_dequant_f16", "vbqo_gemv", "vbqo_gemv_blob", "vbqo_dense_gemv"):
            getattr(L, f).restype = i
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(rc, what)


HEADER_FIELDS = ("N", "K", "G", "S", "nS", "off_row_off", "off_slice_off", "off_wmap", "off_scales",
                 "off_codes", "total_bytes", "code_bytes", "code_bytes_padded", "row_pad")


def f16_to_f64(h: int) -> float:
    return lib().vbqo_f16_to_f64(int(h))


def f64_to_f16(v: float) -> int:
    return int(lib().vbqo_f64_to_f16_rne(float(v)))


def layout(N: int, K: int, bits: np.ndarray) -> dict:
    h = np.zeros(14, dtype=np.uint64)
    _check(lib().vbqo_layout(N, K, _p(_c(bits, np.uint8)), _p(h)), "layout")
    return {k: int(v) for k, v in zip(HEADER_FIELDS, h)}


def pack(q: np.ndarray, bits: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """q u8[N][K], bits u8[N][G], scales fp16 bits u16[N][G] -> blob u8[total]."""
    q = _c(q, np.uint8)
    N, K = q.shape
    bits = _c(bits, np.uint8)
    scales = _c(scales, np.uint16)
    L = layout(N, K, bits)
    blob = np.empty(L["total_bytes"], dtype=np.uint8)
    _check(lib().vbqo_pack(N, K, _p(q), _p(bits), _p(scales), _p(blob), blob.size), "pack")
    return blob


def header(blob: np.ndarray) -> dict:
    blob = _c(blob, np.uint8)
    h = np.zeros(14, dtype=np.uint64)
    _check(lib().vbqo_header(_p(blob), blob.size, _p(h)), "header")
    return {k: int(v) for k, v in zip(HEADER_FIELDS, h)}


def unpack(blob: np.ndarray):
    blob = _c(blob, np.uint8)
    h = header(blob)
    N, K, G = h["N"], h["K"], h["G"]
    q = np.empty((N, K), np.uint8)
    bits = np.empty((N, G), np.uint8)
    sc = np.empty((N, G), np.uint16)
    _check(lib().vbqo_unpack(_p(blob), blob.size, _p(q), _p(bits), _p(sc)), "unpack")
    return q, bits, sc


def quantize(w, bits):
    """Round-to-nearest codes and fp16 scales for width map bits u8[N][G] from
    weights w (fp32 or fp16 values, [N][K]; fp16 is widened exactly) ->
    (q u8[N][K], scales fp16 bits u16[N][G])."""
    w = np.asarray(w)
    w32 = _c(w.astype(np.float32) if w.dtype == np.float16 else w, np.float32)
    bits = _c(bits, np.uint8)
    N, K = w32.shape
    q = np.empty((N, K), np.uint8)
    s = np.empty((N, K // 64), np.uint16)
    _check(lib().vbqo_quantize(N, K, _p(w32), K, _p(bits), _p(q), _p(s)), "quantize")
    return q, s


def swiglu(gate, up):
    """SwiGLU activation of a gated MLP in fp64: silu(g) * u with
    silu(g) = g * sigmoid(g) = g / (1 + exp(-g)) (the gate's output through
    the sigmoid-weighted linear unit, times the up projection's output)."""
    g = np.asarray(gate, np.float64)
    u = np.asarray(up, np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def dequant(q, bits, scales, dtype=np.float32) -> np.ndarray:
    q = _c(q, np.uint8)
    bits = _c(bits, np.uint8)
    scales = _c(scales, np.uint16)
    N, K = q.shape
    if dtype == np.float32:
        w = np.empty((N, K), np.float32)
        _check(lib().vbqo_dequant_f32(N, K, _p(q), _p(bits), _p(scales), _p(w)), "dequant_f32")
    else:
        w = np.empty((N, K), np.uint16)
        _check(lib().vbqo_dequant_f16(N, K, _p(q), _p(bits), _p(scales), _p(w)), "dequant_f16")
    return w


def gemv(q, bits, scales, x):
    """x fp16 bits u16[M][K] (or [K]) -> (y f64[M][N], bound f64[M][N])."""
    q = _c(q, np.uint8)
    bits = _c(bits, np.uint8)
    scales = _c(scales, np.uint16)
    x = _c(np.atleast_2d(x), np.uint16)
    N, K = q.shape
    M = x.shape[0]
    y = np.empty((M, N), np.float64)
    b = np.empty((M, N), np.float64)
    _check(lib().vbqo_gemv(N, K, M, _p(q), _p(bits), _p(scales), _p(x), x.shape[1], _p(y), _p(b)), "gemv")
    return y, b


def gemv_blob(blob, x):
    blob = _c(blob, np.uint8)
    x = _c(np.atleast_2d(x), np.uint16)
    h = header(blob)
    M = x.shape[0]
    y = np.empty((M, h["N"]), np.float64)
    b = np.empty((M, h["N"]), np.float64)
    _check(lib().vbqo_gemv_blob(_p(blob), blob.size, M, _p(x), x.shape[1], _p(y), _p(b)), "gemv_blob")
    return y, b


def dense_gemv(w16, x):
    w16 = _c(w16, np.uint16)
    x = _c(np.atleast_2d(x), np.uint16)
    N, K = w16.shape
    M = x.shape[0]
    y = np.empty((M, N), np.float64)
    b = np.empty((M, N), np.float64)
    _check(lib().vbqo_dense_gemv(N, K, M, _p(w16), _p(x), x.shape[1], _p(y), _p(b)), "dense_gemv")
    return y, b
