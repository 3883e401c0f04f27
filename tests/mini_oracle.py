"""A second, independent statement of the VBQ1 packing and of the GEMV, in numpy.

Written from the layout's description (include/vbq.h, the packed layout VBQ1) and the
dequant rule w = s * (q - (2^b - 1)/2), without reference to the C oracle's code; the
tests compare the two on random matrices.  Test infrastructure only.
"""
import numpy as np

MAGIC = 0x31514256


def _align(x, a):
    return (x + a - 1) // a * a


def group_bytes(codes, b):
    """64 codes of width b -> 8*b bytes: halves packed LSB-first in 16-bit units,
    word d = unit d of codes 0..31 | unit d of codes 32..63 << 16."""
    out = bytearray()
    per = 16 // b
    halves = (codes[:32], codes[32:])
    for d in range(2 * b):
        units = []
        for h in halves:
            u = 0
            for i in range(per):
                u |= int(h[d * per + i]) << (b * i)
            units.append(u)
        out += (units[0] | units[1] << 16).to_bytes(4, "little")
    return bytes(out)


def pack(q, bits, scales):
    """q u8[N][K], bits u8[N][G], scales fp16 bits u16[N][G] -> VBQ1 blob (numpy u8)."""
    N, K = q.shape
    G = K // 64
    nS = -(-G // 32)
    code_cw = {1: 0, 2: 1, 4: 2, 8: 3}
    rows = []
    slice_off = np.zeros((N, nS), np.uint32)
    wmap = np.zeros((N, nS, 2), np.uint32)
    for n in range(N):
        rec = bytearray()
        for t in range(nS):
            slice_off[n, t] = len(rec)
            gs = range(32 * t, min(G, 32 * t + 32))
            for g in gs:
                c = code_cw[int(bits[n, g])]
                wmap[n, t, 0] |= (c & 1) << (g - 32 * t)
                wmap[n, t, 1] |= (c >> 1) << (g - 32 * t)
            for b in (1, 2, 4, 8):
                for g in gs:
                    if int(bits[n, g]) == b:
                        rec += group_bytes(q[n, 64 * g:64 * g + 64], b)
        rows.append(bytes(rec))
    code_bytes = sum(len(r) for r in rows)
    padded = [_align(len(r), 128) for r in rows]
    row_off = np.zeros(N + 1, np.uint32)
    row_off[1:] = np.cumsum(padded) // 128
    off_row_off = 256
    off_slice_off = _align(off_row_off + 4 * (N + 1), 256)
    off_wmap = _align(off_slice_off + 4 * N * nS, 256)
    off_scales = _align(off_wmap + 8 * N * nS, 256)
    off_codes = _align(off_scales + 2 * N * G, 256)
    total = off_codes + sum(padded)
    blob = bytearray(total)
    hdr = np.array([MAGIC, 1, N, K, G, 32, nS, 128], np.uint32).tobytes()
    hdr += np.array([off_row_off, off_slice_off, off_wmap, off_scales, off_codes, total, code_bytes,
                     sum(padded)], np.uint64).tobytes()
    blob[:len(hdr)] = hdr
    blob[off_row_off:off_row_off + 4 * (N + 1)] = row_off.tobytes()
    blob[off_slice_off:off_slice_off + 4 * N * nS] = slice_off.tobytes()
    blob[off_wmap:off_wmap + 8 * N * nS] = wmap.tobytes()
    blob[off_scales:off_scales + 2 * N * G] = np.ascontiguousarray(scales, np.uint16).tobytes()
    pos = off_codes
    for r, p in zip(rows, padded):
        blob[pos:pos + len(r)] = r
        pos += p
    return np.frombuffer(bytes(blob), np.uint8)


def dequant(q, bits, scales):
    """Dense float64 weights: w = s * (q - (2^b - 1)/2) per group."""
    N, K = q.shape
    s = np.asarray(scales, np.uint16).view(np.float16).astype(np.float64)
    c = ((1 << bits.astype(np.int64)) - 1) / 2.0
    qq = q.reshape(N, K // 64, 64).astype(np.float64)
    with np.errstate(invalid="ignore"):
        return (s[..., None] * (qq - c[..., None])).reshape(N, K)


def gemv(q, bits, scales, x):
    """y[M][N] = X W^T in float64, x as fp16 bit patterns [M][K]."""
    xf = np.atleast_2d(np.asarray(x, np.uint16)).view(np.float16).astype(np.float64)
    return xf @ dequant(q, bits, scales).T
