"""The C ABI without a GPU: the library loads, exports every symbol that
include/vbq.h declares, and its host-side argument checks reject bad calls
before any launch (these calls return before touching the HIP runtime)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def vbq():
    import decode_gemv_vbq_amd as v
    try:
        v.lib()
    except RuntimeError as e:
        pytest.skip(str(e))
    return v


def declared_functions():
    text = open(os.path.join(ROOT, "include", "vbq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vbq_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    v = vbq()
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(v.lib(), n), n
    assert set(names) == set(v.EXPORTS)


def test_version_and_status_strings():
    v = vbq()
    assert "VBQ1" in v.version()
    for code in range(10):
        assert v.lib().vbq_status_string(code)


def test_layout_init_matches_oracle_geometry():
    v = vbq()
    for N, K in [(1, 64), (768, 768), (5632, 2048), (128256, 4096), (8192, 28672)]:
        L = v.layout_init(N, K)
        h = oracle.layout(N, K, np.ones((N, K // 64), np.uint8))
        for f in ("N", "K", "G", "S", "nS", "off_row_off", "off_slice_off", "off_wmap", "off_scales", "off_codes"):
            assert getattr(L, f) == h[f], (N, K, f)
    for N, K in [(0, 64), (1, 0), (1, 96), (-3, 128)]:
        with pytest.raises(v.VbqError) as e:
            v.layout_init(N, K)
        assert e.value.name == "VBQ_ERR_SHAPE"


def test_layout_from_header_accepts_oracle_blob_and_rejects_corruption():
    v = vbq()
    r = np.random.default_rng(0)
    bits = r.choice(np.array([1, 2, 4, 8], np.uint8), (5, 40))
    q = (r.integers(0, 256, (5, 2560)) & np.repeat(np.left_shift(1, bits.astype(np.int32)) - 1, 64, 1)).astype(np.uint8)
    blob = oracle.pack(q, bits, np.ones((5, 40), np.uint16))
    L = v.layout_from_header(blob[:256].tobytes())
    h = oracle.header(blob)
    for f in ("total_bytes", "code_bytes", "code_bytes_padded", "off_codes"):
        assert getattr(L, f) == h[f]
    for off, val in [(0, 0x00), (4, 2), (20, 16), (72, 0), (100, 1)]:
        bad = bytearray(blob[:256].tobytes())
        bad[off] = val
        with pytest.raises(v.VbqError) as e:
            v.layout_from_header(bytes(bad))
        assert e.value.name == "VBQ_ERR_LAYOUT", off


def test_gemv_argument_checks_fail_before_launch():
    v = vbq()
    lib = v.lib()
    r = np.random.default_rng(1)
    bits = np.ones((4, 64), np.uint8)
    blob = oracle.pack(np.zeros((4, 4096), np.uint8), bits, np.ones((4, 64), np.uint16))
    L = v.layout_from_header(blob[:256].tobytes())
    P = ctypes.c_void_p
    fake = P(1 << 20)          # 256-aligned, never dereferenced: checks fail first
    odd = P((1 << 20) + 2)
    null = P(0)
    ref = ctypes.byref(L)
    sz = ctypes.c_size_t(0)
    assert lib.vbq_workspace_size(ref, 16, ctypes.byref(sz)) == 0
    need = sz.value  # rows are never split across workgroups: no workspace
    assert need == 0

    def call(M=1, blob=fake, x=fake, ldx=4096, y=fake, ldy=4, yt=1, ws=fake, wsb=None):
        return v.STATUS[lib.vbq_gemv_batched(ref, blob, M, x, ldx, y, ldy, yt, ws, need if wsb is None else wsb, null)]

    assert call(M=0) == "VBQ_ERR_BATCH"
    assert call(M=17) == "VBQ_ERR_BATCH"
    assert call(blob=null) == "VBQ_ERR_INVALID_ARG"
    assert call(x=null) == "VBQ_ERR_INVALID_ARG"
    assert call(yt=7) == "VBQ_ERR_INVALID_ARG"
    assert call(ldx=4095) == "VBQ_ERR_SHAPE"
    assert call(ldy=3) == "VBQ_ERR_SHAPE"
    assert call(blob=odd) == "VBQ_ERR_ALIGN"
    bad = v.Layout.from_buffer_copy(bytes(L))
    bad.magic = 0
    assert v.STATUS[lib.vbq_gemv(ctypes.byref(bad), fake, fake, fake, 1, fake, need, null)] == "VBQ_ERR_LAYOUT"
    bad = v.Layout.from_buffer_copy(bytes(L))
    bad.total_bytes += 128
    assert v.STATUS[lib.vbq_dequant(ctypes.byref(bad), fake, fake, 0, null)] == "VBQ_ERR_LAYOUT"
    assert v.STATUS[lib.vbq_dense_f16_gemv(4, 60, 1, fake, fake, 60, fake, 4, 1, null)] == "VBQ_ERR_SHAPE"
    assert v.STATUS[lib.vbq_dense_f16_gemv(4, 64, 0, fake, fake, 64, fake, 4, 1, null)] == "VBQ_ERR_BATCH"
    assert v.STATUS[lib.vbq_pack_plan(4, 100, fake, ctypes.byref(v.Layout()), fake, 1 << 20, null)] == "VBQ_ERR_SHAPE"
    assert v.STATUS[lib.vbq_pack_plan(4, 128, fake, ctypes.byref(v.Layout()), fake, 8, null)] == "VBQ_ERR_WORKSPACE"
    assert v.STATUS[lib.vbq_pack(ref, null, fake, fake, fake, fake, null)] == "VBQ_ERR_INVALID_ARG"
    assert v.STATUS[lib.vbq_workspace_size(ref, 0, ctypes.byref(sz))] == "VBQ_ERR_BATCH"


def test_gemv_shared_argument_checks_fail_before_launch():
    v = vbq()
    lib = v.lib()
    P = ctypes.c_void_p
    fake = 1 << 20
    bits = np.ones((4, 64), np.uint8)
    blob = oracle.pack(np.zeros((4, 4096), np.uint8), bits, np.ones((4, 64), np.uint16))
    L = v.layout_from_header(blob[:256].tobytes())
    blob2 = oracle.pack(np.zeros((4, 2048), np.uint8), np.ones((4, 32), np.uint8), np.ones((4, 32), np.uint16))
    L2 = v.layout_from_header(blob2[:256].tobytes())  # a different K
    null = P(0)

    def call(layouts, n=None, M=1, x=fake, ldx=4096, yt=1, blob=fake, ldy=4):
        items = (v.GemvItem * max(1, len(layouts)))()
        for k, lay in enumerate(layouts):
            items[k] = v.GemvItem(ctypes.addressof(lay), blob, fake, ldy)
        return v.STATUS[lib.vbq_gemv_shared(items, len(layouts) if n is None else n, M, P(x), ldx, yt, null)]

    assert call([L], n=0) == "VBQ_ERR_INVALID_ARG"
    assert call([L] * 5) == "VBQ_ERR_INVALID_ARG"
    assert call([L], M=0) == "VBQ_ERR_BATCH"
    assert call([L], M=17) == "VBQ_ERR_BATCH"
    assert call([L], x=0) == "VBQ_ERR_INVALID_ARG"
    assert call([L], yt=9) == "VBQ_ERR_INVALID_ARG"
    assert call([L, L2]) == "VBQ_ERR_SHAPE"
    assert call([L], ldx=4095) == "VBQ_ERR_SHAPE"
    assert call([L], ldy=3) == "VBQ_ERR_SHAPE"
    assert call([L], blob=fake + 64) == "VBQ_ERR_ALIGN"
    bad = v.Layout.from_buffer_copy(bytes(L))
    bad.magic = 0
    assert call([L, bad]) == "VBQ_ERR_LAYOUT"
