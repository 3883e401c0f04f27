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
    # the workspace holds the fp32 partial sums of a K split: none for M <= 2,
    # else a whole number (at most 16) of [M][N] planes
    for M in (1, 2):
        assert lib.vbq_workspace_size(ref, M, ctypes.byref(sz)) == 0 and sz.value == 0
    for M in (3, 17, 32, 16):
        assert lib.vbq_workspace_size(ref, M, ctypes.byref(sz)) == 0
        assert sz.value % (4 * M * 4) == 0 and sz.value <= 16 * 4 * M * 4
    need = sz.value
    assert v.STATUS[lib.vbq_workspace_size(ref, 33, ctypes.byref(sz))] == "VBQ_ERR_BATCH"

    def call(M=1, blob=fake, x=fake, ldx=4096, y=fake, ldy=4, yt=1, ws=fake, wsb=None):
        return v.STATUS[lib.vbq_gemv_batched(ref, blob, M, x, ldx, y, ldy, yt, ws, need if wsb is None else wsb, null)]

    assert call(M=0) == "VBQ_ERR_BATCH"
    assert call(M=33) == "VBQ_ERR_BATCH"
    # more than 16 tokens only on the matrix cores: x 16-byte aligned, ldx % 8 == 0
    assert call(M=17, x=odd) == "VBQ_ERR_ALIGN"
    assert call(M=32, ldx=4100) == "VBQ_ERR_ALIGN"
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


def fake_plan(v, N=4, K=4096, M=1, passes=1):
    """A plan struct that passes the host checks (one row block of N rows)."""
    P = v.Plan()
    P.magic = 0x33504256
    P.N, P.K, P.G, P.M = N, K, K // 64, M
    P.wgs, P.rows = 1, N
    P.passes = passes
    P.per_wave = (-(-passes // 16) + 1 + 3) // 4 * 4
    P.psum = (max(N, 2) * (K // 64) + 1 + 3) // 4 * 4
    P.region_bytes = P.total_bytes = (passes * 1536 + 16 * P.per_wave + 255) // 256 * 256
    return P


def test_plan_argument_checks_fail_before_launch():
    v = vbq()
    lib = v.lib()
    VP = ctypes.c_void_p
    fake, null = VP(1 << 20), VP(0)
    blob = oracle.pack(np.zeros((4, 4096), np.uint8), np.ones((4, 64), np.uint8), np.ones((4, 64), np.uint16))
    L = v.layout_from_header(blob[:256].tobytes())
    out = v.Plan()

    def init(M=1, blob=fake, ws=fake, wsb=16, lay=L):
        return v.STATUS[lib.vbq_plan_init(ctypes.byref(lay), blob, M, 0, ctypes.byref(out), ws, wsb, null)]

    assert init(blob=null) == "VBQ_ERR_INVALID_ARG"
    assert init(M=0) == "VBQ_ERR_BATCH"
    assert init(M=3) == "VBQ_ERR_BATCH"
    assert init(ws=null) == "VBQ_ERR_WORKSPACE"
    assert init(wsb=8) == "VBQ_ERR_WORKSPACE"
    assert init(blob=VP((1 << 20) + 64)) == "VBQ_ERR_ALIGN"
    big = oracle.pack(np.zeros((1, 64 * 513), np.uint8), np.ones((1, 513), np.uint8), np.ones((1, 513), np.uint16))
    Lbig = v.layout_from_header(big[:256].tobytes())
    assert init(lay=Lbig) == "VBQ_ERR_SHAPE"  # K > 32768
    bad = v.Layout.from_buffer_copy(bytes(L))
    bad.version = 7
    assert init(lay=bad) == "VBQ_ERR_LAYOUT"

    P = fake_plan(v)

    def gemv(Pl=P, plan=fake, M=1, x=fake, ldx=4096, y=fake, ldy=4, yt=1):
        return v.STATUS[lib.vbq_gemv_planned(ctypes.byref(Pl), plan, M, x, ldx, y, ldy, yt, null)]

    assert gemv(M=0) == "VBQ_ERR_BATCH"
    assert gemv(M=17) == "VBQ_ERR_BATCH"
    assert gemv(plan=null) == "VBQ_ERR_INVALID_ARG"
    assert gemv(x=null) == "VBQ_ERR_INVALID_ARG"
    assert gemv(yt=5) == "VBQ_ERR_INVALID_ARG"
    assert gemv(ldx=4032) == "VBQ_ERR_SHAPE"
    assert gemv(ldy=3) == "VBQ_ERR_SHAPE"
    assert gemv(plan=VP((1 << 20) + 128)) == "VBQ_ERR_ALIGN"
    assert gemv(y=VP((1 << 20) + 2), yt=0) == "VBQ_ERR_ALIGN"  # f32 outputs need 4-byte alignment
    for field, val in [("magic", 0), ("K", 4032), ("M", 3), ("passes", 0), ("per_wave", 8), ("psum", 5),
                       ("region_bytes", 1024), ("total_bytes", 2048), ("rows", 1)]:
        bad = fake_plan(v)
        setattr(bad, field, val)
        assert gemv(Pl=bad) == "VBQ_ERR_LAYOUT", field
    # a plan whose partial sums do not fit one workgroup's LDS
    big = fake_plan(v, N=1000)
    assert gemv(Pl=big, ldy=1000) == "VBQ_ERR_SHAPE"

    def shared(plans, n=None, x=fake):
        items = (v.PlannedItem * max(1, len(plans)))()
        for k, p in enumerate(plans):
            items[k] = v.PlannedItem(ctypes.addressof(p), fake, fake, 4)
        return v.STATUS[lib.vbq_gemv_planned_shared(items, len(plans) if n is None else n, 1, x, 4096, 1, null)]

    assert shared([P], n=0) == "VBQ_ERR_INVALID_ARG"
    assert shared([P] * 5) == "VBQ_ERR_INVALID_ARG"
    assert shared([P, fake_plan(v, K=2048)]) == "VBQ_ERR_SHAPE"
    assert shared([P, fake_plan(v, N=1000)]) == "VBQ_ERR_SHAPE"  # the larger block's partial sums do not fit
    # vbq_prepare: the plan must describe this layout
    assert v.STATUS[lib.vbq_prepare(ctypes.byref(fake_plan(v, N=8)), ctypes.byref(L), fake, fake, null, null)] == \
        "VBQ_ERR_SHAPE"
    assert v.STATUS[lib.vbq_prepare(ctypes.byref(P), ctypes.byref(L), fake, VP((1 << 20) + 16), null, null)] == \
        "VBQ_ERR_ALIGN"
    assert v.STATUS[lib.vbq_prepare(ctypes.byref(P), ctypes.byref(L), fake, fake, VP((1 << 20) + 2), null)] == \
        "VBQ_ERR_ALIGN"


def test_seq_argument_checks_fail_before_launch():
    """Every item of a step is checked before the first launch: a bad item
    anywhere in the array returns its own error, never the HIP error that a
    launch of an earlier, valid item would give on a host with no GPU."""
    v = vbq()
    lib = v.lib()
    VP = ctypes.c_void_p
    fake, null = 1 << 20, VP(0)
    blob = oracle.pack(np.zeros((4, 4096), np.uint8), np.ones((4, 64), np.uint8), np.ones((4, 64), np.uint16))
    L = v.layout_from_header(blob[:256].tobytes())
    bad = v.Layout.from_buffer_copy(bytes(L))
    bad.magic = 0

    def seq(specs, M=1, yt=1, n=None):
        items = (v.SeqItem * max(1, len(specs)))()
        for k, s in enumerate(specs):
            d = dict(L=L, blob=fake, x=fake, ldx=4096, y=fake, ldy=4, stage=k)
            d.update(s)
            items[k] = v.SeqItem(ctypes.addressof(d["L"]), d["blob"], d["x"], d["ldx"], d["y"], d["ldy"], d["stage"])
        return v.STATUS[lib.vbq_gemv_seq(items, len(specs) if n is None else n, M, yt, null, 0, null)]

    ok = {}
    assert seq([ok], n=0) == "VBQ_ERR_INVALID_ARG"
    assert seq([ok], M=0) == "VBQ_ERR_BATCH"
    assert seq([ok], M=17) == "VBQ_ERR_BATCH"
    assert seq([ok], yt=4) == "VBQ_ERR_INVALID_ARG"
    assert seq([ok, ok, dict(blob=0)]) == "VBQ_ERR_INVALID_ARG"
    assert seq([ok, dict(L=bad)]) == "VBQ_ERR_LAYOUT"
    assert seq([ok, dict(ldx=64)]) == "VBQ_ERR_SHAPE"
    assert seq([ok, dict(ldy=1)]) == "VBQ_ERR_SHAPE"
    assert seq([ok, dict(x=fake + 1)]) == "VBQ_ERR_ALIGN"
    assert seq([ok, dict(blob=fake + 128)]) == "VBQ_ERR_ALIGN"
    assert seq([dict(stage=3), dict(stage=2)]) == "VBQ_ERR_INVALID_ARG"  # stages must not decrease
    assert seq([dict(stage=0)] * 1025) == "VBQ_ERR_INVALID_ARG"  # at most 1024 items per stage

    P = fake_plan(v)
    P2 = fake_plan(v, N=1000)  # its layout checks pass; its partial sums do not fit the LDS
    Pbad = fake_plan(v)
    Pbad.magic = 1

    def pseq(specs, M=1, yt=1):
        items = (v.PlannedSeqItem * len(specs))()
        for k, s in enumerate(specs):
            d = dict(P=P, plan=fake, x=fake, ldx=4096, y=fake, ldy=4, stage=k)
            d.update(s)
            items[k] = v.PlannedSeqItem(ctypes.addressof(d["P"]), d["plan"], d["x"], d["ldx"], d["y"], d["ldy"],
                                        d["stage"])
        return v.STATUS[lib.vbq_gemv_planned_seq(items, len(specs), M, yt, null)]

    assert pseq([ok], M=0) == "VBQ_ERR_BATCH"
    assert pseq([ok, dict(plan=0)]) == "VBQ_ERR_INVALID_ARG"
    assert pseq([ok, dict(P=Pbad)]) == "VBQ_ERR_LAYOUT"
    assert pseq([ok, dict(ldx=4000)]) == "VBQ_ERR_SHAPE"
    assert pseq([ok, dict(ldy=2)]) == "VBQ_ERR_SHAPE"
    assert pseq([ok, dict(plan=fake + 8)]) == "VBQ_ERR_ALIGN"
    assert pseq([ok, dict(P=P2, ldy=1000)]) == "VBQ_ERR_SHAPE"
    assert pseq([dict(stage=1), dict(stage=0)]) == "VBQ_ERR_INVALID_ARG"


def test_quantize_argument_checks_fail_before_launch():
    v = vbq()
    lib = v.lib()
    VP = ctypes.c_void_p
    fake, null = VP(1 << 20), VP(0)

    def call(N=4, K=128, w=fake, wt=0, ldw=128, bits=fake, q=fake, s=fake, st=null):
        return v.STATUS[lib.vbq_quantize(N, K, w, wt, ldw, bits, q, s, st, null)]

    assert call(w=null) == "VBQ_ERR_INVALID_ARG"
    assert call(bits=null) == "VBQ_ERR_INVALID_ARG"
    assert call(q=null) == "VBQ_ERR_INVALID_ARG"
    assert call(s=null) == "VBQ_ERR_INVALID_ARG"
    assert call(wt=2) == "VBQ_ERR_INVALID_ARG"
    assert call(N=0) == "VBQ_ERR_SHAPE"
    assert call(K=96, ldw=96) == "VBQ_ERR_SHAPE"
    assert call(K=32, ldw=32) == "VBQ_ERR_SHAPE"
    assert call(ldw=100) == "VBQ_ERR_SHAPE"
    assert call(w=VP((1 << 20) + 2)) == "VBQ_ERR_ALIGN"          # fp32 weights need 4-byte alignment
    assert call(s=VP((1 << 20) + 1)) == "VBQ_ERR_ALIGN"
    assert call(q=VP((1 << 20) + 4)) == "VBQ_ERR_ALIGN"
    assert call(st=VP((1 << 20) + 2)) == "VBQ_ERR_ALIGN"


def test_planned_argmax_argument_checks_fail_before_launch():
    v = vbq()
    lib = v.lib()
    VP = ctypes.c_void_p
    fake, null = VP(1 << 20), VP(0)
    P = fake_plan(v)

    def call(Pl=P, plan=fake, M=1, x=fake, ldx=4096, ws=fake):
        return v.STATUS[lib.vbq_gemv_planned_argmax(ctypes.byref(Pl), plan, M, x, ldx, ws, null)]

    assert call(plan=null) == "VBQ_ERR_INVALID_ARG"
    assert call(x=null) == "VBQ_ERR_INVALID_ARG"
    assert call(ws=null) == "VBQ_ERR_INVALID_ARG"
    assert call(M=0) == "VBQ_ERR_BATCH"
    assert call(M=17) == "VBQ_ERR_BATCH"
    assert call(ws=VP((1 << 20) + 4)) == "VBQ_ERR_ALIGN"
    assert call(ldx=100) == "VBQ_ERR_SHAPE"
    bad = fake_plan(v)
    bad.magic = 0
    assert call(Pl=bad) == "VBQ_ERR_LAYOUT"


def fake_gemm_plan(v, N=300, K=4096, max_tile=5000):
    G = K // 64
    nb, kc = (N + 127) // 128, (G + 1) // 2
    table = (4 * (nb * kc + 1) + 255) // 256 * 256
    slot = (max_tile + 4095) // 4096 * 4096
    return v.GemmPlan(magic=0x4D4D4756, N=N, K=K, G=G, nb=nb, kc=kc, max_tile=max_tile, slot_bytes=slot,
                      table_bytes=table, total_bytes=table + 100000 + slot)


def test_gemm_argument_checks_fail_before_launch():
    v = vbq()
    lib = v.lib()
    VP = ctypes.c_void_p
    fake, null = VP(1 << 20), VP(0)
    blob = oracle.pack(np.zeros((4, 4096), np.uint8), np.ones((4, 64), np.uint8), np.ones((4, 64), np.uint16))
    L = v.layout_from_header(blob[:256].tobytes())
    out = v.GemmPlan()

    def init(blob=fake, ws=fake, wsb=16, lay=L):
        return v.STATUS[lib.vbq_gemm_plan_init(ctypes.byref(lay), blob, ctypes.byref(out), ws, wsb, null)]

    assert init(blob=null) == "VBQ_ERR_INVALID_ARG"
    assert init(ws=null) == "VBQ_ERR_WORKSPACE"
    assert init(wsb=8) == "VBQ_ERR_WORKSPACE"
    assert init(blob=VP((1 << 20) + 64)) == "VBQ_ERR_ALIGN"
    big = oracle.pack(np.zeros((1, 64 * 513), np.uint8), np.ones((1, 513), np.uint8), np.ones((1, 513), np.uint16))
    assert init(lay=v.layout_from_header(big[:256].tobytes())) == "VBQ_ERR_SHAPE"  # K > 32768
    bad = v.Layout.from_buffer_copy(bytes(L))
    bad.version = 7
    assert init(lay=bad) == "VBQ_ERR_LAYOUT"

    GP = fake_gemm_plan(v)
    n = ctypes.c_size_t(0)
    assert v.STATUS[lib.vbq_gemm_workspace(ctypes.byref(GP), 0, ctypes.byref(n))] == "VBQ_ERR_BATCH"
    assert v.STATUS[lib.vbq_gemm_workspace(ctypes.byref(GP), 64, ctypes.byref(n))] == "VBQ_OK"
    # the copy of X in k-slot order at least (64 token rows of K halves)
    assert n.value >= 64 * 4096 * 2
    big_ws = n.value

    def gemm(Pl=GP, buf=fake, M=64, x=fake, ldx=4096, y=fake, ldy=300, yt=1, ws=fake, wsb=big_ws):
        return v.STATUS[lib.vbq_gemm(ctypes.byref(Pl), buf, M, x, ldx, y, ldy, yt, ws, wsb, null)]

    assert gemm(M=0) == "VBQ_ERR_BATCH"
    assert gemm(M=(1 << 20) + 1) == "VBQ_ERR_BATCH"
    assert gemm(buf=null) == "VBQ_ERR_INVALID_ARG"
    assert gemm(x=null) == "VBQ_ERR_INVALID_ARG"
    assert gemm(ws=null) == "VBQ_ERR_INVALID_ARG"
    assert gemm(yt=5) == "VBQ_ERR_INVALID_ARG"
    assert gemm(ldx=4032) == "VBQ_ERR_SHAPE"
    assert gemm(ldy=299) == "VBQ_ERR_SHAPE"
    assert gemm(buf=VP((1 << 20) + 128)) == "VBQ_ERR_ALIGN"
    assert gemm(x=VP((1 << 20) + 8)) == "VBQ_ERR_ALIGN"
    assert gemm(ldx=4100) == "VBQ_ERR_ALIGN"          # rows of x 16-byte aligned
    assert gemm(y=VP((1 << 20) + 2), yt=0) == "VBQ_ERR_ALIGN"
    assert gemm(ws=VP((1 << 20) + 128)) == "VBQ_ERR_ALIGN"
    assert gemm(wsb=big_ws - 1) == "VBQ_ERR_WORKSPACE"
    for field, val in [("magic", 0), ("K", 4032), ("nb", 2), ("kc", 33), ("slot_bytes", 6000),
                       ("slot_bytes", 6 * 4096), ("max_tile", 9000), ("table_bytes", 256), ("total_bytes", 1024)]:
        badp = fake_gemm_plan(v)
        setattr(badp, field, val)
        assert gemm(Pl=badp) == "VBQ_ERR_LAYOUT", field
    assert v.STATUS[lib.vbq_gemm_prepare(ctypes.byref(fake_gemm_plan(v, N=8)), ctypes.byref(L), fake, fake, null,
                                         null)] == "VBQ_ERR_SHAPE"
    assert v.STATUS[lib.vbq_gemm_prepare(ctypes.byref(fake_gemm_plan(v, N=4)), ctypes.byref(L), fake, fake,
                                         VP((1 << 20) + 2), null)] == "VBQ_ERR_ALIGN"  # status word alignment
