"""decode_gemv_vbq_amd -- MI355X (gfx950) decode path of Variable Bit-width
Quantization: packed mixed-width (1/2/4/8-bit per 64-weight group) weights and
a fused dequantize-and-multiply GEMV for M <= 16 tokens.

This module is a thin ctypes binding over ``libvbq.so`` (``include/vbq.h``).
It only marshals arguments: device memory and streams come from PyTorch, every
step of the path runs in the HIP kernels of the library.  There is no CPU
fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvbq.so")

VBQ_F32, VBQ_F16 = 0, 1
#: device status-word bits (include/vbq.h VBQ_STATUS_*)
STATUS_BITS, STATUS_CODES, STATUS_LAYOUT, STATUS_PLAN = 0x1, 0x2, 0x4, 0x8

STATUS = {
    0: "VBQ_OK", 1: "VBQ_ERR_INVALID_ARG", 2: "VBQ_ERR_SHAPE", 3: "VBQ_ERR_BATCH", 4: "VBQ_ERR_BITS",
    5: "VBQ_ERR_CODE_RANGE", 6: "VBQ_ERR_ALIGN", 7: "VBQ_ERR_WORKSPACE", 8: "VBQ_ERR_LAYOUT", 9: "VBQ_ERR_HIP",
}

#: every symbol include/vbq.h declares
EXPORTS = (
    "vbq_version", "vbq_status_string", "vbq_last_error", "vbq_layout_init", "vbq_layout_from_header",
    "vbq_pack_plan_workspace", "vbq_pack_plan", "vbq_pack", "vbq_status_check", "vbq_dequant",
    "vbq_workspace_size", "vbq_workspace_clear", "vbq_gemv", "vbq_gemv_batched", "vbq_gemv_shared",
    "vbq_plan_init", "vbq_prepare", "vbq_gemv_planned", "vbq_gemv_planned_shared", "vbq_gemv_seq",
    "vbq_gemv_planned_seq", "vbq_dense_f16_gemv", "vbq_quantize", "vbq_gemv_planned_argmax",
    "vbq_gemv_planned_swiglu", "vbq_gemm_plan_init", "vbq_gemm_prepare", "vbq_gemm_workspace", "vbq_gemm",
    "vbq_gemv_planned_argmax_noalloc",
)
MAX_SHARED = 4


class VbqError(RuntimeError):
    def __init__(self, code: int, what: str, detail: str = ""):
        name = STATUS.get(code, str(code))
        super().__init__(f"{what}: {name}" + (f" ({detail})" if detail else ""))
        self.code = code
        self.name = name


class GemvItem(ctypes.Structure):
    """Mirror of ``vbq_gemv_item``."""
    _fields_ = [("L", ctypes.c_void_p), ("blob", ctypes.c_void_p), ("y", ctypes.c_void_p), ("ldy", ctypes.c_int)]


class Plan(ctypes.Structure):
    """Mirror of ``vbq_plan`` (host geometry of a prepared plan)."""
    _fields_ = [("magic", ctypes.c_uint32)] + \
               [(n, ctypes.c_int32) for n in ("N", "K", "G", "M", "wgs", "rows", "passes", "per_wave", "psum",
                                               "lds_bytes", "reserved")] + \
               [("region_bytes", ctypes.c_uint64), ("total_bytes", ctypes.c_uint64)]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


class PlannedItem(ctypes.Structure):
    """Mirror of ``vbq_planned_item``."""
    _fields_ = [("P", ctypes.c_void_p), ("plan", ctypes.c_void_p), ("y", ctypes.c_void_p), ("ldy", ctypes.c_int)]


class SeqItem(ctypes.Structure):
    """Mirror of ``vbq_seq_item``."""
    _fields_ = [("L", ctypes.c_void_p), ("blob", ctypes.c_void_p), ("x", ctypes.c_void_p), ("ldx", ctypes.c_int),
                ("y", ctypes.c_void_p), ("ldy", ctypes.c_int), ("stage", ctypes.c_int)]


class PlannedSeqItem(ctypes.Structure):
    """Mirror of ``vbq_planned_seq_item``."""
    _fields_ = [("P", ctypes.c_void_p), ("plan", ctypes.c_void_p), ("x", ctypes.c_void_p), ("ldx", ctypes.c_int),
                ("y", ctypes.c_void_p), ("ldy", ctypes.c_int), ("stage", ctypes.c_int)]


class GemmPlan(ctypes.Structure):
    """Mirror of ``vbq_gemm_plan`` (host geometry of a GEMM plan)."""
    _fields_ = [("magic", ctypes.c_uint32)] + \
               [(n, ctypes.c_int32) for n in ("N", "K", "G", "nb", "kc", "max_tile", "slot_bytes")] + \
               [("table_bytes", ctypes.c_uint64), ("total_bytes", ctypes.c_uint64)]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


class Layout(ctypes.Structure):
    """Mirror of ``vbq_layout`` (bytes 0..95 of the blob header)."""
    _fields_ = [(n, ctypes.c_uint32) for n in ("magic", "version", "N", "K", "G", "S", "nS", "row_pad")] + \
               [(n, ctypes.c_uint64) for n in ("off_row_off", "off_slice_off", "off_wmap", "off_scales", "off_codes",
                                               "total_bytes", "code_bytes", "code_bytes_padded")]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None


def lib():
    """Load libvbq.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m decode_gemv_vbq_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        LP = ctypes.POINTER(Layout)
        L.vbq_version.restype = ctypes.c_char_p
        L.vbq_status_string.restype = ctypes.c_char_p
        L.vbq_status_string.argtypes = [i]
        L.vbq_last_error.restype = ctypes.c_char_p
        L.vbq_layout_init.argtypes = [i, i, LP]
        L.vbq_layout_from_header.argtypes = [P, LP]
        L.vbq_pack_plan_workspace.argtypes = [i]
        L.vbq_pack_plan_workspace.restype = sz
        L.vbq_pack_plan.argtypes = [i, i, P, LP, P, sz, P]
        L.vbq_pack.argtypes = [LP, P, P, P, P, P, P]
        L.vbq_status_check.argtypes = [P, ctypes.POINTER(ctypes.c_uint32), P]
        L.vbq_dequant.argtypes = [LP, P, P, i, P]
        L.vbq_quantize.argtypes = [i, i, P, i, i, P, P, P, P, P]
        L.vbq_workspace_size.argtypes = [LP, i, ctypes.POINTER(sz)]
        L.vbq_workspace_clear.argtypes = [P, sz, P]
        L.vbq_gemv.argtypes = [LP, P, P, P, i, P, sz, P]
        L.vbq_gemv_batched.argtypes = [LP, P, i, P, i, P, i, i, P, sz, P]
        L.vbq_gemv_shared.argtypes = [ctypes.POINTER(GemvItem), i, i, P, i, i, P]
        PP = ctypes.POINTER(Plan)
        L.vbq_plan_init.argtypes = [LP, P, i, i, PP, P, sz, P]
        L.vbq_prepare.argtypes = [PP, LP, P, P, P, P]
        L.vbq_gemv_planned.argtypes = [PP, P, i, P, i, P, i, i, P]
        L.vbq_gemv_planned_shared.argtypes = [ctypes.POINTER(PlannedItem), i, i, P, i, i, P]
        L.vbq_gemv_planned_argmax.argtypes = [PP, P, i, P, i, P, P]
        L.vbq_gemv_planned_argmax_noalloc.argtypes = [PP, P, i, P, i, P, P, P]
        L.vbq_gemv_planned_swiglu.argtypes = [PP, P, i, P, i, P, i, i, P]
        L.vbq_gemv_seq.argtypes = [ctypes.POINTER(SeqItem), i, i, i, P, sz, P]
        L.vbq_gemv_planned_seq.argtypes = [ctypes.POINTER(PlannedSeqItem), i, i, i, P]
        L.vbq_dense_f16_gemv.argtypes = [i, i, i, P, P, i, P, i, i, P]
        GP = ctypes.POINTER(GemmPlan)
        L.vbq_gemm_plan_init.argtypes = [LP, P, GP, P, sz, P]
        L.vbq_gemm_prepare.argtypes = [GP, LP, P, P, P, P]
        L.vbq_gemm_workspace.argtypes = [GP, i, ctypes.POINTER(sz)]
        L.vbq_gemm.argtypes = [GP, P, i, P, i, P, i, i, P, sz, P]
        for f in EXPORTS:
            if f not in ("vbq_version", "vbq_status_string", "vbq_last_error", "vbq_pack_plan_workspace"):
                getattr(L, f).restype = i
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        detail = lib().vbq_last_error().decode() if rc == 9 else ""
        raise VbqError(rc, what, detail)


def version() -> str:
    return lib().vbq_version().decode()


# ------------------------------------------------------------ torch plumbing

def _torch():
    import torch
    return torch


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("expected contiguous device tensors")


def _x2(x, K: int, what: str = "x"):
    """x as a [M][K] view: a float16 tensor [K] (one token) or [M][K], unit
    column stride.  The device is checked by _on_device after every dtype and
    shape check, so that each rejection can be exercised without one."""
    torch = _torch()
    if x.dtype != torch.float16:
        raise ValueError(f"{what} must be float16, got {x.dtype}")
    if x.dim() not in (1, 2) or x.shape[-1] != K:
        raise ValueError(f"{what} must be [K] or [M][K] with K = {K}, got {tuple(x.shape)}")
    x2 = x.view(1, -1) if x.dim() == 1 else x
    if x2.stride(1) != 1:
        raise ValueError(f"{what} needs unit column stride")
    return x2


def _y2(out, M: int, N: int, one: bool, what: str = "out"):
    """out as a [M][N] view: float16 or float32, shape (M, N), or (N,) /
    (1, N) for a one-token [K] input, unit column stride."""
    torch = _torch()
    if out.dtype not in (torch.float16, torch.float32):
        raise ValueError(f"{what} must be float16 or float32, got {out.dtype}")
    shape = tuple(out.shape)
    if not (shape == (M, N) or (one and shape == (N,))):
        want = f"({N},)" if one else f"({M}, {N})"
        raise ValueError(f"{what} must have shape {want}, got {shape}")
    y2 = out.view(1, -1) if out.dim() == 1 else out
    if y2.stride(1) != 1:
        raise ValueError(f"{what} needs unit column stride")
    return y2


def _on_device(**ts):
    for name, t in ts.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")


def _yt(out):
    return VBQ_F32 if out.dtype == _torch().float32 else VBQ_F16


def _empty_aligned(nbytes: int, device, align: int = 256):
    """A uint8 device buffer whose data pointer is `align`-byte aligned."""
    torch = _torch()
    buf = torch.empty(nbytes + align, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % align
    return buf[off:off + nbytes]


# ------------------------------------------------------------------- layout

def layout_init(N: int, K: int) -> Layout:
    L = Layout()
    _check(lib().vbq_layout_init(N, K, ctypes.byref(L)), "vbq_layout_init")
    return L


def layout_from_header(header: bytes) -> Layout:
    if len(header) < 256:
        raise ValueError("header needs 256 bytes")
    buf = ctypes.create_string_buffer(bytes(header[:256]), 256)
    L = Layout()
    _check(lib().vbq_layout_from_header(ctypes.cast(buf, ctypes.c_void_p), ctypes.byref(L)), "vbq_layout_from_header")
    return L


def layout_of(blob) -> Layout:
    """Layout read back from a device blob's header."""
    return layout_from_header(blob[:256].cpu().numpy().tobytes())


# --------------------------------------------------------------------- pack

def pack_plan(bits, K: int) -> Layout:
    """Plan a blob for widths bits[N][G] (uint8, device). Synchronizes."""
    torch = _torch()
    _need_cuda(bits)
    N = bits.shape[0]
    ws = torch.empty(lib().vbq_pack_plan_workspace(N), dtype=torch.uint8, device=bits.device)
    L = Layout()
    _check(lib().vbq_pack_plan(N, K, _ptr(bits), ctypes.byref(L), _ptr(ws), ws.numel(), _stream()), "vbq_pack_plan")
    return L


def pack(q, bits, scales, L: Layout | None = None, check: bool = True):
    """Pack q[N][K] u8, bits[N][G] u8, scales[N][G] fp16 -> (blob u8 device tensor, Layout)."""
    torch = _torch()
    _need_cuda(q, bits, scales)
    if L is None:
        L = pack_plan(bits, q.shape[1])
    blob = _empty_aligned(L.total_bytes, q.device)
    status = torch.empty(1, dtype=torch.int32, device=q.device)
    _check(lib().vbq_pack(ctypes.byref(L), _ptr(q), _ptr(bits), _ptr(scales), _ptr(blob), _ptr(status), _stream()),
           "vbq_pack")
    if check:
        status_check(status)
    return blob, L


def status_check(status):
    raw = ctypes.c_uint32(0)
    _check(lib().vbq_status_check(_ptr(status), ctypes.byref(raw), _stream()), "vbq_pack (device status)")
    return raw.value


# ------------------------------------------------------------------ dequant

def quantize(w, bits, status=None):
    """Round-to-nearest codes and fp16 scales (vbq_quantize) for weights w
    ([N][K] fp32 or fp16 device tensor, unit column stride) and widths bits
    (u8 [N][G]) -> (q u8 [N][K], scales int16 view of fp16 bits [N][G]).
    With ``status`` (a 1-element int32 device tensor) a bad width is flagged
    there instead of being silent."""
    torch = _torch()
    _need_cuda(bits)
    if w.dim() != 2 or w.stride(1) != 1 or not w.is_cuda or w.dtype not in (torch.float32, torch.float16):
        raise ValueError("w must be a [N][K] fp32 or fp16 device tensor with unit column stride")
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    s = torch.empty((N, K // 64), dtype=torch.int16, device=w.device)
    wt = VBQ_F32 if w.dtype == torch.float32 else VBQ_F16
    _check(lib().vbq_quantize(N, K, _ptr(w), wt, w.stride(0), _ptr(bits), _ptr(q), _ptr(s), _ptr(status),
                              _stream()), "vbq_quantize")
    return q, s


def dequant(L: Layout, blob, dtype=None):
    torch = _torch()
    dtype = dtype or torch.float32
    w = torch.empty((L.N, L.K), dtype=dtype, device=blob.device)
    wt = VBQ_F32 if dtype == torch.float32 else VBQ_F16
    _check(lib().vbq_dequant(ctypes.byref(L), _ptr(blob), _ptr(w), wt, _stream()), "vbq_dequant")
    return w


# --------------------------------------------------------------------- GEMV

def workspace_size(L: Layout, M: int = 1) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().vbq_workspace_size(ctypes.byref(L), M, ctypes.byref(n)), "vbq_workspace_size")
    return n.value


def workspace(L: Layout, M: int = 16, device="cuda"):
    """A zeroed GEMV workspace for up to M tokens (None when not needed)."""
    n = workspace_size(L, M)
    if n == 0:
        return None
    ws = _empty_aligned(n, device)
    _check(lib().vbq_workspace_clear(_ptr(ws), n, _stream()), "vbq_workspace_clear")
    return ws


def gemv(L: Layout, blob, x, out=None, out_dtype=None, ws=None):
    """y[N] = W x for x fp16[K]."""
    torch = _torch()
    x2 = _x2(x, L.K)
    if x2.shape[0] != 1 or not x.is_contiguous():
        raise ValueError("x must be one contiguous token, [K] or [1][K]")
    out_dtype = out_dtype or torch.float16
    if out is None:
        out = torch.empty(L.N, dtype=out_dtype, device=x.device)
    _y2(out, 1, L.N, True)
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    _on_device(x=x, out=out)
    _need_cuda(blob)
    yt = _yt(out)
    if ws is None:
        ws = workspace(L, 1, x.device)
    _check(lib().vbq_gemv(ctypes.byref(L), _ptr(blob), _ptr(x), _ptr(out), yt, _ptr(ws),
                          0 if ws is None else ws.numel(), _stream()), "vbq_gemv")
    return out


def gemv_batched(L: Layout, blob, x, out=None, out_dtype=None, ws=None):
    """Y[M][N] = X[M][K] W^T for 1 <= M <= 32 (x fp16, rows may be strided; M > 16
    needs x 16-byte aligned and a row stride that is a multiple of 8)."""
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("x must be [M][K]")
    x = _x2(x, L.K)
    M = x.shape[0]
    out_dtype = out_dtype or torch.float16
    if out is None:
        out = torch.empty((M, L.N), dtype=out_dtype, device=x.device)
    _y2(out, M, L.N, False)
    _on_device(x=x, out=out)
    _need_cuda(blob)
    yt = _yt(out)
    if ws is None:
        ws = workspace(L, M, x.device)
    _check(lib().vbq_gemv_batched(ctypes.byref(L), _ptr(blob), M, _ptr(x), x.stride(0), _ptr(out), out.stride(0), yt,
                                  _ptr(ws), 0 if ws is None else ws.numel(), _stream()), "vbq_gemv_batched")
    return out


def gemv_shared(mats, x, outs=None, out_dtype=None):
    """[W_i x for (L_i, blob_i) in mats] in one launch where possible: the
    matrices share K and the activations x ([M][K], or [K] for one token)."""
    torch = _torch()
    if not mats:
        raise ValueError("no matrices")
    one = x.dim() == 1
    x2 = _x2(x, mats[0][0].K)
    M = x2.shape[0]
    out_dtype = out_dtype or torch.float16
    if outs is None:
        outs = [torch.empty((M, L.N), dtype=out_dtype, device=x.device) for L, _ in mats]
    if len(outs) != len(mats):
        raise ValueError("one output per matrix")
    ys = []
    for k, ((L, blob), out) in enumerate(zip(mats, outs)):
        if L.K != mats[0][0].K:
            raise ValueError("the matrices of a shared launch have one K")
        ys.append(_y2(out, M, L.N, one, f"outs[{k}]"))
        if out.dtype != outs[0].dtype:
            raise ValueError("outputs have one dtype")
    items = (GemvItem * len(mats))()
    for k, ((L, blob), y2) in enumerate(zip(mats, ys)):
        _on_device(x=x2, out=y2)
        _need_cuda(blob)
        items[k] = GemvItem(ctypes.addressof(L), _ptr(blob), _ptr(y2), y2.stride(0))
    yt = _yt(outs[0])
    _check(lib().vbq_gemv_shared(items, len(mats), M, _ptr(x2), x2.stride(0), yt, _stream()), "vbq_gemv_shared")
    return outs


# -------------------------------------------------------------- plans

def plan_init(L: Layout, blob, M: int = 1, wgs: int = 0) -> Plan:
    """Geometry of the prepared plan of (L, blob) for up to M tokens. Synchronizes."""
    torch = _torch()
    _need_cuda(blob)
    ws = torch.empty(16, dtype=torch.uint8, device=blob.device)
    P = Plan()
    _check(lib().vbq_plan_init(ctypes.byref(L), _ptr(blob), M, wgs, ctypes.byref(P), _ptr(ws), 16, _stream()),
           "vbq_plan_init")
    return P


def prepare(L: Layout, blob, M: int = 1, wgs: int = 0, check: bool = True):
    """Prepared plan of a packed matrix -> (plan u8 device tensor, Plan).
    With ``check`` the device status word is read back (synchronizes)."""
    torch = _torch()
    P = plan_init(L, blob, M, wgs)
    plan = _empty_aligned(P.total_bytes, blob.device)
    status = torch.empty(1, dtype=torch.int32, device=blob.device)
    _check(lib().vbq_prepare(ctypes.byref(P), ctypes.byref(L), _ptr(blob), _ptr(plan), _ptr(status), _stream()),
           "vbq_prepare")
    if check:
        status_check(status)
    return plan, P


def gemv_planned(P: Plan, plan, x, out=None, out_dtype=None):
    """Y[M][N] = X[M][K] W^T from a prepared plan (y[N] for 1-D x)."""
    torch = _torch()
    x2 = _x2(x, P.K)
    M = x2.shape[0]
    out_dtype = out_dtype or torch.float16
    if out is None:
        out = torch.empty((M, P.N) if x.dim() == 2 else (P.N,), dtype=out_dtype, device=x.device)
    y2 = _y2(out, M, P.N, x.dim() == 1)
    _on_device(x=x2, out=y2)
    _need_cuda(plan)
    yt = _yt(out)
    _check(lib().vbq_gemv_planned(ctypes.byref(P), _ptr(plan), M, _ptr(x2), x2.stride(0), _ptr(y2), y2.stride(0), yt,
                                  _stream()), "vbq_gemv_planned")
    return out


def gemv_planned_swiglu(P: Plan, plan, x, out=None, out_dtype=None):
    """silu(gate) * up per output pair of an interleaved (gate, up) matrix plan
    -> [M][N/2] (or [N/2] for 1-D x)."""
    torch = _torch()
    x2 = _x2(x, P.K)
    M = x2.shape[0]
    out_dtype = out_dtype or torch.float16
    if out is None:
        out = torch.empty((M, P.N // 2) if x.dim() == 2 else (P.N // 2,), dtype=out_dtype, device=x.device)
    h2 = _y2(out, M, P.N // 2, x.dim() == 1)
    _on_device(x=x2, out=h2)
    _need_cuda(plan)
    ht = _yt(out)
    _check(lib().vbq_gemv_planned_swiglu(ctypes.byref(P), _ptr(plan), M, _ptr(x2), x2.stride(0), _ptr(h2),
                                         h2.stride(0), ht, _stream()), "vbq_gemv_planned_swiglu")
    return out


ARGMAX_WS_BYTES = 8 * 16 + 16 + 4 * 16 + 4 * 16  # sizeof(vbq_argmax_ws)


def argmax_workspace(device="cuda"):
    """A zeroed vbq_argmax_ws (int32 tensor view; index at [36:52], value bits at [52:68])."""
    torch = _torch()
    return torch.zeros(ARGMAX_WS_BYTES // 4, dtype=torch.int32, device=device)


def gemv_planned_argmax(P: Plan, plan, x, ws=None):
    """Greedy-decode argmax of W x per token from a plan: -> (index int32[M], value float32[M])
    device tensors (views into the workspace, valid until its next use)."""
    torch = _torch()
    x2 = _x2(x, P.K)
    M = x2.shape[0]
    _on_device(x=x2)
    _need_cuda(plan)
    if ws is None:
        ws = argmax_workspace(x.device)
    if ws.dtype != torch.int32 or ws.numel() * 4 < ARGMAX_WS_BYTES:
        raise ValueError(f"ws must be an int32 tensor of {ARGMAX_WS_BYTES // 4} entries")
    _need_cuda(ws)
    _check(lib().vbq_gemv_planned_argmax(ctypes.byref(P), _ptr(plan), M, _ptr(x2), x2.stride(0), _ptr(ws),
                                         _stream()), "vbq_gemv_planned_argmax")
    return ws[36:36 + M], ws[52:52 + M].view(torch.float32)


def gemv_planned_argmax_noalloc(P: Plan, plan, x, index=None, value=None):
    """vbq_gemv_planned_argmax without a workspace (the library's own device
    array holds the keys): -> (index int32[M], value float32[M])."""
    torch = _torch()
    x2 = _x2(x, P.K)
    M = x2.shape[0]
    _on_device(x=x2)
    _need_cuda(plan)
    if index is None:
        index = torch.empty(M, dtype=torch.int32, device=x.device)
    if value is None:
        value = torch.empty(M, dtype=torch.float32, device=x.device)
    _need_cuda(index, value)
    if index.dtype != torch.int32 or value.dtype != torch.float32 or index.numel() < M or value.numel() < M:
        raise ValueError("index must be int32 and value float32 device tensors of M entries")
    _check(lib().vbq_gemv_planned_argmax_noalloc(ctypes.byref(P), _ptr(plan), M, _ptr(x2), x2.stride(0),
                                                 _ptr(index), _ptr(value), _stream()),
           "vbq_gemv_planned_argmax_noalloc")
    return index, value


def gemv_planned_shared(plans, x, outs=None, out_dtype=None):
    """[W_i x for (P_i, plan_i) in plans] in one launch (shared activations x)."""
    torch = _torch()
    if not plans:
        raise ValueError("no plans")
    one = x.dim() == 1
    x2 = _x2(x, plans[0][0].K)
    M = x2.shape[0]
    out_dtype = out_dtype or torch.float16
    if outs is None:
        outs = [torch.empty((M, P.N), dtype=out_dtype, device=x.device) for P, _ in plans]
    if len(outs) != len(plans):
        raise ValueError("one output per plan")
    ys = []
    for k, ((P, plan), out) in enumerate(zip(plans, outs)):
        if P.K != plans[0][0].K:
            raise ValueError("the plans of a shared launch have one K")
        ys.append(_y2(out, M, P.N, one, f"outs[{k}]"))
        if out.dtype != outs[0].dtype:
            raise ValueError("outputs have one dtype")
    items = (PlannedItem * len(plans))()
    for k, ((P, plan), y2) in enumerate(zip(plans, ys)):
        _on_device(x=x2, out=y2)
        _need_cuda(plan)
        items[k] = PlannedItem(ctypes.addressof(P), _ptr(plan), _ptr(y2), y2.stride(0))
    yt = _yt(outs[0])
    _check(lib().vbq_gemv_planned_shared(items, len(plans), M, _ptr(x2), x2.stride(0), yt, _stream()),
           "vbq_gemv_planned_shared")
    return outs


# -------------------------------------------------------- step executors

class Seq:
    """One decode step's GEMVs, in stage order, as one C call.

    ``items`` holds ``(L, blob, x, y, stage)`` (packed blobs, ``planned=False``)
    or ``(P, plan, x, y, stage)`` (prepared plans, ``planned=True``), with x a
    [M][K] (or [K]) fp16 device tensor and y a [M][N] (or [N]) device tensor,
    all outputs of one dtype.  The item array is built once; ``run()``
    enqueues the whole step on the current stream (vbq_gemv_seq /
    vbq_gemv_planned_seq), so it can be called inside a graph capture.  The
    object keeps references to everything the array points at.
    """

    def __init__(self, items, planned: bool):
        torch = _torch()
        items = list(items)
        if not items:
            raise ValueError("a step needs at least one GEMV")
        self.planned = planned
        self.keep = items
        Item = PlannedSeqItem if planned else SeqItem
        self.arr = (Item * len(items))()
        self.M = None
        ydt = None
        views = []
        for k, (meta, buf, x, y, stage) in enumerate(items):
            x2 = _x2(x, meta.K, f"items[{k}] x")
            if self.M is not None and x2.shape[0] != self.M:
                raise ValueError("every GEMV of a step has the same token count M")
            y2 = _y2(y, x2.shape[0], meta.N, x.dim() == 1, f"items[{k}] y")
            if ydt is not None and y2.dtype != ydt:
                raise ValueError("the outputs of a step have one dtype")
            self.M, ydt = x2.shape[0], y2.dtype
            views.append((x2, y2))
        for k, ((meta, buf, x, y, stage), (x2, y2)) in enumerate(zip(items, views)):
            _on_device(x=x2, y=y2)
            _need_cuda(buf)
            self.arr[k] = Item(ctypes.addressof(meta), _ptr(buf), _ptr(x2), x2.stride(0), _ptr(y2), y2.stride(0),
                               int(stage))
        self.yt = VBQ_F32 if ydt == torch.float32 else VBQ_F16
        self.n = len(items)

    def run(self):
        if self.planned:
            _check(lib().vbq_gemv_planned_seq(self.arr, self.n, self.M, self.yt, _stream()), "vbq_gemv_planned_seq")
        else:
            _check(lib().vbq_gemv_seq(self.arr, self.n, self.M, self.yt, None, 0, _stream()), "vbq_gemv_seq")


def gemv_seq(items):
    """Run one step over packed blobs: items of (L, blob, x, y, stage)."""
    Seq(items, planned=False).run()


def gemv_planned_seq(items):
    """Run one step over prepared plans: items of (P, plan, x, y, stage)."""
    Seq(items, planned=True).run()


# -------------------------------------------------------------- prefill GEMM

def gemm_plan_init(L: Layout, blob) -> GemmPlan:
    """Geometry of the GEMM plan of (L, blob). Synchronizes."""
    torch = _torch()
    _need_cuda(blob)
    ws = torch.empty(16, dtype=torch.uint8, device=blob.device)
    GP = GemmPlan()
    _check(lib().vbq_gemm_plan_init(ctypes.byref(L), _ptr(blob), ctypes.byref(GP), _ptr(ws), 16, _stream()),
           "vbq_gemm_plan_init")
    return GP


def gemm_prepare(L: Layout, blob, check: bool = True):
    """GEMM plan of a packed matrix -> (plan u8 device tensor, GemmPlan).
    With ``check`` the device status word is read back (synchronizes)."""
    torch = _torch()
    GP = gemm_plan_init(L, blob)
    buf = _empty_aligned(GP.total_bytes, blob.device)
    status = torch.empty(1, dtype=torch.int32, device=blob.device)
    _check(lib().vbq_gemm_prepare(ctypes.byref(GP), ctypes.byref(L), _ptr(blob), _ptr(buf), _ptr(status),
                                  _stream()), "vbq_gemm_prepare")
    if check:
        status_check(status)
    return buf, GP


def gemm_workspace_size(GP: GemmPlan, M: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().vbq_gemm_workspace(ctypes.byref(GP), M, ctypes.byref(n)), "vbq_gemm_workspace")
    return n.value


def gemm_workspace(GP: GemmPlan, M: int, device="cuda"):
    """A workspace for vbq_gemm calls of up to M tokens (any contents)."""
    return _empty_aligned(max(gemm_workspace_size(GP, M), 256), device)


def gemm(GP: GemmPlan, buf, x, out=None, out_dtype=None, ws=None):
    """Y[M][N] = X[M][K] W^T from a GEMM plan (the prefill path, M > 16)."""
    torch = _torch()
    x2 = _x2(x, GP.K)
    M = x2.shape[0]
    out_dtype = out_dtype or torch.float16
    if out is None:
        out = torch.empty((M, GP.N) if x.dim() == 2 else (GP.N,), dtype=out_dtype, device=x.device)
    y2 = _y2(out, M, GP.N, x.dim() == 1)
    _on_device(x=x2, out=y2)
    _need_cuda(buf)
    yt = _yt(out)
    if ws is None:
        ws = gemm_workspace(GP, M, x.device)
    _check(lib().vbq_gemm(ctypes.byref(GP), _ptr(buf), M, _ptr(x2), x2.stride(0), _ptr(y2), y2.stride(0), yt,
                          _ptr(ws), ws.numel() * ws.element_size(), _stream()), "vbq_gemm")
    return out


def dense_f16_gemv(w16, x, out=None, out_dtype=None):
    """Dense fp16 control: y[M][N] = x[M][K] W16^T (or y[N] for 1-D x)."""
    torch = _torch()
    if w16.dtype != torch.float16 or w16.dim() != 2:
        raise ValueError("w16 must be a float16 [N][K] tensor")
    N, K = w16.shape
    one = x.dim() == 1
    x2 = _x2(x, K)
    M = x2.shape[0]
    out_dtype = out_dtype or torch.float16
    if out is None:
        out = torch.empty((N,) if one else (M, N), dtype=out_dtype, device=x.device)
    y2 = _y2(out, M, N, one)
    _on_device(x=x2, out=y2)
    _need_cuda(w16)
    yt = _yt(out)
    _check(lib().vbq_dense_f16_gemv(N, K, M, _ptr(w16), _ptr(x2), x2.stride(0), _ptr(y2), y2.stride(0), yt,
                                    _stream()), "vbq_dense_f16_gemv")
    return out
