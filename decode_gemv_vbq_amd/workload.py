"""Seeded synthetic workloads for the VBQ decode path.

This module only draws inputs; it holds none of the method's arithmetic (no
dequant, no packing, no products), so the oracle side and the GPU side can both
be fed from it without sharing any computation.

The shapes and statistics follow the "Variable Bit-width Quantization" page
(Abstract): 64-weight groups with widths in {1, 2, 4, 8}, 69% of groups at one
bit, an LM head near one bit, a first MLP block around 2.5 bits.  The pages
train on text corpora and report no weights; the synthetic draws below stand in
for a frozen recipe:

* widths i.i.d. per group from a mixture (or runs of 8 groups sharing a width);
* codes uniform on [0, 2^b - 1];
* scales fp16(exp(N(-4, 0.5^2)));
* activations fp16(N(0, 1)), optionally with 1% outlier channels at 20x.

Every tensor comes from ``numpy.random.default_rng(SeedSequence([20260703,
workload_id, layer, proj_id, field_id]))`` on the host, or from a torch
generator seeded from the same sequence on the device.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ROOT_SEED = 20260703

#: width mixture of the bulk of the layers (mean 1.79 bits)
MIX_BASE = {1: 0.69, 2: 0.15, 4: 0.12, 8: 0.04}
#: first MLP block / 1B MLP down projection (mean 2.65 bits)
MIX_WIDE = {1: 0.45, 2: 0.20, 4: 0.25, 8: 0.10}
#: LM head as the explicit probabilities (mean 1.03 bits)
MIX_HEAD = {1: 0.97, 2: 0.03}
#: LM head variant whose mean is the page's 1.09 bits
MIX_HEAD_109 = {1: 0.91, 2: 0.09}
MIX_U4 = {4: 1.0}
MIX_U8 = {8: 1.0}

FIELD_BITS, FIELD_CODES, FIELD_SCALES, FIELD_X, FIELD_OUTLIERS = range(5)


@dataclass(frozen=True)
class MatrixSpec:
    name: str
    N: int
    K: int
    mix: dict
    layer: int = 0
    proj_id: int = 0
    cluster: int = 1  # groups per run sharing one width (1 = i.i.d.)

    @property
    def G(self) -> int:
        return self.K // 64


@dataclass
class Workload:
    name: str
    wid: int
    mats: list
    M: int = 1
    outliers: float = 0.0  # fraction of x channels scaled by 20
    notes: str = ""
    extra: dict = field(default_factory=dict)


PROJ = {"qkv": 0, "o": 1, "gate": 2, "up": 3, "down": 4, "head": 5}


def _decoder(n_layers, d, qkv_n, ffn, vocab, first_mlp_mix, base_mix, head_mix):
    mats = []
    for layer in range(n_layers):
        mlp_mix = first_mlp_mix if layer == 0 else base_mix
        mats += [
            MatrixSpec("qkv", qkv_n, d, base_mix, layer, PROJ["qkv"]),
            MatrixSpec("o", d, d, base_mix, layer, PROJ["o"]),
            MatrixSpec("gate", ffn, d, mlp_mix, layer, PROJ["gate"]),
            MatrixSpec("up", ffn, d, mlp_mix, layer, PROJ["up"]),
            MatrixSpec("down", d, ffn, mlp_mix, layer, PROJ["down"]),
        ]
    mats.append(MatrixSpec("head", vocab, d, head_mix, n_layers, PROJ["head"]))
    return mats


def workload(name: str, M: int = 1, variant: str = "clustered", head_mix: dict | None = None) -> Workload:
    """Named workloads.

    linear768   one 768x768 layer, M=1
    mlp1b       one SwiGLU block of a ~1B decoder (gate/up 5632x2048, down 2048x5632)
    decode1b    a ~1B decoder step: 24 layers x (qkv, o, gate, up, down) + LM head 32000x2048
    decode9b    a ~9B decoder step: 32 layers (GQA qkv 6144x4096) + LM head 128256x4096
    batched70b  28672x8192 up and 8192x28672 down, M in {1,4,8,16}; variants
                clustered (runs of 8 groups), u4, u8; 1% outlier channels
    """
    if name == "linear768":
        return Workload(name, 0, [MatrixSpec("linear", 768, 768, MIX_BASE)], M=M)
    if name == "mlp1b":
        return Workload(name, 1, [
            MatrixSpec("gate", 5632, 2048, MIX_BASE, 0, PROJ["gate"]),
            MatrixSpec("up", 5632, 2048, MIX_BASE, 0, PROJ["up"]),
            MatrixSpec("down", 2048, 5632, MIX_WIDE, 0, PROJ["down"]),
        ], M=M)
    if name == "decode1b":
        return Workload(name, 2, _decoder(24, 2048, 6144, 5632, 32000, MIX_WIDE, MIX_BASE, head_mix or MIX_HEAD), M=M)
    if name == "decode9b":
        return Workload(name, 3, _decoder(32, 4096, 6144, 14336, 128256, MIX_BASE, MIX_BASE, head_mix or MIX_HEAD),
                        M=M)
    if name == "batched70b":
        mix, cl = {"clustered": (MIX_BASE, 8), "u4": (MIX_U4, 1), "u8": (MIX_U8, 1)}[variant]
        return Workload(name, 4, [
            MatrixSpec("up", 28672, 8192, mix, 0, PROJ["up"], cl),
            MatrixSpec("down", 8192, 28672, mix, 0, PROJ["down"], cl),
        ], M=M, outliers=0.01, extra={"variant": variant})
    raise KeyError(name)


WORKLOADS = ("linear768", "mlp1b", "decode1b", "decode9b", "batched70b")


def seed_sequence(wid: int, spec: MatrixSpec, fld: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([ROOT_SEED, wid, spec.layer, spec.proj_id, fld])


def rng(wid: int, spec: MatrixSpec, fld: int) -> np.random.Generator:
    return np.random.default_rng(seed_sequence(wid, spec, fld))


def torch_seed(wid: int, spec: MatrixSpec, fld: int) -> int:
    return int(seed_sequence(wid, spec, fld).generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


# ---------------------------------------------------------------- host draws

def draw_bits(spec: MatrixSpec, wid: int, N: int | None = None) -> np.ndarray:
    """u8[N][G] widths in {1,2,4,8}."""
    N = spec.N if N is None else N
    G = spec.G
    r = rng(wid, spec, FIELD_BITS)
    widths = np.array(sorted(spec.mix), dtype=np.uint8)
    p = np.array([spec.mix[w] for w in sorted(spec.mix)], dtype=np.float64)
    p = p / p.sum()
    runs = (G + spec.cluster - 1) // spec.cluster
    b = r.choice(widths, size=(N, runs), p=p)
    return np.ascontiguousarray(np.repeat(b, spec.cluster, axis=1)[:, :G]).astype(np.uint8)


def draw_codes(spec: MatrixSpec, wid: int, bits: np.ndarray) -> np.ndarray:
    """u8[N][K], uniform on [0, 2^b - 1] for each group's width b."""
    N, G = bits.shape
    r = rng(wid, spec, FIELD_CODES)
    raw = r.integers(0, 256, size=(N, G * 64), dtype=np.uint16).astype(np.uint8)
    mask = ((np.left_shift(1, bits.astype(np.uint16)) - 1).astype(np.uint8))
    return raw & np.repeat(mask, 64, axis=1)


def draw_scales(spec: MatrixSpec, wid: int, N: int | None = None) -> np.ndarray:
    """fp16 bit patterns u16[N][G] of exp(N(-4, 0.5^2))."""
    N = spec.N if N is None else N
    r = rng(wid, spec, FIELD_SCALES)
    return np.exp(r.normal(-4.0, 0.5, size=(N, spec.G))).astype(np.float16).view(np.uint16)


def draw_x(spec: MatrixSpec, wid: int, M: int, outliers: float = 0.0) -> np.ndarray:
    """fp16 bit patterns u16[M][K] of N(0,1), with round(outliers*K) channels at 20x."""
    r = rng(wid, spec, FIELD_X)
    z = r.normal(0.0, 1.0, size=(M, spec.K))
    if outliers > 0:
        ro = rng(wid, spec, FIELD_OUTLIERS)
        ch = ro.choice(spec.K, size=int(round(outliers * spec.K)), replace=False)
        z[:, ch] *= 20.0
    return z.astype(np.float16).view(np.uint16)


def draw_matrix(spec: MatrixSpec, wid: int, M: int = 1, outliers: float = 0.0, N: int | None = None):
    """(q, bits, scales, x) host arrays; N may shrink the row count (first rows)."""
    bits = draw_bits(spec, wid, N)
    q = draw_codes(spec, wid, bits)
    s = draw_scales(spec, wid, N)
    x = draw_x(spec, wid, M, outliers)
    return q, bits, s, x


# -------------------------------------------------------------- device draws

def draw_matrix_torch(spec: MatrixSpec, wid: int, M: int = 1, outliers: float = 0.0, device="cuda"):
    """Same distributions drawn on the device with seeded torch generators.

    Returns torch tensors (q u8[N][K], bits u8[N][G], scales i16 view of fp16
    bits [N][G], x fp16 [M][K]).  Used where the host draw would be too slow
    (full decode-step weight sets); values differ from the host draw.
    """
    import torch

    def gen(fld):
        g = torch.Generator(device=device)
        g.manual_seed(torch_seed(wid, spec, fld))
        return g

    N, G, K = spec.N, spec.G, spec.K
    widths = sorted(spec.mix)
    p = torch.tensor([spec.mix[w] for w in widths], dtype=torch.float64)
    cdf = torch.cumsum(p / p.sum(), 0).to(device=device, dtype=torch.float32)
    runs = (G + spec.cluster - 1) // spec.cluster
    u = torch.rand((N, runs), generator=gen(FIELD_BITS), device=device)
    idx = torch.searchsorted(cdf, u.contiguous(), right=True).clamp_(max=len(widths) - 1)
    wt = torch.tensor(widths, dtype=torch.uint8, device=device)
    bits = wt[idx].repeat_interleave(spec.cluster, dim=1)[:, :G].contiguous()
    raw = torch.randint(0, 256, (N, K), generator=gen(FIELD_CODES), device=device, dtype=torch.int16)
    mask = ((1 << bits.to(torch.int16)) - 1).repeat_interleave(64, dim=1)
    q = (raw & mask).to(torch.uint8)
    del raw, mask
    s = torch.exp(torch.randn((N, G), generator=gen(FIELD_SCALES), device=device) * 0.5 - 4.0).half()
    z = torch.randn((M, K), generator=gen(FIELD_X), device=device, dtype=torch.float32)
    if outliers > 0:
        n_out = int(round(outliers * K))
        ch = torch.randperm(K, generator=gen(FIELD_OUTLIERS), device=device)[:n_out]
        z[:, ch] *= 20.0
    return q, bits, s.view(torch.int16), z.half()
