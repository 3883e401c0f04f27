"""One decode step: the stage-ordered VBQ GEMVs of a synthetic decoder, resident in HBM.

Builds every weight matrix of a workload on the device (seeded draw -> vbq_pack,
then, on the default path, vbq_prepare: the one-time plan each GEMV reads),
keeps the packed blobs, plans, activations, outputs and workspaces, and runs
the step through the step executor (one C call that enqueues the stage-ordered
launches on one stream) -- eagerly, or replayed from a captured HIP graph (one
host launch per step).  A stage is one GEMV, or the gate and up projections of
a layer, which read the same activations and run as one shared launch.  The bench times exactly this object and the full-size
parity test checks exactly this object.
"""
from __future__ import annotations

import numpy as np

import decode_gemv_vbq_amd as v
from decode_gemv_vbq_amd import accounting as acc
from decode_gemv_vbq_amd import workload as wl


class Matrix:
    __slots__ = ("spec", "L", "blob", "x", "y", "ws", "P", "plan", "pass_count", "sample_rows", "sample", "w16",
                 "y16")

    def __init__(self, spec, L, blob, x, y, ws):
        self.spec, self.L, self.blob, self.x, self.y, self.ws = spec, L, blob, x, y, ws
        self.P = None
        self.plan = None
        self.pass_count = 0
        self.sample_rows = None
        self.sample = None
        self.w16 = None
        self.y16 = None


def plan_read_bytes(m) -> int:
    """Bytes one GEMV over m's plan loads: 1536 per pass record of every row
    block (1 KiB of codes and the 512-byte word area: each lane loads 8 bytes
    of it whatever the width) and the width bytes of each wavefront."""
    return int(m.pass_count) * 1536 + int(m.P.wgs) * 16 * int(m.P.per_wave)


def count_passes(P, plan) -> int:
    """Pass records in use over all row blocks of a plan (nonzero width bytes)."""
    region = plan.view(int(P.wgs), int(P.region_bytes))
    off = int(P.passes) * 1536
    return int((region[:, off:off + 16 * int(P.per_wave)] != 0).sum().item())


class DecodeStep:
    def __init__(self, name: str = "decode9b", M: int = 1, variant: str = "clustered", device="cuda",
                 keep_rows: int = 0, out_dtype=None, log=None, planned: bool = True, sample_frac: float = 0.0,
                 copies: int = 1):
        import dataclasses

        import torch
        self.torch = torch
        self.planned = planned
        self.W = wl.workload(name, M=M, variant=variant)
        # `copies` repeats the workload's matrices with fresh draws (other
        # layer ids), stage after stage, so that a small workload streams its
        # weights from HBM instead of the memory-side cache
        self.copies = copies
        if copies > 1:
            self.W.mats = [dataclasses.replace(sp, layer=sp.layer + 1000 * c) for c in range(copies)
                           for sp in self.W.mats]
        self.M = M
        self.device = torch.device(device)
        self.out_dtype = out_dtype or torch.float16
        self.mats: list[Matrix] = []
        self.graph = None
        self.graph16 = None
        self.graph16t = None
        self._seq = None
        rng = np.random.default_rng(12345)
        self.stages: list[list[int]] = []
        # sample_frac keeps that fraction of the rows of every matrix of the
        # first copy (the device draws copied back), the inputs a CPU timing of
        # the oracle runs on
        n_one = len(self.W.mats) // copies
        every = max(40, len(self.W.mats) // 10)
        for i, spec in enumerate(self.W.mats):
            q, bits, s, x = wl.draw_matrix_torch(spec, self.W.wid, M, self.W.outliers, device=self.device)
            # the up projection reads the same activations as the gate projection
            # of its layer: one stage, one launch
            shares = (spec.name == "up" and self.mats and self.mats[-1].spec.name == "gate"
                      and self.mats[-1].spec.layer == spec.layer and self.mats[-1].spec.K == spec.K)
            if shares:
                x = self.mats[-1].x
                self.stages[-1].append(i)
            else:
                self.stages.append([i])
            blob, L = v.pack(q, bits, s.view(torch.float16))
            y = torch.empty((M, spec.N), dtype=self.out_dtype, device=self.device)
            ws = v.workspace(L, M, self.device)
            m = Matrix(spec, L, blob, x, y, ws)
            n_keep = max(keep_rows, int(round(sample_frac * spec.N))) if i < n_one else 0
            if n_keep:
                n_keep = min(n_keep, spec.N)
                rows = np.unique(np.concatenate([[0, spec.N - 1], rng.choice(spec.N, size=n_keep, replace=False)]))
                idx = torch.from_numpy(rows).to(self.device)
                m.sample_rows = rows
                m.sample = (q.index_select(0, idx).cpu().numpy(), bits.index_select(0, idx).cpu().numpy(),
                            s.index_select(0, idx).cpu().numpy().view(np.uint16),
                            x.cpu().numpy().view(np.uint16))
            del q, bits, s
            self.mats.append(m)
            if log and (i % every == 0 or i == len(self.W.mats) - 1):
                log(f"built {i + 1}/{len(self.W.mats)} matrices")
        torch.cuda.synchronize()
        self.shared_ok = [True] * len(self.stages)
        if self.planned:
            self.prepare_plans(log)

    def prepare_plans(self, log=None):
        """One plan per matrix.  The matrices of a shared stage split the
        device's compute units in proportion to their rows, so that the stage
        is one launch spanning the device once."""
        torch = self.torch
        cus = torch.cuda.get_device_properties(self.device).multi_processor_count
        for k, st in enumerate(self.stages):
            ms = [self.mats[i] for i in st]
            total = sum(m.spec.N for m in ms)
            for m in ms:
                wgs = 0 if len(ms) == 1 else max(1, round(cus * m.spec.N / total))
                m.plan, m.P = v.prepare(m.L, m.blob, M=min(2, self.M), wgs=wgs)
                m.pass_count = count_passes(m.P, m.plan)
            if len(ms) > 1:
                P0 = ms[0].P
                self.shared_ok[k] = all(m.P.K == P0.K and m.P.M == P0.M for m in ms)
        torch.cuda.synchronize()
        if log:
            log(f"prepared {len(self.mats)} plans, {self.plan_bytes() / 1e6:.1f} MB read per step")

    def plan_bytes(self) -> int:
        """Bytes the step's GEMVs read from memory: every pass record's code
        bytes and words as the kernel loads them (16 code bytes and 8 word
        bytes per lane of each pass, partly filled passes included), the width
        bytes, plus the activations once per matrix (the workgroups of a
        launch share them through the caches)."""
        tot = 0
        for m in self.mats:
            if m.P is None:
                continue
            tot += plan_read_bytes(m) + 2 * self.M * m.spec.K
        return tot

    # ------------------------------------------------------------- the step
    def seq(self):
        """The whole step as one executor call (vbq_gemv_planned_seq or
        vbq_gemv_seq), built once."""
        if self._seq is None:
            items = []
            for k, st in enumerate(self.stages):
                for i in st:
                    m = self.mats[i]
                    meta, buf = (m.P, m.plan) if self.planned else (m.L, m.blob)
                    items.append((meta, buf, m.x, m.y, k))
            self._seq = v.Seq(items, planned=self.planned)
        return self._seq

    def run(self):
        """Enqueue every GEMV of the step, in stage order, on the current stream."""
        self.seq().run()

    def run_stage(self, st):
        """Enqueue one stage: a single GEMV, or one launch for matrices sharing x."""
        if self.planned:
            ms = [self.mats[i] for i in st]
            if len(ms) == 1:
                m = ms[0]
                v.gemv_planned(m.P, m.plan, m.x, out=m.y)
            elif self.shared_ok[self.stages.index(st)]:
                v.gemv_planned_shared([(m.P, m.plan) for m in ms], ms[0].x, outs=[m.y for m in ms])
            else:
                for m in ms:
                    v.gemv_planned(m.P, m.plan, m.x, out=m.y)
            return
        if len(st) == 1:
            m = self.mats[st[0]]
            if self.M == 1:
                v.gemv(m.L, m.blob, m.x[0], out=m.y[0], ws=m.ws)
            else:
                v.gemv_batched(m.L, m.blob, m.x, out=m.y, ws=m.ws)
        else:
            ms = [self.mats[i] for i in st]
            v.gemv_shared([(m.L, m.blob) for m in ms], ms[0].x, outs=[m.y for m in ms])

    def run_stages(self, stages):
        for st in stages:
            self.run_stage(st)

    def capture_stages(self, stages):
        """A graph of the given stages, back to back."""
        torch = self.torch
        self.run_stages(stages)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run_stages(stages)
        torch.cuda.synchronize()
        return g

    def stage_name(self, st) -> str:
        return "+".join(self.mats[i].spec.name for i in st)

    def capture(self):
        torch = self.torch
        self.run()  # first launches set kernel attributes outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        torch.cuda.synchronize()
        self.graph = g
        return g

    def replay(self):
        self.graph.replay()

    # ------------------------------------------------------- fp16 control
    def build_control(self):
        torch = self.torch
        for m in self.mats:
            m.w16 = v.dequant(m.L, m.blob, torch.float16)
            m.y16 = torch.empty((self.M, m.spec.N), dtype=self.out_dtype, device=self.device)
        torch.cuda.synchronize()

    def run_control(self):
        for m in self.mats:
            v.dense_f16_gemv(m.w16, m.x, out=m.y16)

    def capture_control(self):
        torch = self.torch
        self.run_control()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run_control()
        torch.cuda.synchronize()
        self.graph16 = g
        return g

    def run_torch_control(self):
        """The same dense fp16 weights through torch.matmul (the vendor GEMV/GEMM)."""
        for m in self.mats:
            self.torch.mm(m.x, m.w16.t(), out=m.y16)

    def capture_torch_control(self):
        torch = self.torch
        self.run_torch_control()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run_torch_control()
        torch.cuda.synchronize()
        self.graph16t = g
        return g

    def free_control(self):
        for m in self.mats:
            m.w16 = None
            m.y16 = None
        self.graph16 = None
        self.graph16t = None

    # ----------------------------------------------------------- accounting
    def alg_bytes(self) -> int:
        return sum(acc.vbq_read_bytes(m.L, self.M) for m in self.mats)

    def layout_bytes(self) -> int:
        return sum(acc.vbq_layout_bytes(m.L, self.M) for m in self.mats)

    def dense_bytes(self) -> int:
        return sum(acc.dense_read_bytes(m.spec.N, m.spec.K, self.M) for m in self.mats)

    def weights(self) -> int:
        return sum(m.spec.N * m.spec.K for m in self.mats)

    def mean_bits(self) -> float:
        return 8.0 * sum(int(m.L.code_bytes) for m in self.mats) / (64.0 * sum(m.spec.N * m.spec.G for m in self.mats))
