"""GPU checks of the decode-step executors (vbq_gemv_seq, vbq_gemv_planned_seq).

* A step of several stages (single GEMVs, a gate/up pair sharing x, two GEMVs
  of one stage with different x) gives, per matrix, the bits of the
  single-matrix calls the executor documents, and each output is within
  1e-3 * sum|w||x| of the oracle.
* Stage order: in a chain where stage k reads stage k-1's fp16 output, every
  output matches the oracle run on the GPU's own previous output.
* A captured step replays to the eager bits after its inputs change.
* M = 16 on the planned path (token chunks) equals the single-matrix call.
"""
import numpy as np
import pytest

import oracle
from decode_gemv_vbq_amd import workload as wl
from tests.gpu_util import to_dev, upload, within_bound

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def vbq():
    import decode_gemv_vbq_amd as v
    v.lib()
    return v


class Mat:
    def __init__(self, v, N, K, seed, M, scale_shift=0):
        spec = wl.MatrixSpec("t", N, K, wl.MIX_BASE, layer=seed, cluster=1)
        q, bits, s, x = wl.draw_matrix(spec, 92, M=M, outliers=0.0)
        if scale_shift:
            s = (s.view(np.float16) * np.float16(2.0 ** -scale_shift)).view(np.uint16)
        self.q, self.bits, self.s, self.x_host = q, bits, s, x
        dq, db, ds, dx = upload(q, bits, s, x, torch)
        self.blob, self.L = v.pack(dq, db, ds)
        self.x = dx
        self.N, self.K = N, K
        self.plan, self.P = None, None

    def prepare(self, v, M, wgs=0):
        self.plan, self.P = v.prepare(self.L, self.blob, M=min(2, M), wgs=wgs)


def step_mats(v, M):
    """stage 0: one GEMV; stage 1: gate + up sharing x; stage 2: two GEMVs with
    their own x; stage 3: one GEMV with K unlike the others."""
    A = Mat(v, 512, 1024, 1, M)
    G = Mat(v, 1536, 1024, 2, M)
    U = Mat(v, 1536, 1024, 3, M)
    U.x = G.x
    U.x_host = G.x_host
    B = Mat(v, 700, 1536, 4, M)
    C = Mat(v, 300, 1536, 5, M)
    D = Mat(v, 1000, 2112, 6, M)
    return [(A, 0), (G, 1), (U, 1), (B, 2), (C, 2), (D, 3)]


@pytest.mark.parametrize("M", [1, 2, 5])
@pytest.mark.parametrize("yt", [torch.float16, torch.float32])
def test_seq_blob_matches_single_calls_and_oracle(M, yt):
    v = vbq()
    mats = step_mats(v, M)
    ys = [torch.empty((M, m.N), dtype=yt, device="cuda") for m, _ in mats]
    v.gemv_seq([(m.L, m.blob, m.x, y, st) for (m, st), y in zip(mats, ys)])
    # the launches the executor documents: batched for a lone GEMV, shared for the gate/up pair
    ref = [torch.empty_like(y) for y in ys]
    A, G, U, B, C, D = [m for m, _ in mats]
    v.gemv_batched(A.L, A.blob, A.x, out=ref[0])
    v.gemv_shared([(G.L, G.blob), (U.L, U.blob)], G.x, outs=[ref[1], ref[2]])
    v.gemv_batched(B.L, B.blob, B.x, out=ref[3])
    v.gemv_batched(C.L, C.blob, C.x, out=ref[4])
    v.gemv_batched(D.L, D.blob, D.x, out=ref[5])
    torch.cuda.synchronize()
    for k, ((m, st), y, r) in enumerate(zip(mats, ys, ref)):
        assert torch.equal(y, r), f"item {k} stage {st}"
        y_ref, bound = oracle.gemv(m.q, m.bits, m.s, m.x_host)
        ok, worst, idx = within_bound(y.float().cpu().numpy(), y_ref, bound)
        assert ok, f"item {k}: worst err/bound {worst:.3g} at {idx}"


@pytest.mark.parametrize("M", [1, 2, 16])
def test_seq_planned_matches_single_calls_and_oracle(M):
    v = vbq()
    mats = step_mats(v, M)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for m, st in mats:
        # the gate/up pair splits the device in proportion to N, as a decode step does
        m.prepare(v, M, wgs=cus // 2 if st == 1 else 0)
    ys = [torch.empty((M, m.N), dtype=torch.float32, device="cuda") for m, _ in mats]
    v.gemv_planned_seq([(m.P, m.plan, m.x, y, st) for (m, st), y in zip(mats, ys)])
    ref = [torch.empty_like(y) for y in ys]
    for (m, _), r in zip(mats, ref):
        v.gemv_planned(m.P, m.plan, m.x, out=r)
    torch.cuda.synchronize()
    for k, ((m, st), y, r) in enumerate(zip(mats, ys, ref)):
        assert torch.equal(y, r), f"item {k} stage {st}"
        y_ref, bound = oracle.gemv(m.q, m.bits, m.s, m.x_host)
        ok, worst, idx = within_bound(y.cpu().numpy(), y_ref, bound)
        assert ok, f"item {k}: worst err/bound {worst:.3g} at {idx}"


@pytest.mark.parametrize("planned", [False, True])
def test_seq_stage_chain_reads_previous_outputs(planned):
    """Stage k's activations are stage k-1's fp16 outputs, in the same step."""
    v = vbq()
    M = 2
    shapes = [(512, 1024), (1536, 512), (768, 1536), (256, 768)]
    mats = [Mat(v, N, K, 10 + i, M, scale_shift=4) for i, (N, K) in enumerate(shapes)]
    ys = [torch.empty((M, m.N), dtype=torch.float16, device="cuda") for m in mats]
    xs = [mats[0].x] + ys[:-1]
    if planned:
        for m in mats:
            m.prepare(v, M)
        v.gemv_planned_seq([(m.P, m.plan, x, y, k) for k, (m, x, y) in enumerate(zip(mats, xs, ys))])
    else:
        v.gemv_seq([(m.L, m.blob, x, y, k) for k, (m, x, y) in enumerate(zip(mats, xs, ys))])
    torch.cuda.synchronize()
    x_prev = mats[0].x_host
    for k, (m, y) in enumerate(zip(mats, ys)):
        y_ref, bound = oracle.gemv(m.q, m.bits, m.s, x_prev)
        yh = y.cpu().numpy()
        assert np.isfinite(yh).all()
        ok, worst, idx = within_bound(yh.astype(np.float64), y_ref, bound)
        assert ok, f"stage {k}: worst err/bound {worst:.3g} at {idx}"
        x_prev = yh.view(np.uint16)


@pytest.mark.parametrize("planned", [False, True])
def test_seq_graph_replays_match_eager(planned):
    v = vbq()
    M = 2
    mats = step_mats(v, M)
    if planned:
        for m, _ in mats:
            m.prepare(v, M)
    ys = [torch.empty((M, m.N), dtype=torch.float16, device="cuda") for m, _ in mats]
    seq = v.Seq([((m.P if planned else m.L), (m.plan if planned else m.blob), m.x, y, st)
                 for (m, st), y in zip(mats, ys)], planned=planned)
    seq.run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq.run()
    torch.cuda.synchronize()
    xs = {id(m.x): m.x for m, _ in mats}
    for rep in range(3):
        gen = np.random.default_rng(100 + rep)
        for x in xs.values():
            new = (gen.standard_normal(tuple(x.shape)) * 0.5).astype(np.float16)
            x.copy_(to_dev(new, torch))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [y.clone() for y in ys]
        seq.run()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(got, ys)):
            assert torch.equal(a, b), f"replay {rep} item {k}"
