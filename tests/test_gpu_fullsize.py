"""Full-size parity: the decode steps exactly as bench.py times them (the same
DecodeStep object, HIP-graph replay, M = 1), checked against the oracle on
sampled output rows of every matrix, plus graph-replay consistency; and the
batched workload's full matrices (28672x8192 up, 8192x28672 down) at M = 16
through both the prepared plans and vbq_gemv_batched, sampled rows against the
oracle, with each token of the plan path equal to its own single-token run."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import within_bound

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def check_step(step):
    bad = []
    worst_all = 0.0
    for i, m in enumerate(step.mats):
        q, bits, s, x = m.sample
        y_ref, bound = oracle.gemv(q, bits, s, x)
        y = m.y[:, m.sample_rows].float().cpu().numpy().astype(np.float64)
        ok, worst, _ = within_bound(y, y_ref, bound)
        worst_all = max(worst_all, worst)
        if not ok:
            bad.append((i, m.spec.name, m.spec.layer, worst))
    return bad, worst_all


@pytest.mark.parametrize("name,rows", [("decode1b", 12), ("decode9b", 6)])
def test_decode_step_sampled_parity(name, rows):
    from decode_gemv_vbq_amd.step import DecodeStep
    step = DecodeStep(name, M=1, keep_rows=rows)
    step.capture()
    step.replay()
    torch.cuda.synchronize()
    bad, worst = check_step(step)
    assert not bad, f"{len(bad)} matrices outside the bound, first {bad[:3]}"
    print(f"{name}: worst err/bound {worst:.2e}")
    # replays interleaved with eager work give the eager result every time
    ref = [m.y.clone() for m in step.mats]
    for rep in range(3):
        for m in step.mats:
            m.y.fill_(float("nan"))
        _ = torch.randn(1024, device="cuda").sum().item()  # unrelated eager work
        step.replay()
        torch.cuda.synchronize()
        for m, r in zip(step.mats, ref):
            assert torch.equal(m.y, r), f"replay {rep}: {m.spec.name} layer {m.spec.layer}"
    step.run()
    torch.cuda.synchronize()
    for m, r in zip(step.mats, ref):
        assert torch.equal(m.y, r)


@pytest.mark.parametrize("variant,planned", [("clustered", True), ("clustered", False), ("u4", True), ("u8", True)])
def test_batched70b_m16_sampled_parity(variant, planned):
    from decode_gemv_vbq_amd.step import DecodeStep
    step = DecodeStep("batched70b", M=16, variant=variant, keep_rows=6, planned=planned)
    step.run()
    torch.cuda.synchronize()
    bad, worst = check_step(step)
    assert not bad, f"{variant} planned={planned}: {bad}"
    print(f"batched70b {variant} planned={planned} M=16: worst err/bound {worst:.2e}")
    if planned:
        import decode_gemv_vbq_amd as v
        for m in step.mats:
            for t in (0, 15):  # a token's bits do not depend on the batch it runs in
                yt = v.gemv_planned(m.P, m.plan, m.x[t].contiguous(), out_dtype=m.y.dtype)
                torch.cuda.synchronize()
                assert torch.equal(yt, m.y[t]), (m.spec.name, t)
