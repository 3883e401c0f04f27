"""The Python binding rejects activations and outputs the C entry points cannot
check themselves (dtype, length, row count), before any library call.  CPU
tensors suffice: dtype and shape are checked before the device."""
import pytest

torch = pytest.importorskip("torch")

import decode_gemv_vbq_amd as v

N, K, M = 96, 128, 3


def f16(*shape):
    return torch.zeros(shape, dtype=torch.float16)


def plan():
    return v.Plan(magic=0, N=N, K=K, G=K // 64, M=2)


def layout():
    return v.layout_init(N, K)


def gemm_plan():
    return v.GemmPlan(magic=0, N=N, K=K, G=K // 64)


BUF = torch.zeros(256, dtype=torch.uint8)

# (name, call(x, out)) for every wrapper taking activations and one output
CALLS = [
    ("gemv_planned", lambda x, out: v.gemv_planned(plan(), BUF, x, out=out)),
    ("gemv_batched", lambda x, out: v.gemv_batched(layout(), BUF, x, out=out)),
    ("gemm", lambda x, out: v.gemm(gemm_plan(), BUF, x, out=out)),
    ("dense_f16_gemv", lambda x, out: v.dense_f16_gemv(f16(N, K), x, out=out)),
    ("gemv_planned_shared", lambda x, out: v.gemv_planned_shared([(plan(), BUF)], x, outs=[out])),
    ("gemv_shared", lambda x, out: v.gemv_shared([(layout(), BUF)], x, outs=[out])),
    ("seq_planned", lambda x, out: v.Seq([(plan(), BUF, x, out, 0)], planned=True)),
    ("seq_blob", lambda x, out: v.Seq([(layout(), BUF, x, out, 0)], planned=False)),
]


@pytest.mark.parametrize("name,call", CALLS, ids=[c[0] for c in CALLS])
def test_rejects_bad_activations_and_outputs(name, call):
    good_out = f16(M, N)
    with pytest.raises(ValueError, match="float16"):
        call(torch.zeros(M, K, dtype=torch.float32), good_out)  # fp32 x is not read as fp16
    with pytest.raises(ValueError, match="float16"):
        call(torch.zeros(M, K, dtype=torch.bfloat16), good_out)
    with pytest.raises(ValueError, match=f"K = {K}"):
        call(f16(M, K - 64), good_out)  # short x
    with pytest.raises(ValueError, match=f"K = {K}"):
        call(f16(M, K + 64), good_out)
    with pytest.raises(ValueError, match="float16 or float32"):
        call(f16(M, K), torch.zeros(M, N, dtype=torch.uint8))  # 1-byte outputs would take fp16 stores
    with pytest.raises(ValueError, match="shape"):
        call(f16(M, K), f16(M - 1, N))  # too few rows: the kernel would write past it
    with pytest.raises(ValueError, match="shape"):
        call(f16(M, K), f16(M, N - 1))
    with pytest.raises(ValueError, match=r"shape|must be \[M\]\[K\]"):
        call(f16(K), f16(N - 1))  # one token, short output (the batched call takes only [M][K])
    with pytest.raises(ValueError, match="device tensor"):
        call(f16(M, K), good_out)  # everything right but on the host


def test_single_token_gemv_checks():
    L = layout()
    with pytest.raises(ValueError, match="float16"):
        v.gemv(L, BUF, torch.zeros(K), out=f16(N))
    with pytest.raises(ValueError, match=f"K = {K}"):
        v.gemv(L, BUF, f16(K - 1), out=f16(N))
    with pytest.raises(ValueError, match="one contiguous token"):
        v.gemv(L, BUF, f16(2, K), out=f16(N))
    with pytest.raises(ValueError, match="device tensor"):
        v.gemv(L, BUF, f16(K), out=f16(N))


def test_swiglu_and_argmax_checks():
    P = plan()
    with pytest.raises(ValueError, match="shape"):
        v.gemv_planned_swiglu(P, BUF, f16(M, K), out=f16(M, N))  # outputs are N/2 wide
    with pytest.raises(ValueError, match="device tensor"):
        v.gemv_planned_swiglu(P, BUF, f16(M, K), out=f16(M, N // 2))
    with pytest.raises(ValueError, match=f"K = {K}"):
        v.gemv_planned_argmax(P, BUF, f16(M, 64))
    with pytest.raises(ValueError, match="float16"):
        v.gemv_planned_argmax_noalloc(P, BUF, torch.zeros(M, K))


def test_shared_launch_checks():
    P2 = v.Plan(magic=0, N=N, K=2 * K, G=2 * K // 64, M=2)
    with pytest.raises(ValueError, match="one K"):
        v.gemv_planned_shared([(plan(), BUF), (P2, BUF)], f16(M, K), outs=[f16(M, N), f16(M, N)])
    with pytest.raises(ValueError, match="one dtype"):
        v.gemv_planned_shared([(plan(), BUF), (plan(), BUF)], f16(M, K),
                              outs=[f16(M, N), torch.zeros(M, N, dtype=torch.float32)])
    with pytest.raises(ValueError, match="one output per"):
        v.gemv_planned_shared([(plan(), BUF), (plan(), BUF)], f16(M, K), outs=[f16(M, N)])
    with pytest.raises(ValueError, match="same token count"):
        v.Seq([(plan(), BUF, f16(M, K), f16(M, N), 0), (plan(), BUF, f16(M + 1, K), f16(M + 1, N), 1)],
              planned=True)
