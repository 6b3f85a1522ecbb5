"""Edge cases of the column reductions, the weight-gradient layout, the folded
gains, LayerNorm and the given row sums: one row, one K chunk of 8, fewer rows
than a 32-row block, a single 8-column chunk, through the C ABI against the
fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as w

from gpu_util import announce, assert_close, lib

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def CR():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return lib()


def bf16(x):
    return torch.from_numpy(w.bf16_bits_from_f64(x).view(np.int16)).view(torch.bfloat16).cuda()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_ops(ops):
    return [(n, {k: (f64(v) if isinstance(v, torch.Tensor) else v) for k, v in a.items()
                 if k not in ("out", "row_ss", "row_ss_col", "row_s_col")}) for n, a in ops]


def run(CR, A, B, ops, layout="KN", **kw):
    coda, runner = CR
    call = runner.Call(A, B, ops, layout, **kw)
    coda.check(call.fused(), "fused")
    torch.cuda.synchronize()
    return call


@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (3, 16, 8), (31, 24, 16), (33, 8, 72)])
def test_column_reductions_few_rows(CR, M, N, K):
    announce(f"colred few rows {M}x{N}x{K}")
    rng = np.random.default_rng(111)
    A, B = bf16(rng.standard_normal((M, K))), bf16(rng.standard_normal((K, N)))
    outs = torch.zeros((N, 2), dtype=torch.float32, device="cuda")
    ops = [("silu", {}), ("col_sum", {"out": outs, "col": 0}), ("col_sumsq", {"out": outs, "col": 1})]
    call = run(CR, A, B, ops)
    ref, reds = oracle.forward(f64(A), f64(B), oracle_ops(ops), "KN")
    assert_close(f64(call.D), ref, "D")
    assert_close(f64(outs)[:, 0], reds[0][2], "col_sum")
    assert_close(f64(outs)[:, 1], reds[1][2], "col_sumsq")


@pytest.mark.parametrize("T,Fi,Fo", [(8, 8, 8), (8, 24, 16), (16, 8, 264)])
def test_weight_gradient_tiny(CR, T, Fi, Fo):
    announce(f"weight grad tiny {T}x{Fi}x{Fo}")
    rng = np.random.default_rng(112)
    X, dY = bf16(rng.standard_normal((T, Fi))), bf16(rng.standard_normal((T, Fo)))
    call = run(CR, X, dY, [("gelu_tanh", {})], a_layout="KM")
    ref, _ = oracle.forward(f64(X).T, f64(dY), [("gelu_tanh", {})], "KN")
    assert_close(f64(call.D), ref, "dW")


@pytest.mark.parametrize("fold", [False, True])
@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (5, 16, 8), (40, 24, 24)])
def test_norms_with_one_k_chunk(CR, M, N, K, fold):
    announce(f"norms tiny {M}x{N}x{K} fold={fold}")
    rng = np.random.default_rng(113)
    A = bf16(rng.standard_normal((M, K)) + 0.5)
    B = bf16(rng.standard_normal((K, N)) / np.sqrt(K))
    g = bf16(1 + 0.1 * rng.standard_normal(K))
    for ops in ([("rms_rowscale", {"gamma": g, "eps": 1e-6}), ("add_col", {"vec": bf16(rng.standard_normal(N))})],
                [("ln_rowscale", {"gamma": g, "beta": bf16(0.1 * rng.standard_normal(K)), "eps": 1e-5}),
                 ("silu", {})]):
        call = run(CR, A, B, ops, fold_gain=fold)
        ref, _ = oracle.forward(f64(A), f64(B), oracle_ops(ops), "KN")
        assert_close(f64(call.D), ref, f"{ops[0][0]} fold={fold}")


def test_given_row_sums_one_row(CR):
    announce("given row sums, one row")
    rng = np.random.default_rng(114)
    M, N, K = 1, 16, 24
    a = rng.standard_normal((M, K))
    A = bf16(a)
    B = bf16(rng.standard_normal((K, N)) / np.sqrt(K))
    ss = torch.from_numpy((f64(A) ** 2).sum(axis=1, keepdims=True).astype(np.float32)).cuda()
    g = bf16(1 + 0.1 * rng.standard_normal(K))
    ops = [("rms_rowscale", {"gamma": g, "eps": 1e-6, "row_ss": ss, "row_ss_col": 0})]
    call = run(CR, A, B, ops, fold_gain=True)
    ref, _ = oracle.forward(f64(A), f64(B), oracle_ops(ops), "KN")
    assert_close(f64(call.D), ref, "D")


def test_text_program_end_to_end(CR):
    """An epilogue program written as statements, lowered by the front end and
    run through the C ABI, against the oracle of the same lowered list."""
    from gemm_epilogue_transformer_bf16_amd.frontend import lower
    announce("text program end to end")
    rng = np.random.default_rng(115)
    M, N, K = 300, 264, 136
    A, B = bf16(rng.standard_normal((M, K))), bf16(rng.standard_normal((K, N)) / np.sqrt(K))
    stats = torch.zeros((M, 2), dtype=torch.float32, device="cuda")
    names = {"gamma": bf16(1 + 0.1 * rng.standard_normal(K)), "bias": bf16(0.1 * rng.standard_normal(N)),
             "R": bf16(rng.standard_normal((M, N))), "stats": stats}
    ops = lower("""EPILOGUE {
        output = rmsnorm(input, gamma, 1e-6);
        output = output + bias;
        output = gelu(output);
        output = output + 0.5 * R;
        stats[0] = rowsum(output);
        stats[1] = rowsumsq(output);
    }""", names, M, N)
    call = run(CR, A, B, ops)
    ref, reds = oracle.forward(f64(A), f64(B), oracle_ops(ops), "KN")
    assert_close(f64(call.D), ref, "D")
    assert_close(f64(stats)[:, 0], reds[0][2], "rowsum")
    assert_close(f64(stats)[:, 1], reds[1][2], "rowsumsq")
