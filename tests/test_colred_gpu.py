"""Column reductions (COL_SUM / COL_SUMSQ: one value per output column, over all
rows) on the GPU through the C ABI, against the fp64 oracle.  With the
GPT-2-medium backward layer the column sum of dH = (dY W2^T) * GELU'(P) is the
gradient of the bias added before the activation."""
import numpy as np
import pytest
import torch

import oracle
import workloads as w

from gpu_util import announce, assert_close, lib
from workloads.gen import to_f64

pytestmark = pytest.mark.gpu

U = 2.0 ** -8   # bf16 unit roundoff


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
    return [(n, {k: (f64(v) if isinstance(v, torch.Tensor) else v) for k, v in a.items() if k != "out"})
            for n, a in ops]


def backward_case(rng, M, N, K):
    dY = bf16(rng.standard_normal((M, K)))
    W2 = bf16(rng.standard_normal((N, K)) / np.sqrt(K))     # stored [N x K], used transposed
    P = bf16(rng.standard_normal((M, N)))
    return dY, W2, P


def run(CR, A, B, ops, layout, mode, tile=0):
    coda, runner = CR
    call = runner.Call(A, B, ops, layout, tile=tile)
    coda.check(call.fused() if mode == "fused" else call.unfused(), mode)
    torch.cuda.synchronize()
    return call


def unfused_bound_dgelu(dY, W2, P):
    """Unfused [mul_dgelu_tanh(P), ...]: the GEMM output C and D are stored in
    bf16, so |error| <= u |C| |GELU'(P)| + u |D| per element (first order)."""
    C = f64(dY) @ f64(W2).T
    g = oracle.gelu_tanh_grad(f64(P))
    return U * np.abs(C) * np.abs(g) + U * np.abs(C * g)


SHAPES = [(136, 264, 72), (520, 392, 136), (300, 520, 200), (64, 128, 64)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("mode", ["fused", "unfused"])
def test_bias_gradient_of_backward_layer(CR, shape, mode):
    M, N, K = shape
    announce(f"colred backward {shape} {mode}")
    rng = np.random.default_rng(81)
    dY, W2, P = backward_case(rng, M, N, K)
    db = torch.zeros((N, 1), dtype=torch.float32, device="cuda")
    rs = torch.zeros((M, 1), dtype=torch.float32, device="cuda")
    ops = [("mul_dgelu_tanh", {"mat": P}), ("col_sum", {"out": db, "col": 0}), ("row_sum", {"out": rs, "col": 0})]
    call = run(CR, dY, W2, ops, "NK", mode)
    ref, reds = oracle.forward(f64(dY), f64(W2), oracle_ops(ops), "NK")
    ext = None if mode == "fused" else unfused_bound_dgelu(dY, W2, P)
    assert_close(f64(call.D), ref, f"{mode} D", ext)
    assert_close(f64(db)[:, 0], reds[0][2], f"{mode} col_sum", None if ext is None else ext.sum(axis=0))
    assert_close(f64(rs)[:, 0], reds[1][2], f"{mode} row_sum", None if ext is None else ext.sum(axis=1))


@pytest.mark.parametrize("tile", [1, 2, 3])
@pytest.mark.parametrize("layout", ["KN", "NK"])
def test_column_reductions_every_tile_and_after_swiglu(CR, tile, layout):
    announce(f"colred tile{tile} {layout}")
    rng = np.random.default_rng(82)
    M, N, K = 520, 528, 200
    a = rng.standard_normal((M, K))
    b = rng.standard_normal((K, N)) / np.sqrt(K)
    A = bf16(a)
    B = bf16(b if layout == "KN" else np.ascontiguousarray(b.T))
    outs = torch.zeros((N, 3), dtype=torch.float32, device="cuda")
    rows = torch.zeros((M, 1), dtype=torch.float32, device="cuda")
    ops = [("add_col", {"vec": bf16(0.1 * rng.standard_normal(N))}), ("col_sumsq", {"out": outs, "col": 0}),
           ("swiglu_pair", {}), ("row_sum", {"out": rows, "col": 0}), ("col_sum", {"out": outs, "col": 1})]
    call = run(CR, A, B, ops, layout, "fused", tile)
    ref, reds = oracle.forward(f64(A), f64(B), oracle_ops(ops), layout)
    assert_close(f64(call.D), ref, "D")
    assert_close(f64(outs)[:, 0], reds[0][2], "col_sumsq (width N)")
    assert_close(f64(rows)[:, 0], reds[1][2], "row_sum")
    assert_close(f64(outs)[: N // 2, 1], reds[2][2], "col_sum after swiglu (width N/2)")
    assert np.all(f64(outs)[N // 2:, 1] == 0.0), "col_sum wrote past the width"
    assert np.all(f64(outs)[:, 2] == 0.0), "untouched output column written"
    # bitwise repeatable
    first = outs.clone()
    coda, _ = CR
    coda.check(call.fused(), "repeat")
    torch.cuda.synchronize()
    assert torch.equal(first, outs)


def test_column_reduction_counters_left_zero(CR):
    coda, runner = CR
    announce("colred workspace counters")
    rng = np.random.default_rng(83)
    M, N, K = 1100, 264, 72            # 5 tile rows of 256 (or 9 of 128)
    dY, W2, P = backward_case(rng, M, N, K)
    db = torch.zeros((N, 1), dtype=torch.float32, device="cuda")
    ops = [("mul_dgelu_tanh", {"mat": P}), ("col_sum", {"out": db, "col": 0})]
    for tile in (0, 1, 3):
        call = runner.Call(dY, W2, ops, "NK", tile=tile)
        ws = call.ws[0]
        assert ws is not None and ws.numel() > 0
        for _ in range(2):
            coda.check(call.fused(), "fused")
            torch.cuda.synchronize()
            # the column counters are the workspace's last uint32 [grid_n] region
            assert int(ws.view(torch.int32)[-64:].count_nonzero()) == 0
        ref, reds = oracle.forward(f64(dY), f64(W2), oracle_ops(ops), "NK")
        assert_close(f64(db)[:, 0], reds[0][2], f"col_sum tile{tile}")


def test_full_size_backward_layer_bias_gradient(CR):
    """The GPT-2-medium backward layer at its full shape (M = 8192 tokens,
    N = 4096, K = 1024), every row: the column sums of dH against the oracle."""
    coda, runner = CR
    spec = w.get_config(5)
    announce(f"colred full size {spec.M}x{spec.N}x{spec.K}")
    inputs = w.make_inputs(spec)
    dt = {t.name: t.dtype for t in spec.tensors}
    to_dev = lambda name: runner.storage_to_tensor(inputs[name], dt[name])
    dY, W2, P = to_dev("dY"), to_dev("W2"), to_dev("P")
    db = torch.zeros((spec.N, 1), dtype=torch.float32, device="cuda")
    ops = [("mul_dgelu_tanh", {"mat": P}), ("col_sum", {"out": db, "col": 0})]
    call = run(CR, dY, W2, ops, "NK", "fused")
    del call
    _, reds = oracle.forward(to_f64(inputs["dY"], "bf16"), to_f64(inputs["W2"], "bf16"),
                             [("mul_dgelu_tanh", {"mat": to_f64(inputs["P"], "bf16")}), ("col_sum", {})], "NK")
    assert_close(f64(db)[:, 0], reds[0][2], "full-size col_sum")
