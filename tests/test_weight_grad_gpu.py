"""The weight-gradient GEMM dW = X^T dY with A stored [K x M] (CODA_A_KM: X is
[tokens x features], tokens the contraction) on the GPU through the C ABI,
against the fp64 oracle of the transposed product."""
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
    return [(n, {k: (f64(v) if isinstance(v, torch.Tensor) else v) for k, v in a.items() if k != "out"})
            for n, a in ops]


def run(CR, X, dY, ops, layout, tile=0, mode="fused", D=None):
    coda, runner = CR
    call = runner.Call(X, dY, ops, layout, tile=tile, a_layout="KM", D=D)
    coda.check(call.fused() if mode == "fused" else call.unfused(), mode)
    torch.cuda.synchronize()
    return call


# (tokens T = K, features in = M, features out = N): ragged tails in every dimension
SHAPES = [(200, 136, 264), (520, 264, 392), (64, 128, 128), (1000, 392, 136)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("layout", ["KN", "NK"])
@pytest.mark.parametrize("mode", ["fused", "unfused"])
def test_weight_gradient(CR, shape, layout, mode):
    T, Fi, Fo = shape
    announce(f"weight grad {shape} {layout} {mode}")
    rng = np.random.default_rng(91)
    X = bf16(rng.standard_normal((T, Fi)))
    dy = rng.standard_normal((T, Fo)) / np.sqrt(T)
    dY = bf16(dy if layout == "KN" else np.ascontiguousarray(dy.T))
    ops = [("scale", {"alpha": 0.5})]
    call = run(CR, X, dY, ops, layout, mode=mode)
    ref, _ = oracle.forward(f64(X).T, f64(dY), oracle_ops(ops), layout)
    # unfused: one stored bf16 intermediate (the GEMM output) before the scale
    ext = None if mode == "fused" else 2.0 ** -8 * np.abs(ref)
    assert_close(f64(call.D), ref, f"dW {mode}", ext)


@pytest.mark.parametrize("tile", [1, 2, 3])
def test_weight_gradient_accumulates_every_tile(CR, tile):
    """dW_acc += X^T dY in place (ADD_MAT with D aliasing the accumulator),
    with the column sum of the update (a bias-style reduction over features)."""
    announce(f"weight grad accumulate tile{tile}")
    rng = np.random.default_rng(92)
    T, Fi, Fo = 600, 520, 264
    X = bf16(rng.standard_normal((T, Fi)))
    dY = bf16(rng.standard_normal((T, Fo)) / np.sqrt(T))
    acc0 = rng.standard_normal((Fi, Fo))
    acc = bf16(acc0)
    acc_ref = f64(acc)
    cs = torch.zeros((Fo, 1), dtype=torch.float32, device="cuda")
    ops = [("col_sum", {"out": cs, "col": 0}), ("add_mat", {"mat": acc, "beta": 1.0})]
    run(CR, X, dY, ops, "KN", tile=tile, D=acc)
    ref, reds = oracle.forward(f64(X).T, f64(dY), [("col_sum", {}), ("add_mat", {"mat": acc_ref, "beta": 1.0})], "KN")
    assert_close(f64(acc), ref, f"accumulated dW tile{tile}")
    assert_close(f64(cs)[:, 0], reds[0][2], f"column sum tile{tile}")


def test_weight_gradient_rejects_row_norm(CR):
    coda, runner = CR
    X = bf16(np.ones((64, 128)))
    dY = bf16(np.ones((64, 128)))
    call = runner.Call(X, dY, [("rms_rowscale", {"gamma": bf16(np.ones(64)), "eps": 1e-6})], "KN", a_layout="KM")
    assert call.fused() == coda.CODA_ERR_UNSUPPORTED


def test_weight_gradient_gpt2_small_mlp_up(CR):
    """The GPT-2-small MLP up-projection's weight gradient at its full shape:
    X [8192 tokens x 768], dY [8192 x 3072] -> dW [768 x 3072], K = 8192."""
    announce("weight grad GPT-2-small MLP up, full size")
    rng = np.random.default_rng(93)
    T, Fi, Fo = 8192, 768, 3072
    X = bf16(rng.standard_normal((T, Fi)))
    dY = bf16(rng.standard_normal((T, Fo)) / np.sqrt(T))
    call = run(CR, X, dY, [], "KN")
    ref = f64(X).T @ f64(dY)
    assert_close(f64(call.D), ref, "dW full size")
