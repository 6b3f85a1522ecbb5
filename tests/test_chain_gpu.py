"""Cross-layer chain: a layer's fp32 row sums of squares
(its ROW_SUMSQ output) feed the next layer's RMSNorm row scale, whose gain is
folded into the weights, so the next layer's main loop is the plain GEMM.
Checked against the fp64 oracle of the second layer on the stored output of
the first."""
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


# (tokens, hidden of layer 1 in, model width = K of layer 2, layer 2 GEMM width)
SHAPES = [(300, 200, 264, 528), (1000, 136, 392, 264)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("tile", [0, 1, 3])
def test_bert_stats_feed_the_next_rmsnorm(CR, shape, tile):
    coda, runner = CR
    T, H, Dm, N2 = shape
    announce(f"chain {shape} tile{tile}")
    rng = np.random.default_rng(101)
    # layer 1: the BERT-style down-projection with residual and row stats
    Hin = bf16(np.abs(rng.standard_normal((T, H))))
    W1 = bf16(rng.standard_normal((H, Dm)) / np.sqrt(H))
    bias = bf16(0.1 * rng.standard_normal(Dm))
    R = bf16(rng.standard_normal((T, Dm)))
    stats = torch.zeros((T, 2), dtype=torch.float32, device="cuda")
    ops1 = [("add_col", {"vec": bias}), ("add_mat", {"mat": R, "beta": 1.0}),
            ("row_sum", {"out": stats, "col": 0}), ("row_sumsq", {"out": stats, "col": 1})]
    c1 = runner.Call(Hin, W1, ops1, "KN", tile=tile)
    coda.check(c1.fused(), "layer 1")
    # layer 2: RMSNorm (its mean square from layer 1's stats) + SwiGLU
    W2 = bf16(rng.standard_normal((Dm, N2)) / np.sqrt(Dm))
    gamma = bf16(1 + 0.1 * rng.standard_normal(Dm))
    ops2 = [("rms_rowscale", {"gamma": gamma, "eps": 1e-6, "row_ss": stats, "row_ss_col": 1}), ("swiglu_pair", {})]
    c2 = runner.Call(c1.D, W2, ops2, "KN", tile=tile, fold_gain=True)
    coda.check(c2.fused(), "layer 2")
    torch.cuda.synchronize()
    # the oracle of layer 2 on layer 1's stored (bf16) output; the stats are of
    # its fp32 values before rounding, a difference far below the bar
    ref, _ = oracle.forward(f64(c1.D), f64(W2), [("rms_rowscale", {"gamma": f64(gamma), "eps": 1e-6}),
                                                 ("swiglu_pair", {})], "KN")
    assert_close(f64(c2.D), ref, f"chained layer 2 tile{tile}")
    # and the same layer gathering its own sums in the loop agrees
    ops2b = [("rms_rowscale", {"gamma": gamma, "eps": 1e-6}), ("swiglu_pair", {})]
    c3 = runner.Call(c1.D, W2, ops2b, "KN", tile=tile, fold_gain=True)
    coda.check(c3.fused(), "layer 2, own sums")
    torch.cuda.synchronize()
    assert_close(f64(c3.D), ref, "layer 2 own sums")


@pytest.mark.parametrize("tile", [0, 1, 3])
def test_bert_stats_feed_the_next_layernorm(CR, tile):
    """The BERT-style layer's (row sum, row sum of squares) output is exactly
    what the next layer's deferred LayerNorm needs: mean and variance."""
    coda, runner = CR
    T, H, Dm, N2 = 520, 136, 392, 264
    announce(f"chain LayerNorm tile{tile}")
    rng = np.random.default_rng(102)
    Hin = bf16(np.abs(rng.standard_normal((T, H))))
    W1 = bf16(rng.standard_normal((H, Dm)) / np.sqrt(H))
    R = bf16(rng.standard_normal((T, Dm)) + rng.standard_normal((T, 1)))   # rows with offsets
    stats = torch.zeros((T, 2), dtype=torch.float32, device="cuda")
    ops1 = [("add_mat", {"mat": R, "beta": 1.0}), ("row_sum", {"out": stats, "col": 0}),
            ("row_sumsq", {"out": stats, "col": 1})]
    c1 = runner.Call(Hin, W1, ops1, "KN", tile=tile)
    coda.check(c1.fused(), "layer 1")
    W2 = bf16(rng.standard_normal((Dm, N2)) / np.sqrt(Dm))
    gamma = bf16(1 + 0.1 * rng.standard_normal(Dm))
    beta = bf16(0.1 * rng.standard_normal(Dm))
    ops2 = [("ln_rowscale", {"gamma": gamma, "beta": beta, "eps": 1e-5, "row_ss": stats, "row_ss_col": 1,
                             "row_s_col": 0}), ("gelu_tanh", {})]
    c2 = runner.Call(c1.D, W2, ops2, "KN", tile=tile, fold_gain=True)
    coda.check(c2.fused(), "layer 2")
    torch.cuda.synchronize()
    ref, _ = oracle.forward(f64(c1.D), f64(W2), [("ln_rowscale", {"gamma": f64(gamma), "beta": f64(beta),
                                                                  "eps": 1e-5}), ("gelu_tanh", {})], "KN")
    assert_close(f64(c2.D), ref, f"chained LayerNorm layer 2 tile{tile}")


def test_given_sums_need_the_folded_gain(CR):
    coda, runner = CR
    A = bf16(np.ones((64, 64)))
    B = bf16(np.ones((64, 128)))
    ss = torch.ones((64, 1), dtype=torch.float32, device="cuda")
    call = runner.Call(A, B, [("rms_rowscale", {"gamma": bf16(np.ones(64)), "eps": 1e-6, "row_ss": ss})], "KN")
    assert call.fused() == coda.CODA_ERR_UNSUPPORTED
