"""The RMS norm's backward on the GPU: ROW_DOT (a row reduction of the running
value times a matrix), RMS_BWD (the norm's input gradient given its row
statistics) and RMS_DGAMMA (its gain gradient), through the C ABI, against the fp64 oracle.  Gradients are among
the operators the d9bl.com page's Fig. 4 splits into a GEMM and an epilogue;
the agentlenshq.com page ("How it works") has the primitives cover the backward
pass as well as the forward."""
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


def f32(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).cuda()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


SHAPES = [(136, 264, 72), (300, 520, 200), (64, 128, 64), (520, 392, 256)]


@pytest.mark.parametrize("mode", ["fused", "unfused"])
@pytest.mark.parametrize("shape", SHAPES)
def test_row_dot(CR, shape, mode):
    coda, runner = CR
    M, N, K = shape
    announce(f"row_dot {shape} {mode}")
    rng = np.random.default_rng(71)
    A = bf16(rng.standard_normal((M, K)))
    B = bf16(rng.standard_normal((K, N)) / np.sqrt(K))
    Mat = bf16(rng.standard_normal((M, N)))
    bias = bf16(0.1 * rng.standard_normal(N))
    outs = torch.zeros((M, 2), dtype=torch.float32, device="cuda")
    ops = [("add_col", {"vec": bias}), ("row_dot", {"mat": Mat, "out": outs, "col": 0}),
           ("gelu_tanh", {}), ("row_sum", {"out": outs, "col": 1})]
    call = runner.Call(A, B, ops, "KN")
    coda.check(call.fused() if mode == "fused" else call.unfused(), mode)
    torch.cuda.synchronize()
    o_ops = [("add_col", {"vec": f64(bias)}), ("row_dot", {"mat": f64(Mat)}), ("gelu_tanh", {}), ("row_sum", {})]
    ref, reds = oracle.forward(f64(A), f64(B), o_ops, "KN")
    extra = extra_d = None
    if mode == "unfused":
        # the sequence stores the GEMM output C and the biased value v in bf16
        # (2^-9 relative each) before it reduces and before GELU (|GELU'| < 1.13)
        C = oracle.forward(f64(A), f64(B), [], "KN")[0]
        v = oracle.forward(f64(A), f64(B), o_ops[:1], "KN")[0]
        extra = 2.0 ** -8 * (np.abs(v) * np.abs(f64(Mat))).sum(axis=1)
        extra_d = 1.13 * 2.0 ** -9 * (np.abs(C) + np.abs(v))
    assert_close(f64(outs)[:, 0], reds[0][2], f"row_dot {shape} {mode}", extra)
    assert_close(f64(call.D), ref, f"row_dot D {shape} {mode}", extra_d)


@pytest.mark.parametrize("tile", [1, 2, 3])
@pytest.mark.parametrize("layout", ["KN", "NK"])
def test_row_dot_every_tile(CR, tile, layout):
    coda, runner = CR
    announce(f"row_dot tile{tile} {layout}")
    rng = np.random.default_rng(72)
    M, N, K = 300, 520, 200
    b = rng.standard_normal((K, N)) / np.sqrt(K)
    A, B = bf16(rng.standard_normal((M, K))), bf16(b if layout == "KN" else np.ascontiguousarray(b.T))
    Mat = f32(rng.standard_normal((M, N)))
    outs = torch.zeros((M, 1), dtype=torch.float32, device="cuda")
    call = runner.Call(A, B, [("row_dot", {"mat": Mat, "out": outs, "col": 0})], layout, tile=tile)
    coda.check(call.fused(), "fused")
    torch.cuda.synchronize()
    _, reds = oracle.forward(f64(A), f64(B), [("row_dot", {"mat": f64(Mat)})], layout)
    assert_close(f64(outs)[:, 0], reds[0][2], f"row_dot tile{tile} {layout}")


def _rms_bwd_inputs(rng, M, Kf, Np, dtype="bf16"):
    """x [M x Kf] (the norm's input), gamma, the projection W [Kf x Np] and an
    upstream gradient dP [M x Np]; rows of x at several scales."""
    conv = bf16 if dtype == "bf16" else f32
    x = rng.standard_normal((M, Kf)) * rng.uniform(0.2, 4.0, (M, 1))
    x[0] = 0.5
    g = 1 + 0.2 * rng.standard_normal(Kf)
    W = rng.standard_normal((Kf, Np)) / np.sqrt(Kf)
    dP = rng.standard_normal((M, Np))
    return conv(x), conv(g), conv(W), conv(dP)


def _stats_from_oracle(X, G, W, dP, eps):
    # sum of squares of x, and t_i = sum_l dP_il P_il with P = rmsnorm(x) W
    x = f64(X)
    P = oracle.rmsnorm(x, f64(G), eps) @ f64(W)
    return np.stack([np.sum(x * x, axis=1), np.sum(f64(dP) * P, axis=1)], axis=1)


@pytest.mark.parametrize("mode", ["fused", "unfused"])
@pytest.mark.parametrize("shape", [(136, 264, 72), (300, 520, 200), (64, 128, 64), (520, 392, 256)])
def test_rms_bwd_op(CR, shape, mode):
    """dX = RMS_BWD(dP W^T): the GEMM reads W stored [Kf x Np] as its [N x K]
    operand; the row statistics are given (computed by the oracle from the
    seeded inputs)."""
    coda, runner = CR
    M, Kf, Np = shape
    announce(f"rms_bwd {shape} {mode}")
    rng = np.random.default_rng(73)
    X, G, W, dP = _rms_bwd_inputs(rng, M, Kf, Np)
    eps = 1e-5
    stats = f32(_stats_from_oracle(X, G, W, dP, eps))
    dg = torch.zeros((Kf, 1), dtype=torch.float32, device="cuda")
    ops = [("rms_dgamma", {"x": X, "eps": eps, "stats": stats, "sumsq_col": 0, "out": dg, "col": 0}),
           ("rms_bwd", {"x": X, "gamma": G, "eps": eps, "stats": stats, "sumsq_col": 0, "t_col": 1})]
    call = runner.Call(dP, W, ops, "NK")
    coda.check(call.fused() if mode == "fused" else call.unfused(), mode)
    torch.cuda.synchronize()
    ref, reds = oracle.forward(f64(dP), f64(W), [("rms_dgamma", {"x": f64(X), "eps": eps}),
                                                 ("rms_bwd", {"x": f64(X), "gamma": f64(G), "eps": eps})], "NK")
    extra = extra_g = None
    if mode == "unfused":
        # the sequence stores dP W^T in bf16 before the norm's backward scales
        # it by gamma / r and before the gain gradient sums it times x / r
        r = oracle.rms(f64(X), eps)
        e_dy = 2.0 ** -8 * np.abs(f64(dP) @ f64(W).T)
        extra = np.abs(f64(G))[None, :] * e_dy / r[:, None]
        extra_g = np.sum(e_dy * np.abs(f64(X)) / r[:, None], axis=0)
    assert_close(f64(call.D), ref, f"rms_bwd {shape} {mode}", extra)
    assert_close(f64(dg)[:, 0], reds[0][2], f"rms_dgamma {shape} {mode}", extra_g)


@pytest.mark.parametrize("tile", [1, 2, 3])
def test_rms_bwd_every_tile_f32(CR, tile):
    coda, runner = CR
    announce(f"rms_bwd tile{tile} f32")
    rng = np.random.default_rng(74)
    M, Kf, Np = 300, 520, 200
    X, G, W, dP = _rms_bwd_inputs(rng, M, Kf, Np, "f32")
    eps = 1e-6
    stats = f32(_stats_from_oracle(X, G, W, dP, eps))
    dg = torch.zeros((Kf, 2), dtype=torch.float32, device="cuda")
    ops = [("rms_dgamma", {"x": X, "eps": eps, "stats": stats, "out": dg, "col": 1}),
           ("rms_bwd", {"x": X, "gamma": G, "eps": eps, "stats": stats})]
    call = runner.Call(dP, W, ops, "NK", tile=tile, d_dtype=torch.float32)
    coda.check(call.fused(), "fused")
    torch.cuda.synchronize()
    ref, reds = oracle.forward(f64(dP), f64(W), [("rms_dgamma", {"x": f64(X), "eps": eps}),
                                                 ("rms_bwd", {"x": f64(X), "gamma": f64(G), "eps": eps})], "NK")
    assert_close(f64(call.D), ref, f"rms_bwd tile{tile} f32")
    assert_close(f64(dg)[:, 1], reds[0][2], f"rms_dgamma tile{tile} f32")
    assert np.all(f64(dg)[:, 0] == 0.0)


def test_rms_bwd_chain_with_row_dot(CR):
    """The whole backward of x -> rmsnorm -> projection on the GPU: the GEMM
    that produces dP = G H takes ROW_DOT against P (t), and dX's GEMM takes
    RMS_BWD with that t.  P is the forward output rounded to bf16 (an input
    here, from the oracle); the oracle's reference is built from G, H, x, gamma
    and W alone, so the bar adds the first-order effect of the bf16 roundings
    of dP and P."""
    coda, runner = CR
    announce("rms_bwd chain")
    rng = np.random.default_rng(75)
    M, Kf, Np, Kg = 260, 392, 264, 136
    X, Gm, W, _ = _rms_bwd_inputs(rng, M, Kf, Np)
    Gup = bf16(rng.standard_normal((M, Kg)))
    Hup = bf16(rng.standard_normal((Kg, Np)) / np.sqrt(Kg))
    eps = 1e-5
    x, g, Wf = f64(X), f64(Gm), f64(W)
    P_exact = oracle.rmsnorm(x, g, eps) @ Wf
    P = bf16(P_exact)
    stats = torch.zeros((M, 2), dtype=torch.float32, device="cuda")
    stats[:, 0] = f32(np.sum(x * x, axis=1))
    up = runner.Call(Gup, Hup, [("row_dot", {"mat": P, "out": stats, "col": 1})], "KN")
    coda.check(up.fused(), "dP with ROW_DOT")
    torch.cuda.synchronize()
    dP = up.D
    dg = torch.zeros((Kf, 1), dtype=torch.float32, device="cuda")
    dn = runner.Call(dP, W, [("rms_dgamma", {"x": X, "eps": eps, "stats": stats, "out": dg, "col": 0}),
                             ("rms_bwd", {"x": X, "gamma": Gm, "eps": eps, "stats": stats})], "NK")
    coda.check(dn.fused(), "dX with RMS_BWD")
    torch.cuda.synchronize()
    dP_ref = f64(Gup) @ f64(Hup)
    dX_ref, dg_ref = oracle.rmsnorm_backward(x, g, eps, dP_ref @ Wf.T)
    r = oracle.rms(x, eps)
    u = 2.0 ** -8
    # dP rounded once (u |dP|) in both terms; P rounded once inside t
    e_dy = u * np.abs(dP_ref) @ np.abs(Wf).T
    e_t = u * np.sum(np.abs(dP_ref) * (np.abs(P_exact) + np.abs(P_exact)), axis=1)
    extra = np.abs(g)[None, :] * e_dy / r[:, None] + np.abs(x) * (e_t / (Kf * r ** 2))[:, None]
    assert_close(f64(dn.D), dX_ref, "rms_bwd chain dX", extra)
    assert_close(f64(dg)[:, 0], dg_ref, "rms_bwd chain dgamma", np.sum(e_dy * np.abs(x) / r[:, None], axis=0))
    # t itself against the oracle's row dot of the exact dP with the stored P
    t_ref = np.sum(dP_ref * f64(P), axis=1)
    assert_close(f64(stats)[:, 1], t_ref, "chain t")


def test_rms_backward_text_program_end_to_end(CR):
    """The front end's backward statements, lowered with device operands and run
    through the C ABI, against the oracle's gradients."""
    from gemm_epilogue_transformer_bf16_amd.frontend import lower
    coda, runner = CR
    announce("rms backward text program")
    rng = np.random.default_rng(76)
    M, Kf, Np, eps = 136, 264, 72, 1e-5
    X, G, W, dP = _rms_bwd_inputs(rng, M, Kf, Np)
    st = f32(_stats_from_oracle(X, G, W, dP, eps))
    dg = torch.zeros((Kf, 1), dtype=torch.float32, device="cuda")
    ops = lower("""EPILOGUE {
        dg[0] = rmsdgamma(output, x, st, 1e-5);
        output = rmsnorm_backward(output, x, g, st, 1e-5);
    }""", {"x": X, "g": G, "st": st, "dg": dg}, M, Kf)
    call = runner.Call(dP, W, ops, "NK")
    coda.check(call.fused(), "text program")
    torch.cuda.synchronize()
    dX_ref, dg_ref = oracle.rmsnorm_backward(f64(X), f64(G), eps, f64(dP) @ f64(W).T)
    assert_close(f64(call.D), dX_ref, "text program dX")
    assert_close(f64(dg)[:, 0], dg_ref, "text program dgamma")
