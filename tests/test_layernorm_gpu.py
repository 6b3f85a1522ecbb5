"""Deferred LayerNorm on the GPU (the mean-centred row norm moved past the
projection, as the zeli.app page's "augment_me" comment moves a row-wise
norm's per-row factors; the norm of the d9bl.com page's Fig. 4 Transformer
operators), through the C ABI, against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as w

from gpu_util import announce, assert_close, lib, run_and_compare

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


def oracle_ops(ops):
    out = []
    for name, a in ops:
        out.append((name, {k: (f64(v) if isinstance(v, torch.Tensor) else v) for k, v in a.items() if k != "out"}))
    return out


# several tiles and ragged tails in every dimension, K of 1 to 4 K steps
SMALL = [(136, 264, 72), (300, 520, 200), (64, 128, 64), (520, 392, 256)]


@pytest.mark.parametrize("fold", [False, True])
@pytest.mark.parametrize("shape", SMALL)
@pytest.mark.parametrize("mode", ["fused", "unfused"])
def test_layernorm_workload_small(CR, shape, mode, fold):
    spec = w.scaled_config(6, *shape)
    run_and_compare(spec, w.make_inputs(spec), mode=mode, label=f"ln small {shape} fold={fold}",
                    check_determinism=(mode == "fused"), fold_gain=fold)


@pytest.mark.parametrize("fold", [False, True])
@pytest.mark.parametrize("tile", [1, 2, 3])
def test_layernorm_every_tile(CR, tile, fold):
    spec = w.scaled_config(6, 300, 520, 200)
    run_and_compare(spec, w.make_inputs(spec), tile=tile, label=f"ln tile{tile} fold={fold}", fold_gain=fold)


@pytest.mark.parametrize("fold", [False, True])
@pytest.mark.parametrize("mode", ["fused", "unfused"])
def test_layernorm_full_size_every_row(CR, mode, fold):
    spec = w.get_config(6)
    run_and_compare(spec, w.make_inputs(spec), mode=mode, label=f"ln full fold={fold}",
                    check_determinism=True, fold_gain=fold)


@pytest.mark.parametrize("layout", ["KN", "NK"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ln_fold_matches_oracle(CR, layout, dtype):
    coda, runner = CR
    announce(f"ln_fold {layout} {dtype}")
    rng = np.random.default_rng(61)
    K, N = 776, 1032
    b = rng.standard_normal((K, N)) / np.sqrt(K)
    g = 1 + 0.1 * rng.standard_normal(K)
    bt = 0.1 * rng.standard_normal(K)
    conv = bf16 if dtype == "bf16" else f32
    Bs = conv(b if layout == "KN" else np.ascontiguousarray(b.T))
    G, BT = conv(g), conv(bt)
    u = torch.empty(N, dtype=torch.float32, device="cuda")
    c = torch.empty(N, dtype=torch.float32, device="cuda")
    st = coda.coda_ln_fold(Bs.data_ptr(), K, N, Bs.stride(0), coda.CODA_B_KN if layout == "KN" else coda.CODA_B_NK,
                           runner.CODA_DT[Bs.dtype], G.data_ptr(), BT.data_ptr(), u.data_ptr(), c.data_ptr(),
                           runner.current_stream_ptr())
    coda.check(st, "coda_ln_fold")
    torch.cuda.synchronize()
    Bl = oracle.logical_b(f64(Bs), layout)
    u_ref, c_ref = oracle.ln_fold(Bl, f64(G), f64(BT))
    # fp32 sums of exact products: |error| <= K * 2^-24 * sum_k |w_k b_kj|
    bound_u = K * 2.0 ** -24 * (np.abs(f64(G)) @ np.abs(Bl)) + 1e-30
    bound_c = K * 2.0 ** -24 * (np.abs(f64(BT)) @ np.abs(Bl)) + 1e-30
    assert np.all(np.abs(f64(u) - u_ref) <= bound_u)
    assert np.all(np.abs(f64(c) - c_ref) <= bound_c)


def _ln_case(CR, A, B, layout, gamma, beta, eps, extra_ops=(), tile=0, d_dtype=None, label="", fold=False):
    coda, runner = CR
    ops = [("ln_rowscale", {"gamma": gamma, "beta": beta, "eps": eps})] + list(extra_ops)
    call = runner.Call(A, B, ops, layout, tile=tile, d_dtype=d_dtype, fold_gain=fold)
    coda.check(call.fused(), f"fused {label}")
    torch.cuda.synchronize()
    ref, reds = oracle.forward(f64(A), f64(B), oracle_ops(ops), layout)
    assert_close(f64(call.D), ref, f"{label} D")
    return call, reds


def fused_ln_operand_bound(A, gamma, B, eps):
    """Worst-case first-order error of the fused GEMM output under LN_ROWSCALE.

    The fused path feeds the MFMA bf16((x - s) * gamma), s being the mean of the
    row's first 64 stored values (zeros past K), and scales by rstd afterwards:
    each product term carries a rounding of at most u = 2^-8 relative, so
    |error[i, j]| <= u * rstd_i * sum_k |x_ik - s_i| |gamma_k| |B_kj|.
    """
    A = np.asarray(A, dtype=np.float64)
    K = A.shape[1]
    first = np.zeros((A.shape[0], 64))
    first[:, :min(64, K)] = A[:, :min(64, K)]
    s = first.sum(axis=1) / 64.0
    mu = A.mean(axis=1)
    rstd = 1.0 / np.sqrt(((A - mu[:, None]) ** 2).mean(axis=1) + eps)
    return 2.0 ** -8 * rstd[:, None] * ((np.abs(A - s[:, None]) * np.abs(gamma)[None, :]) @ np.abs(B))


@pytest.mark.parametrize("layout", ["KN", "NK"])
def test_layernorm_b_nk_and_reductions(CR, layout):
    announce(f"ln {layout} with reductions")
    rng = np.random.default_rng(62)
    M, N, K = 260, 392, 136
    a = rng.standard_normal((M, K)) + rng.standard_normal((M, 1))
    b = rng.standard_normal((K, N)) / np.sqrt(K)
    A = bf16(a)
    B = bf16(b if layout == "KN" else np.ascontiguousarray(b.T))
    outs = torch.zeros((M, 2), dtype=torch.float32, device="cuda")
    extra = [("add_col", {"vec": bf16(0.1 * rng.standard_normal(N))}), ("row_sum", {"out": outs, "col": 0}),
             ("silu", {}), ("row_sumsq", {"out": outs, "col": 1})]
    G = bf16(1 + 0.1 * rng.standard_normal(K))
    BT = bf16(0.1 * rng.standard_normal(K))
    _, reds = _ln_case(CR, A, B, layout, G, BT, 1e-5, extra, label=f"ln {layout}")
    # The reductions see the fp32 values, so the operand rounding of the deferred
    # form adds up along the row: with E the bound above, row_sum (after add_col)
    # is off by at most sum_j E, and row_sumsq (after silu, |silu'| < 1.1) by
    # sum_j (2 |v| 1.1 E + (1.1 E)^2), v the value it squares.
    E = fused_ln_operand_bound(f64(A), f64(G), oracle.logical_b(f64(B), layout), 1e-5)
    v_sq = oracle.forward(f64(A), f64(B), oracle_ops(
        [("ln_rowscale", {"gamma": G, "beta": BT, "eps": 1e-5})] + extra[:1] + extra[2:3]), layout)[0]
    red_extra = [E.sum(axis=1), (2 * np.abs(v_sq) * 1.1 * E + (1.1 * E) ** 2).sum(axis=1)]
    for i, (_, _, r) in enumerate(reds):
        assert_close(f64(outs)[:, i], r, f"ln {layout} reduction {i}", red_extra[i])


def test_layernorm_degenerate_rows(CR):
    """Rows the deferred form must not lose: constant rows (zero variance: the
    output is beta's term alone), rows whose mean is large against their
    spread, a zero row, and ordinary rows."""
    announce("ln degenerate rows")
    rng = np.random.default_rng(63)
    M, N, K = 192, 264, 200
    a = rng.standard_normal((M, K))
    a[0] = 3.0
    a[1] = -0.75
    a[2] = 0.0
    a[3] = 64.0 + 0.25 * rng.standard_normal(K)
    a[4] = -100.0 + rng.standard_normal(K)
    a[5, :] = 1.0
    a[5, 0] = 2.0            # the row's first element (the shift) is the outlier
    a[130] = 5.0             # in a second tile row
    b = rng.standard_normal((K, N)) / np.sqrt(K)
    A, B = bf16(a), bf16(b)
    for tile in (0, 1, 3):
        g, bt = bf16(1 + 0.1 * rng.standard_normal(K)), bf16(0.2 * rng.standard_normal(K))
        bias = bf16(0.1 * rng.standard_normal(N))
        for fold in (False, True):
            _ln_case(CR, A, B, "KN", g, bt, 1e-5, [("add_col", {"vec": bias})], tile=tile, fold=fold,
                     label=f"ln degenerate tile{tile} fold={fold}")


@pytest.mark.parametrize("layout", ["KN", "NK"])
def test_layernorm_f32_operands(CR, layout):
    announce(f"ln f32 operands {layout}")
    rng = np.random.default_rng(64)
    M, N, K = 100, 200, 64
    a = rng.standard_normal((M, K)) + 2.0 * rng.standard_normal((M, 1))
    a[7] = 1.5
    b = rng.standard_normal((K, N)) / np.sqrt(K)
    A = f32(a)
    B = f32(b if layout == "KN" else np.ascontiguousarray(b.T))
    _ln_case(CR, A, B, layout, f32(1 + 0.1 * rng.standard_normal(K)), f32(0.1 * rng.standard_normal(K)), 1e-5,
             [("gelu_tanh", {})], d_dtype=torch.float32, label=f"ln f32 {layout}")


def test_layernorm_without_beta_and_unfused_agree(CR):
    coda, runner = CR
    announce("ln without beta, fused vs oracle and unfused vs oracle")
    rng = np.random.default_rng(65)
    M, N, K = 200, 328, 96
    A = bf16(rng.standard_normal((M, K)) + 0.5)
    B = bf16(rng.standard_normal((K, N)) / np.sqrt(K))
    ops = [("ln_rowscale", {"gamma": bf16(1 + 0.1 * rng.standard_normal(K)), "eps": 1e-5}), ("gelu_tanh", {})]
    call = runner.Call(A, B, ops, "KN")
    coda.check(call.fused(), "fused")
    torch.cuda.synchronize()
    ref, _ = oracle.forward(f64(A), f64(B), oracle_ops(ops), "KN")
    assert_close(f64(call.D), ref, "ln no beta fused")
    coda.check(call.unfused(), "unfused")
    torch.cuda.synchronize()
    # unfused: normalised A and the GEMM output are stored in bf16
    Y = oracle.layernorm(f64(A), f64(ops[0][1]["gamma"]), 1e-5)
    u = 2.0 ** -8
    extra = u * (np.abs(Y) @ np.abs(f64(B))) + 2 * u * np.abs(Y @ f64(B))
    assert_close(f64(call.D), ref, "ln no beta unfused", extra)
