"""Pins of the fp64 oracle against things other than itself.

Each test ties one part of the oracle to brute force on tiny inputs, a closed
form, an exact algebraic identity, or an independent library routine, so that
a dropped term, a wrong sign or index, or a transposed operand fails.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import coda_oracle as co
import workloads as w


# ----------------------------------------------------------------------------
# brute force: scalar pure-Python loops, written without numpy
# ----------------------------------------------------------------------------

def _bf_gelu(v):
    return 0.5 * v * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (v + 0.044715 * v * v * v)))


def _bf_sigmoid(v):
    return 1.0 / (1.0 + math.exp(-v)) if v >= 0 else math.exp(v) / (1.0 + math.exp(v))


def brute_force(A, B_logical, ops):
    """Scalar loops over lists: normalise -> triple-loop GEMM -> ops per element."""
    M, K = len(A), len(A[0]) if A else 0
    N = len(B_logical[0]) if B_logical else 0
    Y = [list(row) for row in A]
    ops = list(ops)
    if ops and ops[0][0] == "rms_rowscale":
        g, eps = ops[0][1]["gamma"], ops[0][1]["eps"]
        for i in range(M):
            ss = 0.0
            for k in range(K):
                ss += A[i][k] * A[i][k]
            r = math.sqrt(ss / K + eps)
            for k in range(K):
                Y[i][k] = A[i][k] / r * g[k]
        ops = ops[1:]
    elif ops and ops[0][0] == "ln_rowscale":
        g, eps = ops[0][1]["gamma"], ops[0][1]["eps"]
        bt = ops[0][1].get("beta", [0.0] * K)
        for i in range(M):
            mu = 0.0
            for k in range(K):
                mu += A[i][k]
            mu /= K
            var = 0.0
            for k in range(K):
                var += (A[i][k] - mu) * (A[i][k] - mu)
            var /= K
            for k in range(K):
                Y[i][k] = (A[i][k] - mu) / math.sqrt(var + eps) * g[k] + bt[k]
        ops = ops[1:]
    V = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = 0.0
            for k in range(K):
                s += Y[i][k] * B_logical[k][j]
            V[i][j] = s
    reds = []
    for name, a in ops:
        width = len(V[0]) if V else 0
        if name == "scale":
            V = [[x * a["alpha"] for x in row] for row in V]
        elif name == "scale_row":
            V = [[x * a["vec"][i] for x in row] for i, row in enumerate(V)]
        elif name == "scale_col":
            V = [[x * a["vec"][j] for j, x in enumerate(row)] for row in V]
        elif name == "add_col":
            V = [[x + a["vec"][j] for j, x in enumerate(row)] for row in V]
        elif name == "add_row":
            V = [[x + a["vec"][i] for x in row] for i, row in enumerate(V)]
        elif name == "add_mat":
            V = [[x + a.get("beta", 1.0) * a["mat"][i][j] for j, x in enumerate(row)] for i, row in enumerate(V)]
        elif name == "gelu_tanh":
            V = [[_bf_gelu(x) for x in row] for row in V]
        elif name == "silu":
            V = [[x * _bf_sigmoid(x) for x in row] for row in V]
        elif name == "swiglu_pair":
            V = [[row[2 * j] * _bf_sigmoid(row[2 * j]) * row[2 * j + 1] for j in range(width // 2)] for row in V]
        elif name == "mul_dgelu_tanh":
            h = 1e-5
            out = []
            for i, row in enumerate(V):
                out.append([x * (_bf_gelu(a["mat"][i][j] + h) - _bf_gelu(a["mat"][i][j] - h)) / (2 * h)
                            for j, x in enumerate(row)])
            V = out
        elif name == "row_sum":
            reds.append([sum(row) for row in V])
        elif name == "row_sumsq":
            reds.append([sum(x * x for x in row) for row in V])
        elif name == "row_mean":
            reds.append([sum(row) / len(row) for row in V])
        elif name == "col_sum":
            reds.append([sum(V[i][j] for i in range(len(V))) for j in range(width)])
        elif name == "col_sumsq":
            reds.append([sum(V[i][j] * V[i][j] for i in range(len(V))) for j in range(width)])
    return V, reds


def _tiny_case(rng, M, N, K, ints=False):
    if ints:
        A = rng.integers(-3, 4, size=(M, K)).astype(np.float64)
        B = rng.integers(-3, 4, size=(K, N)).astype(np.float64)
    else:
        A = rng.standard_normal((M, K))
        B = rng.standard_normal((K, N)) / math.sqrt(K)
    return A, B


def _lists(x):
    return [list(map(float, r)) for r in np.atleast_2d(x)]


def test_empty_list_is_textbook_gemm_exact_integers():
    rng = np.random.default_rng(1)
    for (M, N, K) in [(4, 4, 4), (3, 5, 4), (5, 2, 7)]:
        A, B = _tiny_case(rng, M, N, K, ints=True)
        D, reds = oracle.forward(A, B, [], "KN")
        V, _ = brute_force(_lists(A), _lists(B), [])
        assert reds == []
        assert np.array_equal(D, np.array(V))  # integer sums are exact in fp64


def test_b_layout_nk_is_transposed_storage():
    rng = np.random.default_rng(2)
    A, B = _tiny_case(rng, 3, 5, 4, ints=True)   # non-square, catches a transposed operand
    D_kn, _ = oracle.forward(A, B, [], "KN")
    D_nk, _ = oracle.forward(A, np.ascontiguousarray(B.T), [], "NK")
    V, _ = brute_force(_lists(A), _lists(B), [])
    assert np.array_equal(D_kn, np.array(V))
    assert np.array_equal(D_nk, np.array(V))
    with pytest.raises(ValueError):
        oracle.forward(A, B, [], "KK")


PROGRAMS = {
    "cfg1": lambda r, M, N, K: [("rms_rowscale", {"gamma": 1 + 0.1 * r.standard_normal(K), "eps": 1e-6}),
                                ("add_col", {"vec": 0.1 * r.standard_normal(N)}), ("gelu_tanh", {}),
                                ("add_mat", {"mat": r.standard_normal((M, N)), "beta": 1.0})],
    "cfg3": lambda r, M, N, K: [("add_col", {"vec": r.standard_normal(N)}),
                                ("add_mat", {"mat": r.standard_normal((M, N)), "beta": 0.5}),
                                ("row_sum", {}), ("row_sumsq", {})],
    "cfg4": lambda r, M, N, K: [("rms_rowscale", {"gamma": 1 + 0.1 * r.standard_normal(K), "eps": 1e-6}),
                                ("swiglu_pair", {}), ("row_mean", {})],
    "cfg5": lambda r, M, N, K: [("mul_dgelu_tanh", {"mat": r.standard_normal((M, N))}), ("row_sum", {})],
    "colred": lambda r, M, N, K: [("mul_dgelu_tanh", {"mat": r.standard_normal((M, N))}), ("col_sum", {}),
                                  ("add_col", {"vec": r.standard_normal(N)}), ("col_sumsq", {}),
                                  ("swiglu_pair", {}), ("col_sum", {}), ("row_sum", {})],
    "ln": lambda r, M, N, K: [("ln_rowscale", {"gamma": 1 + 0.1 * r.standard_normal(K),
                                               "beta": 0.1 * r.standard_normal(K), "eps": 1e-5}),
                              ("add_col", {"vec": r.standard_normal(N)}), ("gelu_tanh", {}), ("row_sum", {})],
    "scales": lambda r, M, N, K: [("scale", {"alpha": -1.5}), ("scale_row", {"vec": r.standard_normal(M)}),
                                  ("scale_col", {"vec": r.standard_normal(N)}), ("add_row", {"vec": r.standard_normal(M)}),
                                  ("silu", {}), ("row_sum", {})],
}


@pytest.mark.parametrize("prog", sorted(PROGRAMS))
def test_oracle_matches_brute_force(prog):
    rng = np.random.default_rng(7)
    M, N, K = 3, 6, 5
    A, B = _tiny_case(rng, M, N, K)
    ops = PROGRAMS[prog](rng, M, N, K)
    bf_ops = [(n, {k: (_lists(v) if isinstance(v, np.ndarray) and v.ndim == 2 else
                       (list(map(float, v)) if isinstance(v, np.ndarray) else v)) for k, v in a.items()})
              for n, a in ops]
    D, reds = oracle.forward(A, B, ops, "KN")
    V, bred = brute_force(_lists(A), _lists(B), bf_ops)
    # mul_dgelu_tanh's brute force uses a finite difference (error ~1e-10)
    tol = 1e-8 if prog in ("cfg5", "colred") else 1e-12
    assert np.allclose(D, np.array(V), rtol=tol, atol=tol)
    assert len(reds) == len(bred)
    for (_, _, r1), r2 in zip(reds, bred):
        assert np.allclose(r1, np.array(r2), rtol=tol, atol=tol)


# ----------------------------------------------------------------------------
# the deferred-scale identity (zeli.app comment: the row scale commutes past
# the following projection)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("idx", [1, 2, 4])
def test_deferred_equals_normalise_first_at_config_shapes(idx):
    spec = w.get_config(idx)
    M = min(spec.M, 512)       # rows are independent; a row block suffices for the identity
    rng = np.random.default_rng(spec.seed)
    X = rng.standard_normal((M, spec.K))
    g = 1 + 0.1 * rng.standard_normal(spec.K)
    W = rng.standard_normal((spec.K, spec.N)) / math.sqrt(spec.K)
    eps = 1e-6
    C_first = oracle.gemm(oracle.rmsnorm(X, g, eps), W)
    C_def = oracle.deferred_rmsnorm_gemm(X, g, W, eps)
    scale = np.abs(C_first).max()
    assert np.abs(C_first - C_def).max() <= 1e-12 * scale


def test_deferred_identity_small_exact_rows():
    # a row scaled by 2 has half the normalised output; the identity holds per row
    X = np.array([[1.0, 2.0, 2.0], [2.0, 4.0, 4.0]])
    g = np.array([1.0, 1.0, 1.0])
    W = np.eye(3)
    Y = oracle.rmsnorm(X, g, 0.0)
    assert np.allclose(Y[0], Y[1])
    assert np.allclose(Y[0], np.array([1, 2, 2]) / math.sqrt(3.0))   # rms([1,2,2]) = sqrt(9/3)
    assert np.allclose(oracle.deferred_rmsnorm_gemm(X, g, W, 0.0), Y)


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------

def test_rms_constant_row_closed_form():
    K, eps = 16, 1e-6
    for c in (0.0, 1e-4, 0.5, -3.0, 100.0):
        X = np.full((1, K), c)
        r = oracle.rms(X, eps)
        assert r[0] == pytest.approx(math.sqrt(c * c + eps), rel=1e-15)
        D, _ = oracle.forward(X, np.eye(K), [("rms_rowscale", {"gamma": np.ones(K), "eps": eps})])
        assert np.allclose(D, c / math.sqrt(c * c + eps), rtol=1e-14, atol=0)


def test_rms_mean_square_invariant_pins_mean_over_k_and_eps_inside_root():
    rng = np.random.default_rng(3)
    K, eps = 24, 0.25
    X = rng.standard_normal((5, K))
    D, _ = oracle.forward(X, np.eye(K), [("rms_rowscale", {"gamma": np.ones(K), "eps": eps})])
    ms = (X * X).mean(axis=1)
    assert np.allclose((D * D).mean(axis=1), ms / (ms + eps), rtol=1e-13)


def test_rms_gamma_scales_feature_not_row():
    K = 4
    X = np.array([[1.0, 1.0, 1.0, 1.0]])
    g = np.array([1.0, 2.0, 3.0, 4.0])
    D, _ = oracle.forward(X, np.eye(K), [("rms_rowscale", {"gamma": g, "eps": 0.0})])
    assert np.allclose(D[0], g)


# ----------------------------------------------------------------------------
# the mean-centred norm (LayerNorm) and its deferred form
# ----------------------------------------------------------------------------

def test_layernorm_zero_mean_rows_reduce_to_rmsnorm():
    # with every row's mean exactly zero, centring does nothing and the
    # variance is the mean square: LayerNorm is RMSNorm (pinned separately)
    rng = np.random.default_rng(11)
    K = 16
    H = rng.standard_normal((6, K // 2))
    X = np.concatenate([H, -H], axis=1)       # exact zero row sums
    g = 1 + 0.2 * rng.standard_normal(K)
    assert np.allclose(oracle.layernorm(X, g, 1e-3), oracle.rmsnorm(X, g, 1e-3), rtol=1e-14, atol=0)


def test_layernorm_moments_pin_centring_biased_variance_and_eps_inside_root():
    rng = np.random.default_rng(12)
    K, eps = 20, 0.5
    X = 3.0 + 2.0 * rng.standard_normal((7, K))     # far from zero mean
    Y = oracle.layernorm(X, np.ones(K), eps)
    var = X.var(axis=1)                              # numpy's default: 1/K
    assert np.allclose(Y.mean(axis=1), 0.0, atol=1e-14)
    assert np.allclose((Y * Y).mean(axis=1), var / (var + eps), rtol=1e-13)


def test_layernorm_invariant_to_row_shift_and_positive_row_scale():
    rng = np.random.default_rng(13)
    K = 12
    X = rng.standard_normal((4, K))
    g = rng.standard_normal(K)
    shift = rng.standard_normal((4, 1)) * 10
    Y0 = oracle.layernorm(X, g, 0.0)
    assert np.allclose(oracle.layernorm(X + shift, g, 0.0), Y0, rtol=1e-11, atol=1e-11)
    assert np.allclose(oracle.layernorm(X * 7.5, g, 0.0), Y0, rtol=1e-12, atol=1e-12)


def test_ln_fold_brute_force():
    rng = np.random.default_rng(14)
    K, N = 5, 3
    B = rng.standard_normal((K, N))
    g, b = rng.standard_normal(K), rng.standard_normal(K)
    u, c = oracle.ln_fold(B, g, b)
    for j in range(N):
        su = sc = 0.0
        for k in range(K):
            su += g[k] * B[k][j]
            sc += b[k] * B[k][j]
        assert u[j] == pytest.approx(su, rel=1e-13, abs=1e-13)
        assert c[j] == pytest.approx(sc, rel=1e-13, abs=1e-13)


@pytest.mark.parametrize("idx", [2, 3])
def test_deferred_layernorm_equals_normalise_first_at_config_shapes(idx):
    spec = w.get_config(idx)
    M = 256
    rng = np.random.default_rng(spec.seed + 1)
    X = rng.normal(0.5, 1.0, size=(M, spec.K)) + rng.normal(0, 1, size=(M, 1))
    g = 1 + 0.1 * rng.standard_normal(spec.K)
    b = 0.1 * rng.standard_normal(spec.K)
    W = rng.standard_normal((spec.K, spec.N)) / math.sqrt(spec.K)
    eps = 1e-5
    u, c = oracle.ln_fold(W, g, b)
    D_first, _ = oracle.forward(X, W, [("ln_rowscale", {"gamma": g, "eps": eps}), ("add_col", {"vec": c})])
    D_def = oracle.deferred_layernorm_gemm(X, g, b, W, eps)
    assert np.abs(D_first - D_def).max() <= 1e-11 * np.abs(D_first).max()
    # and beta folded after the projection is beta applied before it
    D_beta, _ = oracle.forward(X, W, [("ln_rowscale", {"gamma": g, "beta": b, "eps": eps})])
    assert np.abs(D_beta - D_first).max() <= 1e-11 * np.abs(D_first).max()


def test_hand_worked_layernorm_golden_case():
    import os
    g = _read_golden(os.path.join(os.path.dirname(__file__), "golden", "hand_layernorm_gemm.txt"))
    u, c = oracle.ln_fold(g["B"], g["gamma"], g["beta"])
    assert np.array_equal(u, g["u"]) and np.array_equal(c, g["c"])
    D, _ = oracle.forward(g["A"], g["B"], [("ln_rowscale", {"gamma": g["gamma"], "eps": 0.0}),
                                           ("add_col", {"vec": c})], "KN")
    assert np.allclose(D[0], g["D0"], rtol=1e-14) and np.allclose(D[1], g["D1"], rtol=1e-14)
    D, _ = oracle.forward(g["A"], g["B"], [("ln_rowscale", {"gamma": g["gamma"], "beta": g["beta"],
                                                            "eps": 0.0})], "KN")
    assert np.allclose(D[0], g["D0"], rtol=1e-14) and np.allclose(D[1], g["D1"], rtol=1e-14)
    D_def = oracle.deferred_layernorm_gemm(g["A"], g["gamma"], g["beta"], g["B"], 0.0)
    assert np.allclose(D_def, np.stack([g["D0"], g["D1"]]), rtol=1e-14)


def test_activation_closed_forms():
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert oracle.gelu_tanh_grad(np.array([0.0]))[0] == pytest.approx(0.5, abs=1e-15)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert oracle.gelu_tanh(np.array([10.0]))[0] == pytest.approx(10.0, abs=1e-12)
    assert abs(oracle.gelu_tanh(np.array([-10.0]))[0]) <= 1e-12
    # SiLU(+-1) = +-1 * e^{+-1} / (1 + e^{+-1})
    e = math.e
    assert oracle.silu(np.array([1.0]))[0] == pytest.approx(e / (1 + e), rel=1e-15)
    assert oracle.silu(np.array([-1.0]))[0] == pytest.approx(-1.0 / (1 + e), rel=1e-15)
    # symmetry: GELU(x) - GELU(-x) = x for the tanh form (tanh is odd)
    x = np.linspace(-6, 6, 241)
    assert np.allclose(oracle.gelu_tanh(x) - oracle.gelu_tanh(-x), x, atol=1e-14)


def test_gelu_tanh_close_to_erf_gelu():
    # the tanh form approximates x * Phi(x) to within ~4.7e-4 everywhere
    x = np.linspace(-8, 8, 4001)
    exact = np.array([v * 0.5 * (1 + math.erf(v / math.sqrt(2))) for v in x])
    dexact = np.array([0.5 * (1 + math.erf(v / math.sqrt(2))) + v * math.exp(-v * v / 2) / math.sqrt(2 * math.pi)
                       for v in x])
    assert np.abs(oracle.gelu_tanh(x) - exact).max() < 5e-4
    assert np.abs(oracle.gelu_tanh_grad(x) - dexact).max() < 1e-3


def test_gelu_grad_matches_central_difference():
    x = np.linspace(-6, 6, 1201)
    h = 1e-5
    fd = (oracle.gelu_tanh(x + h) - oracle.gelu_tanh(x - h)) / (2 * h)
    assert np.abs(oracle.gelu_tanh_grad(x) - fd).max() <= 1e-8


def test_silu_matches_library_expit():
    from scipy.special import expit
    x = np.linspace(-40, 40, 2001)
    assert np.allclose(oracle.silu(x), x * expit(x), rtol=1e-14, atol=1e-300)


def test_swiglu_pair_hand_case():
    v = np.array([[1.0, 2.0, -1.0, 3.0]])      # columns g0, u0, g1, u1
    e = math.e
    expect = [e / (1 + e) * 2.0, -1.0 / (1 + e) * 3.0]
    assert np.allclose(oracle.swiglu_pair(v)[0], expect, rtol=1e-15)
    with pytest.raises(ValueError):
        oracle.swiglu_pair(np.ones((1, 3)))


def test_reductions_constant_rows():
    c, N = 0.75, 12
    C = np.full((3, N), c)
    _, reds = oracle.apply_epilogue(C, [("row_sum", {}), ("row_sumsq", {}), ("row_mean", {})])
    assert np.allclose(reds[0][2], N * c) and np.allclose(reds[1][2], N * c * c) and np.allclose(reds[2][2], c)


def test_column_reductions_closed_forms_and_axis():
    # a constant M x N matrix: every column sums to M c, its squares to M c^2
    c, M, N = -1.25, 7, 4
    _, reds = oracle.apply_epilogue(np.full((M, N), c), [("col_sum", {}), ("col_sumsq", {})])
    assert reds[0][2].shape == (N,) and np.allclose(reds[0][2], M * c)
    assert np.allclose(reds[1][2], M * c * c)
    # rows 0..M-1 holding i + 10 j: column j sums to M(M-1)/2 + 10 j M (pins the axis)
    V = np.arange(M)[:, None] + 10.0 * np.arange(N)[None, :]
    _, reds = oracle.apply_epilogue(V, [("col_sum", {}), ("row_sum", {})])
    assert np.array_equal(reds[0][2], M * (M - 1) / 2 + 10.0 * np.arange(N) * M)
    # the total is the same whichever way it is reduced
    assert np.isclose(reds[0][2].sum(), reds[1][2].sum())


def test_column_reduction_of_a_backward_layer_is_the_bias_gradient():
    # y = h W2 + b2 upstream of dY: the gradient of a bias b1 added before the
    # activation is sum over tokens of dY W2^T * GELU'(P), the column sum of dH
    rng = np.random.default_rng(12)
    T, H, O = 6, 5, 3
    dY, W2, P = rng.standard_normal((T, O)), rng.standard_normal((H, O)), rng.standard_normal((T, H))
    _, reds = oracle.forward(dY, W2, [("mul_dgelu_tanh", {"mat": P}), ("col_sum", {})], "NK")
    # finite-difference gradient of L(b1) = sum(dY * (gelu_tanh(P + b1) W2)) at b1 = 0
    h = 1e-6
    def L(b1):
        return float(np.sum(dY * (oracle.gelu_tanh(P + b1[None, :]) @ W2)))
    fd = np.array([(L(h * e) - L(-h * e)) / (2 * h) for e in np.eye(H)])
    assert np.allclose(reds[0][2], fd, rtol=1e-6, atol=1e-8)


def test_chained_row_sumsq_is_the_rms_of_the_next_layer():
    # a layer's ROW_SUMSQ output, divided by the width, is the mean square the
    # next layer's RMS normalisation of that output needs (the cross-layer chain)
    rng = np.random.default_rng(15)
    A, B = rng.standard_normal((5, 6)), rng.standard_normal((6, 8))
    D1, reds = oracle.forward(A, B, [("add_col", {"vec": rng.standard_normal(8)}), ("row_sumsq", {})], "KN")
    eps = 1e-6
    assert np.allclose(oracle.rms(D1, eps), np.sqrt(reds[0][2] / D1.shape[1] + eps), rtol=1e-14)


def test_weight_gradient_is_the_transposed_product():
    # y = x W: dL/dW for L = sum(dy * y) is x^T dy; the oracle's GEMM of the
    # transposed storage against finite differences (pins which operand is
    # transposed and that the contraction runs over the tokens)
    rng = np.random.default_rng(14)
    T, Fi, Fo = 7, 4, 3
    x, dy, W = rng.standard_normal((T, Fi)), rng.standard_normal((T, Fo)), rng.standard_normal((Fi, Fo))
    dW, _ = oracle.forward(x.T, dy, [], "KN")
    h = 1e-6
    fd = np.zeros((Fi, Fo))
    for i in range(Fi):
        for j in range(Fo):
            E = np.zeros((Fi, Fo))
            E[i, j] = h
            fd[i, j] = (np.sum(dy * (x @ (W + E))) - np.sum(dy * (x @ (W - E)))) / (2 * h)
    assert np.allclose(dW, fd, rtol=1e-6, atol=1e-8)


def test_planted_column_sum_over_the_wrong_axis_is_caught(monkeypatch):
    real = oracle.apply_epilogue

    def wrong(C, ops):
        v, reds = real(C, ops)
        return v, [(n, a, (np.sum(v, axis=1) if n == "col_sum" else r)) for n, a, r in reds]
    rng = np.random.default_rng(13)
    M, N, K = 3, 6, 5
    A, B = _tiny_case(rng, M, N, K)
    ops = [("col_sum", {})]
    _, bred = brute_force(_lists(A), _lists(B), ops)
    monkeypatch.setattr(oracle, "apply_epilogue", wrong)
    _, reds = oracle.apply_epilogue(oracle.gemm(A, B), ops)
    assert reds[0][2].shape != np.array(bred[0]).shape or not np.allclose(reds[0][2], bred[0])


def test_reduction_sees_value_at_its_position():
    C = np.full((1, 4), 1.0)
    _, reds = oracle.apply_epilogue(C, [("row_sum", {}), ("scale", {"alpha": 3.0}), ("row_sum", {}),
                                        ("swiglu_pair", {}), ("row_mean", {})])
    assert reds[0][2][0] == 4.0 and reds[1][2][0] == 12.0
    assert reds[2][2][0] == pytest.approx(3.0 * (3.0 * e_sig(3.0)))


def e_sig(x):
    return 1.0 / (1.0 + math.exp(-x))


def test_rms_must_come_first():
    X = np.ones((2, 4))
    with pytest.raises(ValueError):
        oracle.forward(X, np.eye(4), [("add_col", {"vec": np.zeros(4)}),
                                      ("rms_rowscale", {"gamma": np.ones(4), "eps": 1e-6})])
    with pytest.raises(ValueError):
        oracle.rms(np.ones((2, 0)), 1e-6)


# ----------------------------------------------------------------------------
# planted mistakes: each one is caught by a pin above's check
# ----------------------------------------------------------------------------

def _plant(monkeypatch, name, replacement):
    """Replace an oracle function in its module and in the package namespace."""
    monkeypatch.setattr(co, name, replacement)
    monkeypatch.setattr(oracle, name, replacement)


def test_planted_wrong_gelu_constant_is_caught(monkeypatch):
    monkeypatch.setattr(co, "GELU_CUBIC", 0.04715)
    with pytest.raises(AssertionError):
        test_gelu_tanh_close_to_erf_gelu()


def test_planted_eps_outside_root_is_caught(monkeypatch):
    def bad_rms(X, eps):
        X = np.asarray(X, dtype=np.float64)
        return np.sqrt(np.sum(X * X, axis=1) / X.shape[1]) + eps
    _plant(monkeypatch, "rms", bad_rms)
    with pytest.raises(AssertionError):
        test_rms_mean_square_invariant_pins_mean_over_k_and_eps_inside_root()


def test_planted_swapped_gate_up_is_caught(monkeypatch):
    def bad_pair(v):
        return co.silu(v[:, 1::2]) * v[:, 0::2]
    _plant(monkeypatch, "swiglu_pair", bad_pair)
    with pytest.raises(AssertionError):
        test_swiglu_pair_hand_case()


def test_planted_transposed_b_is_caught(monkeypatch):
    _plant(monkeypatch, "logical_b", lambda B, lay: np.asarray(B, dtype=np.float64).T if lay == "KN" else np.asarray(B, dtype=np.float64))
    with pytest.raises((AssertionError, ValueError)):
        test_b_layout_nk_is_transposed_storage()


def test_planted_dropped_derivative_term_is_caught(monkeypatch):
    def bad_grad(p):
        p = np.asarray(p, dtype=np.float64)
        t = np.tanh(co.SQRT_2_OVER_PI * (p + co.GELU_CUBIC * p ** 3))
        return 0.5 * (1.0 + t)
    _plant(monkeypatch, "gelu_tanh_grad", bad_grad)
    with pytest.raises(AssertionError):
        test_gelu_grad_matches_central_difference()


def test_planted_uncentred_layernorm_is_caught(monkeypatch):
    def bad_ln(X, gamma, eps, beta=None):      # forgets the centring: an RMSNorm
        Y = co.rmsnorm(X, gamma, eps)
        return Y if beta is None else Y + np.asarray(beta)[None, :]
    _plant(monkeypatch, "layernorm", bad_ln)
    with pytest.raises(AssertionError):
        test_layernorm_moments_pin_centring_biased_variance_and_eps_inside_root()
    with pytest.raises(AssertionError):
        test_hand_worked_layernorm_golden_case()


def test_planted_unbiased_variance_is_caught(monkeypatch):
    def bad_ln(X, gamma, eps, beta=None):      # 1/(K-1) variance
        X = np.asarray(X, dtype=np.float64)
        Xc = X - X.mean(axis=1, keepdims=True)
        var = (Xc * Xc).sum(axis=1) / (X.shape[1] - 1)
        Y = Xc / np.sqrt(var + eps)[:, None] * np.asarray(gamma)[None, :]
        return Y if beta is None else Y + np.asarray(beta)[None, :]
    _plant(monkeypatch, "layernorm", bad_ln)
    with pytest.raises(AssertionError):
        test_hand_worked_layernorm_golden_case()


def test_planted_wrong_sign_of_mean_term_is_caught(monkeypatch):
    def bad_def(X, gamma, beta, B, eps):
        X = np.asarray(X, dtype=np.float64)
        K = X.shape[1]
        mu = X.sum(axis=1) / K
        var = ((X - mu[:, None]) ** 2).sum(axis=1) / K
        u, c = co.ln_fold(B, gamma, beta)
        P = (X * gamma[None, :]) @ B
        return (P + mu[:, None] * u[None, :]) / np.sqrt(var + eps)[:, None] + c[None, :]
    _plant(monkeypatch, "deferred_layernorm_gemm", bad_def)
    with pytest.raises(AssertionError):
        test_deferred_layernorm_equals_normalise_first_at_config_shapes(2)


def _read_golden(path):
    vals, lines = {}, [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    i = 0
    while i < len(lines):
        key = lines[i][0]
        if key in ("A", "B"):
            r, c = int(lines[i][1]), int(lines[i][2])
            vals[key] = np.array([[float(x) for x in lines[i + 1 + k]] for k in range(r)])
            i += 1 + r
        else:
            vals[key] = np.array([float(x) for x in lines[i][1:]])
            i += 1
    return vals


def test_hand_worked_golden_case():
    import os
    g = _read_golden(os.path.join(os.path.dirname(__file__), "golden", "hand_rmsnorm_gemm_epilogue.txt"))
    ops = [("rms_rowscale", {"gamma": g["gamma"], "eps": 0.0}), ("add_col", {"vec": np.array([1.0, 2.0])}),
           ("row_sum", {}), ("scale", {"alpha": 2.0}), ("row_sumsq", {})]
    D, reds = oracle.forward(g["A"], g["B"], ops, "KN")
    assert np.allclose(D[0], g["D0"], rtol=1e-14) and np.allclose(D[1], g["D1"], rtol=1e-14)
    assert np.allclose(reds[0][2], g["sum"], rtol=1e-14) and np.allclose(reds[1][2], g["sumsq"], rtol=1e-14)


# ----------------------------------------------------------------------------
# the seeded-workload driver: every workload's symbolic program resolves to
# arrays (tensor names) and numbers (scalars) and agrees with the brute force,
# on all rows and on a row subset
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("idx", sorted(w.CONFIGS))
def test_run_workload_matches_brute_force_on_every_program(idx):
    from oracle.run import resolve_program
    from workloads.gen import to_f64
    M, N, K = 5, 8, 6
    spec = w.scaled_config(idx, M, N, K)
    inputs = w.make_inputs(spec)
    dtypes = {t.name: t.dtype for t in spec.tensors}
    A = to_f64(inputs[spec.a_name], dtypes[spec.a_name])
    B = oracle.logical_b(to_f64(inputs[spec.b_name], dtypes[spec.b_name]), spec.b_layout)
    ops = resolve_program(spec, inputs)
    for name, args in ops:
        for key, val in args.items():
            assert key == "out" or not isinstance(val, str), (name, key)
    bf_ops = [(n, {k: (_lists(v) if isinstance(v, np.ndarray) and v.ndim == 2 else
                       (list(map(float, v)) if isinstance(v, np.ndarray) else v)) for k, v in a.items()})
              for n, a in ops]
    V, _ = brute_force(_lists(A), _lists(B), bf_ops)
    D, outs = oracle.run_workload(spec, inputs)
    tol = 1e-8 if idx == 5 else 1e-12
    assert np.allclose(D, np.array(V), rtol=tol, atol=tol)
    rows = [4, 0, 2]
    D_sub, outs_sub = oracle.run_workload(spec, inputs, rows)
    assert np.array_equal(D_sub, D[rows])
    for name in outs:
        assert np.array_equal(outs_sub[name], outs[name][rows])
        assert np.all(np.isfinite(outs[name]))


# --- RMSNorm backward (gradients among d9bl.com Fig. 4's operators; agentlenshq.com "How it works") ---

def _rms_bwd_fd_error(bwd, seed=21, T=5, K=6, eps=1e-2):
    """Largest relative error of ``bwd``'s (dX, dgamma) against central
    differences of L = sum(dY * rmsnorm(X, gamma, eps))."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, K)) * np.array([0.05, 0.3, 1.0, 3.0, 10.0])[:T, None]
    g = 1 + 0.3 * rng.standard_normal(K)
    dY = rng.standard_normal((T, K))
    dX, dg = bwd(X, g, eps, dY)
    h = 1e-6

    def L(Xp, gp):
        return float(np.sum(dY * oracle.rmsnorm(Xp, gp, eps)))
    fdX = np.zeros((T, K))
    for i in range(T):
        for k in range(K):
            E = np.zeros((T, K))
            E[i, k] = h * max(1.0, abs(X[i, k]))
            fdX[i, k] = (L(X + E, g) - L(X - E, g)) / (2 * E[i, k])
    fdg = np.array([(L(X, g + h * e) - L(X, g - h * e)) / (2 * h) for e in np.eye(K)])
    scale = max(np.abs(fdX).max(), np.abs(fdg).max())
    return max(np.abs(dX - fdX).max(), np.abs(dg - fdg).max()) / scale


def test_rmsnorm_backward_matches_finite_differences():
    assert _rms_bwd_fd_error(oracle.rmsnorm_backward) < 1e-6


def test_rmsnorm_backward_closed_forms():
    rng = np.random.default_rng(22)
    T, K = 9, 40
    X = rng.standard_normal((T, K)) * rng.uniform(0.1, 5.0, (T, 1))
    g = 1 + 0.2 * rng.standard_normal(K)
    dY = rng.standard_normal((T, K))
    eps = 1e-3
    dX, _ = oracle.rmsnorm_backward(X, g, eps, dY)
    r = oracle.rms(X, eps)
    s = np.sum(dY * g * X, axis=1)
    # x . dx = eps s / r^3: zero without eps, where the norm is scale invariant
    assert np.allclose(np.sum(X * dX, axis=1), eps * s / r ** 3, rtol=1e-10, atol=1e-13)
    dX0, _ = oracle.rmsnorm_backward(X, g, 0.0, dY)
    assert np.allclose(np.sum(X * dX0, axis=1), 0.0, atol=1e-12 * np.abs(dX0).max() * np.abs(X).max() * K)
    # without eps the norm is homogeneous of degree 0: dX(cX) = dX(X) / c
    dXc, dgc = oracle.rmsnorm_backward(3.5 * X, g, 0.0, dY)
    assert np.allclose(dXc, dX0 / 3.5, rtol=1e-12, atol=1e-15)
    assert np.allclose(dgc, oracle.rmsnorm_backward(X, g, 0.0, dY)[1], rtol=1e-12)
    # one feature without eps: y = sign(x) gamma, constant in x
    dX1, dg1 = oracle.rmsnorm_backward(np.array([[2.0], [-0.5]]), np.array([1.7]), 0.0, np.array([[0.3], [-2.0]]))
    assert np.allclose(dX1, 0.0, atol=1e-15)
    assert np.allclose(dg1, [0.3 * 1.0 + (-2.0) * (-1.0)])


def test_rmsnorm_backward_row_dot_through_the_projection():
    # With Y = rmsnorm(X) feeding P = Y W and dY = dP W^T, the row dot product
    # s_i = sum_j gamma_j dY_ij X_ij equals r_i * sum_l dP_il P_il: the term of
    # the norm's gradient that spans the whole row can be gathered from the
    # projection's output side, where each row is one tile row of the GEMM.
    rng = np.random.default_rng(23)
    T, K, Nn = 6, 10, 7
    X, W = rng.standard_normal((T, K)), rng.standard_normal((K, Nn))
    g, dP, eps = 1 + 0.1 * rng.standard_normal(K), rng.standard_normal((T, Nn)), 1e-5
    P = oracle.rmsnorm(X, g, eps) @ W
    dY = dP @ W.T
    s = np.sum(g * dY * X, axis=1)
    assert np.allclose(s, oracle.rms(X, eps) * np.sum(dP * P, axis=1), rtol=1e-12)


def test_planted_rmsnorm_backward_mistakes_are_caught():
    def dropped_term(X, g, eps, dY):
        dX, dg = oracle.rmsnorm_backward(X, g, eps, dY)
        r = oracle.rms(X, eps)
        return dY * g / r[:, None], dg

    def unbiased_mean(X, g, eps, dY):
        dX, dg = oracle.rmsnorm_backward(X, g, eps, dY)
        K = X.shape[1]
        r = oracle.rms(X, eps)
        s = np.sum(dY * g * X, axis=1)
        return dX + X * (s / (K * r ** 3) - s / ((K - 1) * r ** 3))[:, None], dg

    def r_squared(X, g, eps, dY):
        dX, dg = oracle.rmsnorm_backward(X, g, eps, dY)
        K = X.shape[1]
        r = oracle.rms(X, eps)
        s = np.sum(dY * g * X, axis=1)
        return dX + X * (s / (K * r ** 3) - s / (K * r ** 2))[:, None], dg

    def gain_gradient_without_norm(X, g, eps, dY):
        dX, _ = oracle.rmsnorm_backward(X, g, eps, dY)
        return dX, np.sum(dY * X, axis=0)
    for planted in (dropped_term, unbiased_mean, r_squared, gain_gradient_without_norm):
        assert _rms_bwd_fd_error(planted) > 1e-3, planted.__name__


def test_rms_bwd_epilogue_is_the_gradient_through_the_projection():
    # D = rms_bwd(dP W^T) is dL/dX for L = sum(dP * (rmsnorm(X) W)): central
    # differences through the whole forward, W stored [N x K] as the backward
    # GEMM reads it
    rng = np.random.default_rng(24)
    T, K, Nn, eps = 4, 6, 5, 1e-3
    X = rng.standard_normal((T, K)) * np.array([0.2, 1.0, 4.0, 0.05])[:, None]
    W, g, dP = rng.standard_normal((K, Nn)), 1 + 0.3 * rng.standard_normal(K), rng.standard_normal((T, Nn))
    D, _ = oracle.forward(dP, W, [("rms_bwd", {"x": X, "gamma": g, "eps": eps})], "NK")
    h = 1e-6

    def L(Xp):
        return float(np.sum(dP * (oracle.rmsnorm(Xp, g, eps) @ W)))
    fd = np.zeros((T, K))
    for i in range(T):
        for k in range(K):
            E = np.zeros((T, K))
            E[i, k] = h * max(1.0, abs(X[i, k]))
            fd[i, k] = (L(X + E) - L(X - E)) / (2 * E[i, k])
    assert np.allclose(D, fd, rtol=1e-6, atol=1e-7 * np.abs(fd).max())


def test_row_dot_brute_force():
    rng = np.random.default_rng(25)
    M, N, K = 3, 5, 4
    A, B, Mat = rng.integers(-3, 4, (M, K)), rng.integers(-3, 4, (K, N)), rng.integers(-3, 4, (M, N))
    _, reds = oracle.forward(A, B, [("add_col", {"vec": np.arange(N)}), ("row_dot", {"mat": Mat})], "KN")
    want = []
    for i in range(M):
        t = 0
        for j in range(N):
            c = sum(int(A[i, k]) * int(B[k, j]) for k in range(K)) + j
            t += c * int(Mat[i, j])
        want.append(t)
    assert np.array_equal(reds[0][2], np.array(want, dtype=np.float64))


def test_rms_dgamma_is_the_gain_gradient_through_the_projection():
    # the rms_dgamma column reduction of dP W^T is dL/dgamma for
    # L = sum(dP * (rmsnorm(X, gamma) W)), by central differences in gamma
    rng = np.random.default_rng(26)
    T, K, Nn, eps = 5, 6, 4, 1e-3
    X = rng.standard_normal((T, K)) * np.array([0.2, 1.0, 4.0, 0.05, 2.0])[:, None]
    W, g, dP = rng.standard_normal((K, Nn)), 1 + 0.3 * rng.standard_normal(K), rng.standard_normal((T, Nn))
    _, reds = oracle.forward(dP, W, [("rms_dgamma", {"x": X, "eps": eps}), ("rms_bwd", {"x": X, "gamma": g, "eps": eps})],
                             "NK")
    h = 1e-6

    def L(gp):
        return float(np.sum(dP * (oracle.rmsnorm(X, gp, eps) @ W)))
    fd = np.array([(L(g + h * e) - L(g - h * e)) / (2 * h) for e in np.eye(K)])
    assert np.allclose(reds[0][2], fd, rtol=1e-6, atol=1e-8)
