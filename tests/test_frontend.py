"""The text front end (host only): programs of statements on the running value
lower to the op lists the workloads describe, resolve operands by shape, and
reject what is not a primitive."""
import numpy as np
import pytest

import oracle
import workloads as w
from gemm_epilogue_transformer_bf16_amd.frontend import FrontendError, lower, parse


def operands(M, N, K):
    rng = np.random.default_rng(3)
    return {"gamma": np.ones(K), "beta": np.zeros(K), "bias": rng.standard_normal(N), "R": rng.standard_normal((M, N)),
            "P": rng.standard_normal((M, N)), "rs": rng.standard_normal(M), "stats": np.zeros((M, 2)),
            "db": np.zeros((N, 1)), "half_bias": rng.standard_normal(N // 2)}


def test_the_pages_statement_style_lowers_in_order():
    M, N, K = 6, 8, 4
    ops = lower("""EPILOGUE {
        output = gelu(input);      // the activation of the GEMM result
        output = output + R;       // a residual matrix
      }""", operands(M, N, K), M, N)
    assert [n for n, _ in ops] == ["gelu_tanh", "add_mat"]
    assert ops[1][1]["beta"] == 1.0


@pytest.mark.parametrize("idx,text", [
    (1, "output = rmsnorm(input, gamma, 1e-6); output = output + bias; output = gelu(output); output = output + R;"),
    (3, "output = output + bias; output = output + R; stats[0] = rowsum(output); stats[1] = rowsumsq(output);"),
    (4, "output = rmsnorm(input, gamma, 1e-6); output = swiglu(output);"),
    (5, "output = output * dgelu(P); rowsum_out[0] = rowsum(output);"),
    (6, "output = layernorm(input, gamma, beta, 1e-5); output = output + bias; output = gelu(output);"),
])
def test_lowering_reproduces_the_workload_programs(idx, text):
    """The lowered list computes what the workload's program computes (the
    oracle on both, bit for bit)."""
    M, N, K = 8, 16, 8
    spec = w.scaled_config(idx, M, N, K)
    inputs = w.make_inputs(spec)
    from oracle.run import resolve_program
    from workloads.gen import to_f64
    ref_ops = resolve_program(spec, inputs)
    named = {}
    for name, args in ref_ops:
        for key in ("gamma", "beta", "vec", "mat"):
            if isinstance(args.get(key), np.ndarray):
                named[{"vec": "bias", "mat": "R" if name == "add_mat" else "P"}.get(key, key)] = args[key]
    outs = {o: np.zeros(shape) for o, shape in spec.outputs}
    named.update(outs)
    named["rowsum_out"] = outs.get("rowsum", np.zeros((M, 1)))
    ops = lower(text, named, spec.M, spec.N)
    dtypes = {t.name: t.dtype for t in spec.tensors}
    A = to_f64(inputs[spec.a_name], dtypes[spec.a_name])
    B = to_f64(inputs[spec.b_name], dtypes[spec.b_name])
    strip = lambda o: [(n, {k: v for k, v in a.items() if k not in ("out", "col")}) for n, a in o]
    D1, r1 = oracle.forward(A, B, strip(ref_ops), spec.b_layout)
    D2, r2 = oracle.forward(A, B, strip(ops), spec.b_layout)
    assert [n for n, _ in ops] == [n for n, _ in ref_ops]
    assert np.array_equal(D1, D2)
    for (_, _, a), (_, _, b) in zip(r1, r2):
        assert np.array_equal(a, b)


def test_operands_resolve_by_shape():
    M, N, K = 6, 8, 4
    o = operands(M, N, K)
    ops = lower("""output = output * bias; output = output * rs; output = output + rs; output = 2.5 * output;
                   output = output + 0.5 * R; output = swiglu(output); output = output + half_bias;
                   db[0] = colsum(output); stats[1] = rowmean(output);""", o, M, N)
    assert [n for n, _ in ops] == ["scale_col", "scale_row", "add_row", "scale", "add_mat", "swiglu_pair",
                                   "add_col", "col_sum", "row_mean"]
    assert ops[3][1]["alpha"] == 2.5 and ops[4][1]["beta"] == 0.5
    assert ops[7][1]["col"] == 0 and ops[8][1]["col"] == 1


@pytest.mark.parametrize("text,msg", [
    ("output = dropout(output, 1.0);", "dropout probability"),
    ("output = dropout(output, p);", "dropout probability must be a number"),
    ("output = dropout(output, 0.1, s);", "seed"),
    ("output = output + bias; output = gelu(input);", "first statement"),
    ("output = silu(output); output = swiglu(input);", "first statement"),
    ("output = gelu(output); output = rmsnorm(input, gamma, 1e-6);", "first statement"),
    ("output = output + nothing;", "unbound"),
    ("output = output + 1.0;", "constant"),
    ("output = output * R;", "not a primitive"),
    ("stats[0] = gelu(output);", "reduction"),
    ("output = gelu(output)", "';'"),
    ("output = tanh(output);", "expected"),
    ("stats[1] = rowdot(output);", "1 more argument"),
    ("stats[0] = rowsum(output, P);", "only the running value"),
    ("db[0] = rmsdgamma(output, P, stats, eps);", "eps must be a number"),
    ("output = rmsnorm_backward(output, P, gamma, stats, P);", "eps must be a number"),
])
def test_errors(text, msg):
    M, N, K = 6, 8, 4
    with pytest.raises(FrontendError, match=msg):
        lower(text, operands(M, N, K), M, N)


def test_parse_is_pure_syntax():
    assert parse("EPILOGUE { output = silu(input); }") == [("func", "silu")]
    assert parse("") == []


def test_rms_backward_statements_lower_to_the_norms_gradients():
    # the lowered program, run by the oracle on dP W^T, gives dL/dx and
    # dL/dgamma of the RMS norm (rmsnorm_backward), and rowdot gives t
    rng = np.random.default_rng(4)
    M, F, Np, eps = 5, 8, 6, 1e-3
    x, g = rng.standard_normal((M, F)), 1 + 0.1 * rng.standard_normal(F)
    W, dP = rng.standard_normal((F, Np)), rng.standard_normal((M, Np))
    ops_in = {"x": x, "g": g, "st": np.zeros((M, 2)), "dg": np.zeros((F, 1))}
    text = """EPILOGUE {
        dg[0] = rmsdgamma(output, x, st, 1e-3);   // the gain gradient first: it reads dL/dY
        output = rmsnorm_backward(output, x, g, st, 1e-3);
    }"""
    ops = lower(text, ops_in, M, F)
    assert [n for n, _ in ops] == ["rms_dgamma", "rms_bwd"]
    assert ops[1][1]["sumsq_col"] == 0 and ops[1][1]["t_col"] == 1 and ops[0][1]["col"] == 0
    D, reds = oracle.forward(dP, W, ops, "NK")
    dX, dg = oracle.rmsnorm_backward(x, g, eps, dP @ W.T)
    assert np.allclose(D, dX, rtol=1e-12, atol=1e-12)
    assert np.allclose(reds[0][2], dg, rtol=1e-12, atol=1e-12)
    P = oracle.rmsnorm(x, g, eps) @ W
    up = lower("st[1] = rowdot(output, P);", {"st": np.zeros((M, 2)), "P": P}, M, Np)
    assert up[0][0] == "row_dot" and up[0][1]["col"] == 1
    _, reds = oracle.forward(dP, np.eye(Np), up, "KN")
    assert np.allclose(reds[0][2] * oracle.rms(x, eps), np.sum(g * (dP @ W.T) * x, axis=1), rtol=1e-10)


def test_input_only_in_the_first_statement():
    M, N, K = 6, 8, 4
    assert [n for n, _ in lower("output = gelu(input); output = output + R;", operands(M, N, K), M, N)] == \
        ["gelu_tanh", "add_mat"]


def test_square_output_needs_explicit_vector_orientation():
    # with M == width, a vector of that length could be a row vector or a column vector
    M = N = 8
    o = {"v": np.arange(8.0), "R": np.zeros((8, 8))}
    with pytest.raises(FrontendError, match="row\\(v\\) or col\\(v\\)"):
        lower("output = output + v;", o, M, N)
    with pytest.raises(FrontendError, match="row\\(v\\) or col\\(v\\)"):
        lower("output = output * v;", o, M, N)
    ops = lower("output = output + col(v); output = output * row(v); output = output + row(v); "
                "output = output * col(v);", o, M, N)
    assert [n for n, _ in ops] == ["add_col", "scale_row", "add_row", "scale_col"]
    # the oracle sees the intended orientation
    C = np.arange(64.0).reshape(8, 8)
    D, _ = oracle.apply_epilogue(C, ops[:1])
    assert np.array_equal(D, C + np.arange(8.0)[None, :])
    D, _ = oracle.apply_epilogue(C, ops[1:2])
    assert np.array_equal(D, C * np.arange(8.0)[:, None])
    with pytest.raises(FrontendError, match="length 6"):
        lower("output = output + row(v);", o, 6, 8)


def test_dropout_statement_lowers_with_seed():
    M, N, K = 6, 8, 4
    ops = lower("output = gelu(input); output = dropout(output, 0.1); output = dropout(output, 0.25, 7);",
                operands(M, N, K), M, N, seed=42)
    assert ops[1] == ("dropout", {"p": 0.1, "seed": 42})
    assert ops[2] == ("dropout", {"p": 0.25, "seed": 7})
    # the oracle runs the lowered program: the mask of the seeded generator
    rng = np.random.default_rng(0)
    A, B = rng.standard_normal((M, K)), rng.standard_normal((K, N))
    D, _ = oracle.forward(A, B, ops[:2])
    keep = oracle.dropout_keep(np.arange(M), N, 0.1, 42)
    ref = np.where(keep, oracle.gelu_tanh(A @ B) / (1 - float(np.float32(0.1))), 0.0)
    assert np.allclose(D, ref, rtol=1e-14, atol=0)
