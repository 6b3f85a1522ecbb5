"""Edge cases and per-op coverage on the GPU, through the C ABI."""
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


def run(CR, A, B, ops, b_layout, mode="fused", tile=0, D=None, d_dtype=None):
    coda, runner = CR
    call = runner.Call(A, B, ops, b_layout, D=D, d_dtype=d_dtype, tile=tile)
    st = call.fused() if mode == "fused" else call.unfused()
    coda.check(st, "call")
    torch.cuda.synchronize()
    return call


def oracle_ops(ops):
    """Device-tensor op args -> fp64 numpy args for the oracle."""
    out = []
    for name, a in ops:
        r = {}
        for k, v in a.items():
            if isinstance(v, torch.Tensor) and k != "out":
                r[k] = f64(v)
            elif k != "out":
                r[k] = v
        out.append((name, r))
    return out


def test_empty_problems_are_noops(CR):
    coda, runner = CR
    announce("empty problems")
    A = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda")
    call = runner.Call(A, B, [("gelu_tanh", {})], "KN")
    assert call.fused() == coda.CODA_OK and call.unfused() == coda.CODA_OK
    A = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((64, 0), dtype=torch.bfloat16, device="cuda")
    D = torch.full((16, 8), 7.0, dtype=torch.bfloat16, device="cuda")
    call = runner.Call(A, B, [], "KN", D=D, N=0)
    assert call.fused() == coda.CODA_OK
    torch.cuda.synchronize()
    assert torch.all(D == 7.0)


@pytest.mark.parametrize("mode", ["fused", "unfused"])
def test_k_zero_gives_epilogue_of_zero(CR, mode):
    announce(f"K=0 {mode}")
    rng = np.random.default_rng(3)
    M, N = 40, 72
    A = torch.zeros((M, 8), dtype=torch.bfloat16, device="cuda")[:, :0]
    B = torch.zeros((0, N), dtype=torch.bfloat16, device="cuda")
    bias = bf16(rng.standard_normal(N))
    ops = [("add_col", {"vec": bias}), ("gelu_tanh", {})]
    coda, runner = CR
    D = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    call = runner.Call(A, B, ops, "KN", D=D, M=M, N=N, K=0, lda=8, ldb=N)
    st = call.fused() if mode == "fused" else call.unfused()
    coda.check(st, "K=0")
    torch.cuda.synchronize()
    ref = oracle.gelu_tanh(np.broadcast_to(f64(bias), (M, N)))
    assert_close(f64(D), ref, f"K=0/{mode}")


@pytest.mark.parametrize("shape", [(1, 8, 8), (33, 24, 8), (257, 264, 72)])
@pytest.mark.parametrize("layout", ["KN", "NK"])
def test_tiny_and_ragged_plain_gemm(CR, shape, layout):
    M, N, K = shape
    announce(f"plain gemm {shape} {layout}")
    rng = np.random.default_rng(M * 7 + N)
    a = rng.standard_normal((M, K))
    b = rng.standard_normal((K, N)) / np.sqrt(K)
    A = bf16(a)
    B = bf16(b if layout == "KN" else np.ascontiguousarray(b.T))
    for tile in (1, 2):
        call = run(CR, A, B, [], layout, tile=tile)
        ref, _ = oracle.forward(f64(A), f64(B), [], layout)
        assert_close(f64(call.D), ref, f"plain {shape} {layout} tile{tile}")


def test_b_nk_ragged_n_not_multiple_of_8(CR):
    announce("B_NK ragged N=27*2")
    rng = np.random.default_rng(9)
    M, N, K = 70, 54, 40
    A = bf16(rng.standard_normal((M, K)))
    B = bf16(rng.standard_normal((N, K)) / np.sqrt(K))
    coda, runner = CR
    D = torch.empty((M, 32), dtype=torch.bfloat16, device="cuda")[:, :27]
    stats = torch.zeros((M, 1), dtype=torch.float32, device="cuda")
    ops = [("swiglu_pair", {}), ("row_sum", {"out": stats, "col": 0})]
    call = runner.Call(A, B, ops, "NK", D=D)
    coda.check(call.fused(), "fused")
    torch.cuda.synchronize()
    ref, reds = oracle.forward(f64(A), f64(B), [("swiglu_pair", {}), ("row_sum", {})], "NK")
    assert_close(f64(D), ref, "NK ragged swiglu D")
    assert_close(f64(stats)[:, 0], reds[0][2], "NK ragged swiglu rowsum")


def every_op_program(M, N, K, rng, use_rms=True):
    """A list that uses every primitive once, with mixed side-operand dtypes."""
    def f32(x):
        return torch.from_numpy(np.asarray(x, dtype=np.float32)).cuda()
    outs = torch.zeros((M, 4), dtype=torch.float32, device="cuda")
    ops = []
    if use_rms:
        ops.append(("rms_rowscale", {"gamma": bf16(1 + 0.1 * rng.standard_normal(K)), "eps": 1e-5}))
    ops += [
        ("scale", {"alpha": 1.5}),
        ("scale_row", {"vec": f32(1 + 0.2 * rng.standard_normal(M))}),
        ("scale_col", {"vec": bf16(1 + 0.2 * rng.standard_normal(N))}),
        ("add_row", {"vec": bf16(0.3 * rng.standard_normal(M))}),
        ("add_col", {"vec": f32(0.3 * rng.standard_normal(N))}),
        ("add_mat", {"mat": bf16(rng.standard_normal((M, N))), "beta": -0.5}),
        ("silu", {}),
        ("row_mean", {"out": outs, "col": 0}),
        ("gelu_tanh", {}),
        ("mul_dgelu_tanh", {"mat": f32(rng.standard_normal((M, N)))}),
        ("row_sumsq", {"out": outs, "col": 1}),
        ("swiglu_pair", {}),
        ("add_col", {"vec": bf16(0.1 * rng.standard_normal(N // 2))}),
        ("row_sum", {"out": outs, "col": 2}),
        ("scale", {"alpha": 2.0}),
        ("row_mean", {"out": outs, "col": 3}),
    ]
    if use_rms:   # 16 ops at most: drop the first scale to make room for the RMS op
        ops = [op for i, op in enumerate(ops) if i != 1]
    return ops, outs


@pytest.mark.parametrize("layout", ["KN", "NK"])
@pytest.mark.parametrize("tile", [0, 1, 2, 3])
def test_every_op_fused(CR, layout, tile):
    announce(f"every op fused {layout} tile{tile}")
    rng = np.random.default_rng(21)
    M, N, K = 200, 328, 96
    a = rng.standard_normal((M, K))
    b = rng.standard_normal((K, N)) / np.sqrt(K)
    A = bf16(a)
    B = bf16(b if layout == "KN" else np.ascontiguousarray(b.T))
    ops, outs = every_op_program(M, N, K, rng)
    call = run(CR, A, B, ops, layout, tile=tile)
    ref, reds = oracle.forward(f64(A), f64(B), oracle_ops(ops), layout)
    assert_close(f64(call.D), ref, "every-op D")
    for i, (_, _, r) in enumerate(reds):
        assert_close(f64(outs)[:, i], r, f"every-op reduction {i}")


@pytest.mark.parametrize("layout", ["KN", "NK"])
@pytest.mark.parametrize("tile", [1, 2, 3])
def test_every_op_no_norm(CR, layout, tile):
    # without a row norm the list runs in the kernels that read the first bf16
    # side matrix ahead (here ADD_MAT), while the fp32 one (MUL_DGELU_TANH) is
    # read where it is used
    announce(f"every op, no row norm, {layout} tile{tile}")
    rng = np.random.default_rng(23)
    M, N, K = 300, 264, 136
    a = rng.standard_normal((M, K))
    b = rng.standard_normal((K, N)) / np.sqrt(K)
    A = bf16(a)
    B = bf16(b if layout == "KN" else np.ascontiguousarray(b.T))
    ops, outs = every_op_program(M, N, K, rng, use_rms=False)
    call = run(CR, A, B, ops, layout, tile=tile)
    ref, reds = oracle.forward(f64(A), f64(B), oracle_ops(ops), layout)
    assert_close(f64(call.D), ref, "every-op (no norm) D")
    for i, (_, _, r) in enumerate(reds):
        assert_close(f64(outs)[:, i], r, f"every-op (no norm) reduction {i}")


@pytest.mark.parametrize("layout", ["KN", "NK"])
def test_every_op_f32_operands(CR, layout):
    announce(f"every op f32 operands {layout}")
    rng = np.random.default_rng(22)
    M, N, K = 100, 200, 64
    a = rng.standard_normal((M, K))
    b = rng.standard_normal((K, N)) / np.sqrt(K)
    A = torch.from_numpy(a.astype(np.float32)).cuda()
    Bm = b if layout == "KN" else np.ascontiguousarray(b.T)
    B = torch.from_numpy(Bm.astype(np.float32)).cuda()
    ops, outs = every_op_program(M, N, K, rng, use_rms=False)
    ops = ops[1:]
    ops = [("rms_rowscale", {"gamma": torch.from_numpy((1 + 0.1 * rng.standard_normal(K)).astype(np.float32)).cuda(),
                             "eps": 1e-6})] + ops
    call = run(CR, A, B, ops, layout, d_dtype=torch.float32)
    ref, reds = oracle.forward(f64(A), f64(B), oracle_ops(ops), layout)
    assert_close(f64(call.D), ref, "f32 every-op D")
    for i, (_, _, r) in enumerate(reds):
        assert_close(f64(outs)[:, i], r, f"f32 every-op reduction {i}")


def test_in_place_residual(CR):
    announce("in-place residual D == R")
    rng = np.random.default_rng(31)
    M, N, K = 130, 264, 72
    A = bf16(rng.standard_normal((M, K)))
    B = bf16(rng.standard_normal((K, N)) / np.sqrt(K))
    R = bf16(rng.standard_normal((M, N)))
    R0 = f64(R)
    ops = [("add_mat", {"mat": R, "beta": 1.0})]
    run(CR, A, B, ops, "KN", D=R)
    ref, _ = oracle.forward(f64(A), f64(B), [("add_mat", {"mat": R0, "beta": 1.0})], "KN")
    assert_close(f64(R), ref, "in-place residual")


def test_rms_degenerate_rows(CR):
    """Zero rows give 0 (x / sqrt(eps) with x = 0); constant rows give c / sqrt(c^2 + eps) per unit feature."""
    announce("rms degenerate rows")
    M, K, N = 64, 64, 64
    x = np.zeros((M, K))
    x[1] = 3.0
    x[2] = -0.5
    x[3:] = np.random.default_rng(4).standard_normal((M - 3, K))
    A = bf16(x)
    B = bf16(np.eye(K))
    g = bf16(np.ones(K))
    ops = [("rms_rowscale", {"gamma": g, "eps": 1e-6})]
    for mode in ("fused", "unfused"):
        call = run(CR, A, B, ops, "KN", mode=mode)
        ref, _ = oracle.forward(f64(A), f64(B), [("rms_rowscale", {"gamma": f64(g), "eps": 1e-6})], "KN")
        got = f64(call.D)
        assert np.all(got[0] == 0.0)
        assert_close(got, ref, f"rms degenerate {mode}")


def test_workspace_counters_left_zero(CR):
    announce("workspace counters reset")
    coda, runner = CR
    spec = w.scaled_config(3, 512, 1024, 64)
    inputs = w.make_inputs(spec)
    call = runner.WorkloadCall(spec, inputs, tile=2)
    assert call.ws[0] is not None
    for _ in range(3):
        coda.check(call.fused(), "fused")
    torch.cuda.synchronize()
    M = spec.M
    gn = (spec.N + 127) // 128
    red_bytes = 2 * gn * M * 4
    off = (red_bytes + 255) // 256 * 256
    counters = call.ws[0][off:off + 4 * ((M + 127) // 128)]
    assert int(counters.sum()) == 0
