"""coda_gemm_epi_noalloc (the entry point for callers that cannot allocate)
through the C ABI against coda_gemm_epi on the same inputs: two calls in a
row, the second smaller, covering cross-tile row reductions (partials and
counters in the fixed scratch), column reductions and the split last round,
and the rejection of a call whose scratch need exceeds the fixed maximum."""
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


def layer(rng, M, N, K):
    """A bf16 layer with a bias, a residual, a GELU and row and column sums."""
    A, B = bf16(rng.standard_normal((M, K))), bf16(rng.standard_normal((K, N)) / np.sqrt(K))
    bias, R = bf16(0.1 * rng.standard_normal(N)), bf16(rng.standard_normal((M, N)))
    return A, B, bias, R


def ops_for(bias, R, M, N):
    stats = torch.zeros((M, 2), dtype=torch.float32, device="cuda")
    cols = torch.zeros((N, 1), dtype=torch.float32, device="cuda")
    ops = [("add_col", {"vec": bias}), ("add_mat", {"mat": R}), ("gelu_tanh", {}),
           ("row_sum", {"out": stats, "col": 0}), ("row_sumsq", {"out": stats, "col": 1}),
           ("col_sum", {"out": cols, "col": 0})]
    return ops, stats, cols


def run_both(CR, A, B, ops_a, ops_b, layout="KN"):
    coda, runner = CR
    ref = runner.Call(A, B, ops_a, layout)
    coda.check(ref.fused(), "coda_gemm_epi")
    na = runner.Call(A, B, ops_b, layout)
    d = na.desc
    d.workspace, d.workspace_bytes = None, 0     # ignored by the no-allocation entry point
    st = coda.coda_gemm_epi_noalloc(A.data_ptr(), B.data_ptr(), na.M, na.N, na.K, d,
                                    int(torch.cuda.current_stream().cuda_stream))
    coda.check(st, "coda_gemm_epi_noalloc")
    torch.cuda.synchronize()
    return ref, na


@pytest.mark.parametrize("shapes", [((2944, 2944, 2048), (600, 1040, 256)),      # split round, then no split
                                    ((8192, 1024, 4096), (257, 520, 128))])     # BERT-large shape, then ragged
def test_noalloc_matches_coda_gemm_epi(CR, shapes):
    for n, (M, N, K) in enumerate(shapes):
        announce(f"noalloc call {n} {M}x{N}x{K}")
        rng = np.random.default_rng(7 + n)
        A, B, bias, R = layer(rng, M, N, K)
        ops_a, st_a, col_a = ops_for(bias, R, M, N)
        ops_b, st_b, col_b = ops_for(bias, R, M, N)
        ref, na = run_both(CR, A, B, ops_a, ops_b)
        # the oracle decides both: the bar of the fused path
        D_ref, reds = oracle.forward(f64(A), f64(B), [("add_col", {"vec": f64(bias)}), ("add_mat", {"mat": f64(R)}),
                                                      ("gelu_tanh", {}), ("row_sum", {}), ("row_sumsq", {}),
                                                      ("col_sum", {})], "KN")
        for what, got in (("noalloc", na), ("coda_gemm_epi", ref)):
            assert_close(f64(got.D), D_ref, f"{what} D {M}x{N}x{K}")
        for what, st, cl in (("noalloc", st_b, col_b), ("coda_gemm_epi", st_a, col_a)):
            assert_close(f64(st)[:, 0], reds[0][2], f"{what} row sum")
            assert_close(f64(st)[:, 1], reds[1][2], f"{what} row sumsq")
            assert_close(f64(cl)[:, 0], reds[2][2], f"{what} col sum")
        # the same split (it fits the scratch here), so the same bits
        assert torch.equal(na.D.view(torch.int16), ref.D.view(torch.int16))
        assert torch.equal(st_a, st_b) and torch.equal(col_a, col_b)
        del ref, na


def test_noalloc_caps_the_split(CR):
    """16 x 20 = 320 tiles of 256 x 256: the last round's 64 tiles would be
    split in 4 parts over K = 4096, 64 MiB of partial tiles, above the fixed
    scratch: the entry point splits them into fewer parts instead."""
    coda, runner = CR
    M, N, K = 4096, 5120, 4096
    announce(f"noalloc capped split {M}x{N}x{K}")
    rng = np.random.default_rng(3)
    A = bf16(rng.standard_normal((M, K)))
    B = bf16(rng.standard_normal((K, N)) / np.sqrt(K))
    call = runner.Call(A, B, [("swiglu_pair", {})], "KN")
    assert coda.coda_workspace_size(M, N, K, call.desc, 0) > coda.CODA_NOALLOC_SCRATCH_BYTES
    coda.check(call.fused(), "coda_gemm_epi")
    ref = call.D.clone()
    call.desc.workspace, call.desc.workspace_bytes = None, 0
    st = coda.coda_gemm_epi_noalloc(A.data_ptr(), B.data_ptr(), M, N, K, call.desc,
                                    int(torch.cuda.current_stream().cuda_stream))
    coda.check(st, "noalloc")
    torch.cuda.synchronize()
    rows = np.arange(0, M, 37)
    D_ref, _ = oracle.forward(f64(A[rows]), f64(B), [("swiglu_pair", {})], "KN")
    assert_close(f64(call.D[rows]), D_ref, "noalloc capped split D")
    assert_close(f64(ref[rows]), D_ref, "coda_gemm_epi D")


def test_noalloc_rejects_scratch_beyond_the_maximum(CR):
    coda, runner = CR
    # row reductions over 2 tile columns of 2^23 rows x 8 reductions: 2^23 x 2 x 8 x 4 bytes = 512 MiB
    M, N, K = 1 << 23, 512, 8
    announce("noalloc scratch above maximum (host-side rejection)")
    d = coda.coda_epi_desc()
    d.ab_dtype = d.d_dtype = coda.CODA_BF16
    d.lda, d.ldb, d.ldd = K, N, N
    d.D = 1 << 40
    d.n_ops = 8
    out = torch.zeros((8,), dtype=torch.float32, device="cuda")   # only its address is used
    for i in range(8):
        d.ops[i].kind = coda.CODA_OP_ROW_SUM
        d.ops[i].out = (1 << 41) + i * 4
        d.ops[i].out_stride = 8
    st = coda.coda_gemm_epi_noalloc(1 << 42, 1 << 43, M, N, K, d, 0)
    assert st == coda.CODA_ERR_WORKSPACE, coda.coda_status_string(st)
    assert "maximum" in coda.coda_last_error()
    del out
