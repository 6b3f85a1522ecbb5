"""The binding rejects tensors that do not fit the op that reads or writes
them (host only: nothing is launched).  The C ABI sees raw pointers and cannot
check extents, so these checks stand between a wrong tensor and a kernel
writing past it."""
import pytest
import torch

from gemm_epilogue_transformer_bf16_amd import runner

M, N, K = 16, 24, 32


def mats():
    A = torch.zeros((M, K), dtype=torch.bfloat16)
    B = torch.zeros((K, N), dtype=torch.bfloat16)
    return A, B


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def test_valid_list_is_accepted():
    A, B = mats()
    stats = f32(M, 2)
    runner.Call(A, B, [("add_col", {"vec": bf(N)}), ("add_mat", {"mat": bf(M, N)}), ("swiglu_pair", {}),
                       ("row_sum", {"out": stats, "col": 1}), ("col_sum", {"out": f32(N // 2, 1)}),
                       ("dropout", {"p": 0.1, "seed": 3})], "KN")


@pytest.mark.parametrize("ops,msg", [
    ([("row_sum", {"out": f32(M - 1, 2), "col": 0})], "rows"),                 # too few rows
    ([("row_sum", {"out": bf(M, 2), "col": 0})], "dtype"),                     # not fp32
    ([("row_sum", {"out": f32(M, 2), "col": 2})], "column 2"),                 # column out of range
    ([("row_sum", {"out": f32(M, 4)[:, ::2], "col": 0})], "inner dimension"),  # strided
    ([("col_sum", {"out": f32(N - 8, 1), "col": 0})], "rows"),                 # one row per column
    ([("swiglu_pair", {}), ("col_sum", {"out": f32(N // 2 - 1, 1)})], "rows"),
    ([("add_mat", {"mat": bf(M - 1, N)})], "rows"),
    ([("add_mat", {"mat": bf(M, N - 8)})], "columns"),
    ([("add_mat", {"mat": bf(M, 2 * N)[:, ::2]})], "inner dimension"),
    ([("mul_dgelu_tanh", {"mat": bf(M)})], "2-D"),
    ([("add_col", {"vec": bf(N - 1)})], "at least"),
    ([("scale_row", {"vec": bf(M - 1)})], "at least"),
    ([("swiglu_pair", {}), ("add_col", {"vec": bf(N // 2 - 1)})], "at least"),
    ([("rms_bwd", {"x": bf(M, N), "gamma": bf(N), "eps": 1e-6, "stats": f32(M, 1)})], "t_col"),
    ([("rms_bwd", {"x": bf(M - 1, N), "gamma": bf(N), "eps": 1e-6, "stats": f32(M, 2)})], "rows"),
    ([("rms_dgamma", {"x": bf(M, N), "eps": 1e-6, "stats": bf(M, 2), "out": f32(N, 1)})], "dtype"),
    ([("row_dot", {"mat": bf(M, N), "out": f32(M, 1), "col": 1})], "column 1"),
    ([("dropout", {"p": 1.0})], "outside"),
    ([("rms_rowscale", {"gamma": bf(K - 8), "eps": 1e-6})], "at least"),
    ([("rms_rowscale", {"gamma": torch.zeros(K), "eps": 1e-6})], "dtype"),
])
def test_ill_fitting_operands_are_rejected(ops, msg):
    A, B = mats()
    with pytest.raises(ValueError, match=msg):
        runner.Call(A, B, ops, "KN")
