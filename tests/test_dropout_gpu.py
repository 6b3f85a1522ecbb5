"""Dropout in the epilogue (fused and unfused) against the oracle: the keep
mask bit for bit (a dropped element is exactly 0, a kept one is not and is
within the bar of the oracle's value), at ragged shapes, every tile, both B
layouts, after SWIGLU_PAIR (four columns per lane chunk), with a row
reduction after it, and at the GPT-2-small layer's full size on every row."""
import numpy as np
import pytest
import torch

import oracle
import workloads as w

from gpu_util import announce, assert_close, lib, unfused_extra

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


def check_mask(D, ref, keep, what):
    """Dropped elements exactly zero; kept elements nonzero wherever the oracle's value is."""
    assert D.shape == keep.shape
    dropped_nonzero = int(np.count_nonzero(D[~keep]))
    assert dropped_nonzero == 0, f"{what}: {dropped_nonzero} dropped elements are not 0"
    kept_zero = int(np.count_nonzero((D == 0) & keep & (np.abs(ref) > 1e-6)))
    assert kept_zero == 0, f"{what}: {kept_zero} kept elements are 0"
    print(f"  {what}: mask ok ({int(keep.sum())} kept of {keep.size})", flush=True)


def program(rng, M, N, p, seed, offset, swiglu=False):
    bias = bf16(0.1 * rng.standard_normal(N))
    rs = torch.zeros((M, 1), dtype=torch.float32, device="cuda")
    ops = [("add_col", {"vec": bias}), ("gelu_tanh", {})]
    if swiglu:
        ops.append(("swiglu_pair", {}))
    ops += [("dropout", {"p": p, "seed": seed, "offset": offset}), ("row_sum", {"out": rs, "col": 0})]
    o_ops = [("add_col", {"vec": f64(bias)}), ("gelu_tanh", {})] + ([("swiglu_pair", {})] if swiglu else []) + \
        [("dropout", {"p": p, "seed": seed, "offset": offset}), ("row_sum", {})]
    return ops, o_ops, rs


@pytest.mark.parametrize("mode", ["fused", "unfused"])
@pytest.mark.parametrize("layout", ["KN", "NK"])
@pytest.mark.parametrize("M,N,K", [(136, 264, 72), (257, 520, 128), (1, 8, 8)])
def test_dropout_ragged(CR, mode, layout, M, N, K):
    coda, runner = CR
    announce(f"dropout {mode} {layout} {M}x{N}x{K}")
    rng = np.random.default_rng(300 + M)
    a, b = rng.standard_normal((M, K)), rng.standard_normal((K, N)) / np.sqrt(K)
    A = bf16(a)
    B = bf16(b if layout == "KN" else np.ascontiguousarray(b.T))
    p, seed, offset = 0.1, 0xC0DA5EED, 3
    ops, o_ops, rs = program(rng, M, N, p, seed, offset)
    call = runner.Call(A, B, ops, layout, d_dtype=torch.float32)
    coda.check(call.fused() if mode == "fused" else call.unfused(), f"dropout {mode}")
    torch.cuda.synchronize()
    ref, reds = oracle.forward(f64(A), f64(B), o_ops, layout)
    keep = oracle.dropout_keep(np.arange(M), N, p, seed, offset)
    D = f64(call.D)
    check_mask(D, ref, keep, f"dropout {mode} {layout}")
    assert_close(D, ref, f"dropout {mode} {layout} D")
    # fp32 intermediates on the unfused path: its stored values round at 2^-24
    assert_close(f64(rs)[:, 0], reds[0][2], f"dropout {mode} {layout} row sum after dropout")


@pytest.mark.parametrize("tile", [1, 2, 3])
@pytest.mark.parametrize("mode", ["fused", "unfused"])
def test_dropout_after_swiglu_every_tile(CR, tile, mode):
    coda, runner = CR
    announce(f"dropout after swiglu tile{tile} {mode}")
    rng = np.random.default_rng(41 + tile)
    M, N, K = 300, 528, 136
    A, B = bf16(rng.standard_normal((M, K))), bf16(rng.standard_normal((K, N)) / np.sqrt(K))
    p, seed, offset = 0.3, 12345, 0
    ops, o_ops, rs = program(rng, M, N, p, seed, offset, swiglu=True)
    call = runner.Call(A, B, ops, "KN", d_dtype=torch.float32, tile=tile)
    coda.check(call.fused() if mode == "fused" else call.unfused(), "dropout swiglu")
    torch.cuda.synchronize()
    ref, reds = oracle.forward(f64(A), f64(B), o_ops, "KN")
    keep = oracle.dropout_keep(np.arange(M), N // 2, p, seed, offset)
    D = f64(call.D)
    check_mask(D, ref, keep, f"dropout swiglu tile{tile} {mode}")
    assert_close(D, ref, f"dropout swiglu tile{tile} {mode} D")
    assert_close(f64(rs)[:, 0], reds[0][2], f"dropout swiglu tile{tile} {mode} row sum")


def test_dropout_keep_rate_and_bf16_output(CR):
    coda, runner = CR
    announce("dropout keep rate, bf16 D")
    rng = np.random.default_rng(9)
    M, N, K = 1024, 2048, 64
    A, B = bf16(rng.standard_normal((M, K))), bf16(rng.standard_normal((K, N)) / np.sqrt(K))
    for p in (0.0, 0.5, 0.9):
        call = runner.Call(A, B, [("dropout", {"p": p, "seed": 77, "offset": 1})], "KN")
        coda.check(call.fused(), "dropout bf16")
        torch.cuda.synchronize()
        ref, _ = oracle.forward(f64(A), f64(B), [("dropout", {"p": p, "seed": 77, "offset": 1})], "KN")
        keep = oracle.dropout_keep(np.arange(M), N, p, 77, 1)
        D = f64(call.D)
        check_mask(D, ref, keep, f"dropout p={p} bf16")
        assert_close(D, ref, f"dropout p={p} bf16 D")
        rate = keep.mean()
        assert abs(rate - (1 - p)) < 6 * np.sqrt(max(p * (1 - p), 1e-12) / keep.size) + 1e-12


def test_dropout_full_size_gpt2_small(CR):
    """The GPT-2-small MLP up-projection with dropout after the activation, at
    its full size, compared on every row."""
    coda, runner = CR
    import dataclasses
    spec = w.get_config(2)
    spec = dataclasses.replace(spec, program=spec.program + (("dropout", {"p": 0.1, "seed": 2026, "offset": 5}),))
    announce(f"dropout full size {spec.name} M={spec.M} N={spec.N} K={spec.K}")
    inputs = w.make_inputs(spec)
    call = runner.WorkloadCall(spec, inputs)
    coda.check(call.fused(), "dropout full size")
    torch.cuda.synchronize()
    D = runner.tensor_to_f64(call.D)
    D_ref, _ = oracle.run_workload(spec, inputs)
    keep = oracle.dropout_keep(np.arange(spec.M), spec.N, 0.1, 2026, 5)
    check_mask(D, D_ref, keep, "dropout full size")
    assert_close(D, D_ref, "dropout full size D")
    del call
