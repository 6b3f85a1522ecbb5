"""Cross-workgroup finishes whose count of partials is not a multiple of the
eight loads the finishing workgroup issues together: row reductions over 3,
9 and 17 (or 6, 18 and 34) tile columns and column reductions over 3, 9 and
17 tile rows, on every tile configuration, against the fp64 oracle; and
tiles of the last round split into three parts (in-loop RMSNorm, plain GEMM),
whose other parts come back through LDS or in batches of registers.
Bar: |d - ref| <= max(2e-2, 1e-2 |ref|) per element; results bitwise
repeatable."""
import numpy as np
import pytest
import torch

import oracle
import workloads as w

from gpu_util import announce, assert_close, lib, run_and_compare
from test_colred_gpu import backward_case, f64, oracle_ops
from test_split_gpu import NO_SPLIT, workspace_bytes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def CR():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return lib()


# BERT-large down-projection recipe (bias, residual, row sum and row sum of
# squares); N = 712, 2200, 4352 give 3, 9, 17 tile columns of 256 (6, 18, 34
# of 128)
@pytest.mark.parametrize("tile", [1, 2, 3])
@pytest.mark.parametrize("N", [712, 2200, 4352])
def test_row_reductions_over_odd_tile_counts(CR, tile, N):
    spec = w.scaled_config(3, 264, N, 136)
    run_and_compare(spec, w.make_inputs(spec), tile=tile, check_determinism=True,
                    label=f"row reductions N={N} tile{tile}")


# GPT-2-medium backward recipe with the bias gradient (a column sum of dH):
# M = 700, 2204, 4352 give 3, 9, 17 tile rows of 256 (6, 18, 34 of 128)
@pytest.mark.parametrize("tile", [1, 2, 3])
@pytest.mark.parametrize("M", [700, 2204, 4352])
def test_column_reductions_over_odd_tile_counts(CR, tile, M):
    coda, runner = CR
    announce(f"column reductions M={M} tile{tile}")
    rng = np.random.default_rng(91)
    N, K = 264, 72
    dY, W2, P = backward_case(rng, M, N, K)
    db = torch.zeros((N, 1), dtype=torch.float32, device="cuda")
    ops = [("mul_dgelu_tanh", {"mat": P}), ("col_sum", {"out": db, "col": 0})]
    call = runner.Call(dY, W2, ops, "NK", tile=tile)
    coda.check(call.fused(), "fused")
    torch.cuda.synchronize()
    ref, reds = oracle.forward(f64(dY), f64(W2), oracle_ops(ops), "NK")
    assert_close(f64(call.D), ref, "D")
    assert_close(f64(db)[:, 0], reds[0][2], "col_sum")
    first = db.clone()
    coda.check(call.fused(), "repeat")
    torch.cuda.synchronize()
    assert torch.equal(first, db), "column sums not bitwise repeatable"


# grids under one round with 48 or 49 K steps: every tile is split into three
# parts (the third one short with K = 3096)
@pytest.mark.parametrize("tile", [2, 3])
@pytest.mark.parametrize("idx,shape", [(4, (260, 1048, 3072)), (2, (300, 520, 3096)), (5, (300, 520, 3072))])
def test_three_part_split(CR, idx, shape, tile):
    spec = w.scaled_config(idx, *shape)
    assert workspace_bytes(spec, tile, 0) > workspace_bytes(spec, tile, NO_SPLIT)
    run_and_compare(spec, w.make_inputs(spec), tile=tile, check_determinism=True,
                    label=f"three-part split cfg{idx} {shape} tile{tile}")
