"""GPU parity of the fused and unfused HIP paths against the fp64 oracle,
through the C ABI.  Bar: |d - ref| <= max(2e-2, 1e-2 |ref|) per element."""
import numpy as np
import pytest
import torch

import workloads as w

from gpu_util import lib, run_and_compare

pytestmark = pytest.mark.gpu

# small shapes that span several tiles and leave ragged tails in M, N and K
SMALL = {
    1: (256, 256, 256),
    2: (300, 520, 200),
    3: (300, 392, 264),
    4: (260, 1048, 136),
    5: (300, 520, 200),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib()


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("mode", ["fused", "unfused"])
def test_small_configs(idx, mode):
    spec = w.scaled_config(idx, *SMALL[idx])
    run_and_compare(spec, w.make_inputs(spec), mode=mode, label=f"small cfg{idx}")


@pytest.mark.parametrize("tile", [1, 2, 3])
@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_small_configs_every_tile(idx, tile):
    spec = w.scaled_config(idx, *SMALL[idx])
    run_and_compare(spec, w.make_inputs(spec), mode="fused", tile=tile, label=f"small cfg{idx}")


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_full_size_every_row_fused(idx):
    spec = w.get_config(idx)
    inputs = w.make_inputs(spec)
    run_and_compare(spec, inputs, mode="fused", label=f"full cfg{idx}", check_determinism=True)


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_full_size_every_row_unfused(idx):
    spec = w.get_config(idx)
    inputs = w.make_inputs(spec)
    run_and_compare(spec, inputs, mode="unfused", label=f"full cfg{idx}")


def test_full_cfg1_exact_shape_both_modes():
    spec = w.get_config(1)
    inputs = w.make_inputs(spec)
    run_and_compare(spec, inputs, mode="fused", check_determinism=True)
    run_and_compare(spec, inputs, mode="unfused")
