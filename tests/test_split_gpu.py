"""GPU parity of the split last round: tiles whose K range is shared by
several workgroups (the last to finish adds the fp32 partials in part order
and runs the epilogue), against the fp64 oracle, next to the same calls with
every tile computed whole (CODA_FLAG_NO_SPLIT_K).
Bar: |d - ref| <= max(2e-2, 1e-2 |ref|) per element."""
import numpy as np
import pytest
import torch

import workloads as w

from gpu_util import lib, run_and_compare

pytestmark = pytest.mark.gpu

NO_SPLIT = 1   # CODA_FLAG_NO_SPLIT_K


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib()


def workspace_bytes(spec, tile, flags):
    coda, runner = lib()
    inputs = w.make_inputs(spec)
    call = runner.WorkloadCall(spec, inputs, tile=tile, flags=flags)
    return coda.coda_workspace_size(spec.M, spec.N, spec.K, call.desc, 0)


# every grid here is a fraction of one round: all tiles split, into parts of
# at least 16 K steps of 64 (2 to 4 parts; ragged K gives an uneven last part)
@pytest.mark.parametrize("flags", [0, NO_SPLIT])
@pytest.mark.parametrize("tile", [2, 3])
@pytest.mark.parametrize("idx,shape", [(2, (300, 520, 2048)), (3, (300, 392, 2056)), (4, (260, 1048, 4104)),
                                       (5, (300, 520, 2048)), (2, (200, 264, 4096))])
def test_small_split_and_whole(idx, shape, tile, flags):
    spec = w.scaled_config(idx, *shape)
    if flags == 0:
        assert workspace_bytes(spec, tile, 0) > workspace_bytes(spec, tile, NO_SPLIT)
    run_and_compare(spec, w.make_inputs(spec), tile=tile, flags=flags, check_determinism=(flags == 0),
                    label=f"split cfg{idx} {shape}")


# full rounds plus a split last round: 23 x 23 = 529 tiles of 128 x 128 (two
# per CU: 512 + 17 split in 2) and 17 x 16 = 272 tiles of 256 x 256 (256 + 16
# split in 2 or 4); every row is compared, so whole and split tiles both are
@pytest.mark.parametrize("idx,shape,tile", [(4, (2944, 2944, 2048), 2), (2, (4352, 4096, 2048), 3),
                                            (3, (4352, 4096, 4096), 3)])
def test_full_rounds_plus_split_round(idx, shape, tile):
    spec = w.scaled_config(idx, *shape)
    assert workspace_bytes(spec, tile, 0) > workspace_bytes(spec, tile, NO_SPLIT)
    inputs = w.make_inputs(spec)
    stats, call = run_and_compare(spec, inputs, tile=tile, check_determinism=True,
                                  label=f"rounds+split cfg{idx} {shape}", return_call=True)
    # the split counters (the workspace's last region) are back at zero
    ws = call.ws[0]
    tail = ws[-256:].cpu()
    assert int(tail.sum()) == 0
    del call
