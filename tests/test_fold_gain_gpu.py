"""RMSNorm with the gain folded into the weights (B = diag(gamma) W, prepared
once by coda_fold_gain; (x * gamma) W = x (gamma W) is the reparameterisation
of the zeli.app page's "augment_me" comment), through the C ABI, against the
fp64 oracle of the unfolded layer."""
import numpy as np
import pytest
import torch

import workloads as w

from gpu_util import announce, lib, run_and_compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def CR():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return lib()


@pytest.mark.parametrize("layout", ["KN", "NK"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fold_gain_is_the_rounded_product(CR, layout, dtype):
    """Each element of B_out is gamma[k] * B[k, j] rounded once (bit-exact)."""
    coda, runner = CR
    announce(f"fold_gain {layout} {dtype}")
    rng = np.random.default_rng(71)
    K, N = 136, 264
    b = rng.standard_normal((K, N)) / np.sqrt(K)
    g = 1 + 0.1 * rng.standard_normal(K)
    if dtype == "bf16":
        b_s, g_s = w.bf16_bits_from_f64(b), w.bf16_bits_from_f64(g)
        b64, g64 = w.bf16_bits_to_f64(b_s), w.bf16_bits_to_f64(g_s)
        want = w.bf16_bits_from_f64(g64[:, None] * b64)      # exact product, one RNE rounding
        to_dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
        Bt, Gt = to_dev(b_s if layout == "KN" else b_s.T), to_dev(g_s)
    else:
        b32, g32 = b.astype(np.float32), g.astype(np.float32)
        want = (g32[:, None] * b32).astype(np.float32)       # one fp32 rounding
        Bt = torch.from_numpy(np.ascontiguousarray(b32 if layout == "KN" else b32.T)).cuda()
        Gt = torch.from_numpy(g32).cuda()
    out = torch.empty_like(Bt)
    st = coda.coda_fold_gain(Bt.data_ptr(), K, N, Bt.stride(0), coda.CODA_B_KN if layout == "KN" else coda.CODA_B_NK,
                             runner.CODA_DT[Bt.dtype], Gt.data_ptr(), out.data_ptr(), out.stride(0),
                             runner.current_stream_ptr())
    coda.check(st, "coda_fold_gain")
    torch.cuda.synchronize()
    got = out.cpu()
    got = got.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else got.numpy()
    if layout == "NK":
        got = got.T
    assert np.array_equal(got, want)


SMALL = {1: (256, 256, 256), 2: (136, 264, 72), 4: (130, 528, 64)}
RAGGED = {2: (300, 520, 200), 4: (520, 392, 256)}


@pytest.mark.parametrize("idx", [1, 2, 4])
@pytest.mark.parametrize("mode", ["fused", "unfused"])
def test_folded_small(CR, idx, mode):
    spec = w.scaled_config(idx, *SMALL[idx])
    run_and_compare(spec, w.make_inputs(spec), mode=mode, fold_gain=True, label=f"folded cfg{idx}",
                    check_determinism=(mode == "fused"))


@pytest.mark.parametrize("idx", [2, 4])
@pytest.mark.parametrize("tile", [1, 2, 3])
def test_folded_every_tile(CR, idx, tile):
    spec = w.scaled_config(idx, *RAGGED[idx])
    run_and_compare(spec, w.make_inputs(spec), tile=tile, fold_gain=True, label=f"folded cfg{idx} tile{tile}")


@pytest.mark.parametrize("flags", [0, 1])
def test_folded_split_round(CR, flags):
    # 12 x 12 = 144 tiles of 256 x 256 with 32 K steps: the last, partial round
    # is split over K (flags 0) or computed whole (CODA_FLAG_NO_SPLIT_K)
    spec = w.scaled_config(4, 2944, 2944, 2048)
    run_and_compare(spec, w.make_inputs(spec), tile=3, flags=flags, fold_gain=True,
                    check_determinism=True, label=f"folded split flags={flags}")


@pytest.mark.parametrize("idx", [2, 4])
@pytest.mark.parametrize("mode", ["fused", "unfused"])
def test_folded_full_size_every_row(CR, idx, mode):
    spec = w.get_config(idx)
    run_and_compare(spec, w.make_inputs(spec), mode=mode, fold_gain=True, label=f"folded full cfg{idx}",
                    check_determinism=(mode == "fused"))
