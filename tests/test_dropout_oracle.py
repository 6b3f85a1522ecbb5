"""Pins of the oracle's dropout and its generator (Philox-4x64-10).

The generator is checked against numpy's own Philox bit generator (an
independent implementation of the same published definition, keyed and
counted explicitly), the vectorised form against the scalar one, and the op
against the properties inverted dropout has by definition: the keep rate, the
unchanged expectation, p = 0 as the identity, and a mask that depends on the
element's row and column only.
"""
import numpy as np
import pytest

import oracle
from oracle import coda_oracle as co

M64 = (1 << 64) - 1


def _numpy_philox_block(counter, key):
    """numpy's Philox advances its 256-bit counter before each block, so start it one below."""
    v = sum(int(x) << (64 * i) for i, x in enumerate(counter))
    v = (v - 1) % (1 << 256)
    start = np.array([(v >> (64 * i)) & M64 for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(counter=start, key=np.array(key, dtype=np.uint64))
    return [int(x) for x in bg.random_raw(4)]


CASES = [((0, 0, 0, 0), (0, 0)), ((1, 0, 0, 0), (0, 0)), ((5, 7, 0, 0), (123, 456)),
         ((M64, 3, 9, 1), (1, 2)), ((0x0123456789ABCDEF, M64, M64, M64), (M64, M64)),
         ((12, 34, 56, 78), (0xDEADBEEF, 0))]


@pytest.mark.parametrize("counter,key", CASES)
def test_philox_scalar_matches_numpy(counter, key):
    assert oracle.philox4x64_scalar(counter, key) == _numpy_philox_block(counter, key)


def test_philox_vectorised_matches_scalar():
    rng = np.random.default_rng(11)
    c = rng.integers(0, 2 ** 63, size=(4, 200), dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    c[:, :3] = [[0, M64, 1], [0, M64, 2], [0, M64, 3], [0, M64, 4]]
    key = (0xFEEDFACECAFEBEEF, 0x0123456789ABCDEF)
    got = oracle.philox4x64(c[0], c[1], c[2], c[3], key)
    for t in range(c.shape[1]):
        ref = oracle.philox4x64_scalar([int(c[i, t]) for i in range(4)], key)
        assert [int(got[w][t]) for w in range(4)] == ref


def test_mulhilo_limbs_exact():
    rng = np.random.default_rng(3)
    a = rng.integers(0, 2 ** 64 - 1, size=500, dtype=np.uint64, endpoint=True)
    a[:2] = [M64, 0]
    for b in (co.PHILOX_M0, co.PHILOX_M1, M64, 1):
        hi, lo = co._mulhilo64(a, b)
        for x, h, l in zip(a, hi, lo):
            p = int(x) * b
            assert (int(h), int(l)) == (p >> 64, p & M64)


def test_dropout_words_layout_against_numpy_stream():
    # element (row i, column j) takes 32-bit word j % 8 of block (j // 8, i, offset, 0):
    # the low half of 64-bit word (j % 8) // 2 for even j % 8, the high half for odd
    seed, offset = 2024, 7
    rows = np.array([0, 3, 1000])
    words = oracle.dropout_words(rows, 20, seed, offset)
    for r_i, i in enumerate(rows):
        for blk in range(3):
            raw = _numpy_philox_block((blk, int(i), offset, 0), (seed, 0))
            for j in range(8 * blk, min(8 * blk + 8, 20)):
                e = j % 8
                want = (raw[e // 2] >> (32 * (e % 2))) & 0xFFFFFFFF
                assert int(words[r_i, j]) == want


def test_threshold_closed_forms():
    assert oracle.dropout_threshold(0.0) == 0
    assert oracle.dropout_threshold(0.5) == 2 ** 31
    assert oracle.dropout_threshold(0.25) == 2 ** 30
    # 0.1 is not exact in fp32: the threshold uses its fp32 value
    assert oracle.dropout_threshold(0.1) == int(np.floor(np.float64(np.float32(0.1)) * 2.0 ** 32))
    for bad in (-0.1, 1.0, 1.5):
        with pytest.raises(ValueError):
            oracle.dropout_threshold(bad)


def test_dropout_p0_is_identity():
    v = np.random.default_rng(1).standard_normal((9, 21))
    assert np.array_equal(oracle.dropout(v, 0.0, seed=5), v)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_dropout_keep_rate_and_expectation(p):
    M, N = 512, 2048
    keep = oracle.dropout_keep(np.arange(M), N, p, seed=99)
    n = M * N
    rate = keep.mean()
    sd = np.sqrt(p * (1 - p) / n)
    assert abs(rate - (1 - p)) < 6 * sd
    # inverted dropout keeps the mean: E[dropout(1)] = 1
    out = oracle.dropout(np.ones((M, N)), p, seed=99)
    assert abs(out.mean() - 1.0) < 6 * sd / (1 - np.float32(p))
    assert set(np.unique(out)) <= {0.0, 1.0 / (1.0 - float(np.float32(p)))}


def test_dropout_columns_and_rows_independent():
    # neighbouring elements share no word: no two columns of a row, and no two
    # rows of a column, carry the same mask pattern over a long stretch
    keep = oracle.dropout_keep(np.arange(256), 256, 0.5, seed=1)
    for j in range(1, 16):
        assert not np.array_equal(keep[:, 0], keep[:, j])
    for i in range(1, 16):
        assert not np.array_equal(keep[0], keep[i])
    # the seed and the offset change the mask
    assert not np.array_equal(keep, oracle.dropout_keep(np.arange(256), 256, 0.5, seed=2))
    assert not np.array_equal(keep, oracle.dropout_keep(np.arange(256), 256, 0.5, seed=1, offset=1))


def test_dropout_row_subset_matches_full():
    rng = np.random.default_rng(4)
    A = rng.standard_normal((40, 16))
    B = rng.standard_normal((16, 24))
    prog = [("gelu_tanh", {}), ("dropout", {"p": 0.3, "seed": 77, "offset": 2})]
    D, _ = oracle.forward(A, B, prog)
    rows = np.array([39, 0, 17, 5])
    Ds, _ = oracle.forward(A[rows], B, prog, row_ids=rows)
    assert np.array_equal(Ds, D[rows])
    # without the row ids the subset would be masked as rows 0..3
    D0, _ = oracle.forward(A[rows], B, prog)
    assert not np.array_equal(D0, D[rows])


def test_dropout_after_swiglu_uses_running_width():
    rng = np.random.default_rng(6)
    C = rng.standard_normal((8, 20))
    v, _ = oracle.apply_epilogue(C, [("swiglu_pair", {}), ("dropout", {"p": 0.5, "seed": 3})])
    ref = oracle.swiglu_pair(C)
    keep = oracle.dropout_keep(np.arange(8), 10, 0.5, seed=3)
    assert np.array_equal(v, np.where(keep, ref * 2.0, 0.0))


def test_planted_generator_mistakes_are_caught():
    counter, key = (5, 7, 0, 0), (123, 456)
    ref = _numpy_philox_block(counter, key)

    def variant(m0=co.PHILOX_M0, w0=co.PHILOX_W0, rounds=10, swap=False):
        m64 = M64
        c = list(counter)
        k0, k1 = key
        for _ in range(rounds):
            p0 = m0 * c[0]
            p1 = co.PHILOX_M1 * c[2]
            if swap:
                c = [(p0 >> 64) ^ c[1] ^ k0, p0 & m64, (p1 >> 64) ^ c[3] ^ k1, p1 & m64]
            else:
                c = [(p1 >> 64) ^ c[1] ^ k0, p1 & m64, (p0 >> 64) ^ c[3] ^ k1, p0 & m64]
            k0 = (k0 + w0) & m64
            k1 = (k1 + co.PHILOX_W1) & m64
        return c
    assert variant() == ref
    assert variant(m0=co.PHILOX_M0 ^ 2) != ref
    assert variant(w0=co.PHILOX_W0 + 1) != ref
    assert variant(rounds=7) != ref
    assert variant(swap=True) != ref
