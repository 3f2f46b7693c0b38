"""Pins of the oracle's Philox4x64-10 against an independent implementation.

numpy.random.Philox implements the same published generator (Salmon et al., SC'11).
numpy increments its 256-bit counter before producing a block, so the block for
counter c is the first block numpy returns after its counter is set to c - 1.
"""
import numpy as np
import pytest

from oracle import philox


def numpy_block(counter, key):
    c = [int(x) for x in counter]
    # c - 1 with borrow across the four 64-bit words
    i = 0
    while i < 4 and c[i] == 0:
        c[i] = (1 << 64) - 1
        i += 1
    if i < 4:
        c[i] -= 1
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64),
                          counter=np.array(c, dtype=np.uint64))
    return tuple(int(v) for v in bg.random_raw(4))


CASES = [
    ((0, 0, 0, 0), (0, 0)),
    ((1, 0, 0, 0), (5, 0)),
    ((7, 3, 11, 2), (12345, 0)),
    ((2**64 - 1, 2**64 - 1, 0, 1), (2**63 + 17, 99)),
    ((31, 8, 31, 2), (0, 0)),
]


@pytest.mark.parametrize("counter,key", CASES)
def test_scalar_matches_numpy(counter, key):
    assert philox.philox4x64_scalar(counter, key) == numpy_block(counter, key)


def test_vector_matches_scalar():
    rng = np.random.default_rng(3)
    c = rng.integers(0, 2**63, size=(4, 64), dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    k = rng.integers(0, 2**63, size=(2, 64), dtype=np.uint64)
    out = philox.philox4x64(c[0], c[1], c[2], c[3], k[0], k[1])
    for i in range(64):
        ref = philox.philox4x64_scalar([int(c[w, i]) for w in range(4)],
                                       [int(k[0, i]), int(k[1, i])])
        assert tuple(int(o[i]) for o in out) == ref


def test_uniform_grid_and_range():
    rnd, j, b = np.meshgrid(np.arange(8), np.arange(9), np.arange(32), indexing="ij")
    u = philox.uniform(0, rnd, j, b, philox.PURPOSE_ACCEPT)
    assert u.min() >= 0.0 and u.max() <= 1.0 - 2.0 ** -24
    assert np.all(u * 2**24 == np.floor(u * 2**24))
    # distinct purposes give distinct streams
    u2 = philox.uniform(0, rnd, j, b, philox.PURPOSE_RESAMPLE)
    assert np.mean(u == u2) < 1e-3
    # the uniform is the top 24 bits of word 0
    w0 = philox.philox4x64_scalar((3, 4, 5, 1), (77, 0))[0]
    assert philox.uniform(77, 3, 4, 5, 1) == (w0 >> 40) * 2.0 ** -24


def test_uniform_moments():
    n = np.arange(200000)
    u = philox.uniform(1, n, 0, 0, 0)
    assert abs(u.mean() - 0.5) < 4 * np.sqrt(1 / 12 / n.size)
    assert abs(u.var() - 1 / 12) < 2e-3
