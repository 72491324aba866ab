"""Pins for oracle.philox: numpy's Philox4x64-10 bit generator is the library reference.

numpy advances its 256-bit counter by one before producing a block, so the
block for counter c is what numpy yields when seeded with counter c - 1.
"""

import numpy as np
import pytest

from oracle import philox

MASK = (1 << 64) - 1


def _minus_one(ctr):
    words = list(ctr)
    for i in range(4):
        if words[i] > 0:
            words[i] -= 1
            return tuple(words)
        words[i] = MASK
    return tuple(words)


def _numpy_block(ctr, key):
    bg = np.random.Philox(counter=np.array(_minus_one(ctr), dtype=np.uint64),
                          key=np.array(key, dtype=np.uint64))
    return tuple(int(w) for w in bg.random_raw(4))


CASES = [
    ((0, 0, 0, 0), (0, 0)),
    ((5, 7, 11, 13), (0x0123456789ABCDEF, 0xFEDCBA9876543210)),
    ((MASK, MASK, MASK, 1), (MASK, MASK)),
    ((0, 1, 0, 0), (1, 0)),                        # numpy's seed counter borrows across words
    ((123456, 4096 + 3, 77, 0), (0xDEADBEEF, 0xC0FFEE)),
]


@pytest.mark.parametrize("ctr,key", CASES)
def test_block_matches_numpy_philox(ctr, key):
    assert philox.philox4x64(ctr, key) == _numpy_block(ctr, key)


def test_many_random_blocks_match_numpy():
    rng = np.random.Generator(np.random.PCG64(7))
    for _ in range(200):
        ctr = tuple(int(v) for v in rng.integers(0, 2**63, size=4, dtype=np.int64))
        ctr = (ctr[0] + 1,) + ctr[1:]
        key = tuple(int(v) for v in rng.integers(0, 2**63, size=2, dtype=np.int64))
        assert philox.philox4x64(ctr, key) == _numpy_block(ctr, key)


def test_unit_double_matches_numpy_random():
    """numpy's Generator.random() maps each 64-bit word to (w >> 11) * 2**-53."""
    ctr, key = (9, 8, 7, 6), (5, 4)
    gen = np.random.Generator(np.random.Philox(counter=np.array(_minus_one(ctr), dtype=np.uint64),
                                               key=np.array(key, dtype=np.uint64)))
    expect = gen.random(4)
    words = philox.philox4x64(ctr, key)
    got = [philox.unit_double(w) for w in words]
    assert got == [float(v) for v in expect]


def test_unit_double_range():
    assert philox.unit_double(0) == 0.0
    assert philox.unit_double(MASK) < 1.0
    assert philox.unit_double(MASK) == 1.0 - 2.0 ** -53


def test_decision_uniforms_are_words_0_and_1():
    seed = (11, 22)
    u, v = philox.decision_uniforms(seed, 3, 4100, 9)
    w = philox.philox4x64((3, 4100, 9, 0), seed)
    assert u == philox.unit_double(w[0]) and v == philox.unit_double(w[1])


def test_distinct_keys_give_distinct_streams():
    a = philox.decision_uniforms((1, 2), 0, 10, 0)
    b = philox.decision_uniforms((1, 2), 0, 11, 0)
    c = philox.decision_uniforms((1, 2), 1, 10, 0)
    d = philox.decision_uniforms((1, 2), 0, 10, 1)
    assert len({a, b, c, d}) == 4


def test_reduced_rounds_differ():
    """A dropped round is caught: 9 rounds do not reproduce numpy's output."""
    ctr, key = (5, 7, 11, 13), (3, 4)
    assert philox.philox4x64(ctr, key, rounds=9) != _numpy_block(ctr, key)
