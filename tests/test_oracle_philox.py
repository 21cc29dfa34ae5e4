"""Pins of the oracle's Philox4x64-10 against numpy's independent
implementation (numpy.random.Philox is Philox4x64-10)."""

import numpy as np
import pytest

from oracle import philox


def _numpy_block(counter, key):
    """numpy advances its 256-bit counter by one before producing a block, so
    random_raw(4) from counter c returns the block of c + 1."""
    c = [int(w) for w in counter]
    # c - 1 as a 256-bit integer, little-endian words
    value = sum(w << (64 * i) for i, w in enumerate(c)) - 1
    prev = [(value >> (64 * i)) & ((1 << 64) - 1) for i in range(4)]
    bg = np.random.Philox(counter=np.array(prev, dtype=np.uint64),
                          key=np.array(key, dtype=np.uint64))
    return tuple(int(x) for x in bg.random_raw(4))


def test_block_matches_numpy_random_counters():
    rng = np.random.default_rng(1234)
    for _ in range(200):
        counter = [int(x) for x in rng.integers(0, 2**64, size=4, dtype=np.uint64)]
        counter[0] = max(counter[0], 1)
        key = [int(x) for x in rng.integers(0, 2**64, size=2, dtype=np.uint64)]
        assert philox.block(counter, key) == _numpy_block(counter, key)


@pytest.mark.parametrize("b,k,seed", [(0, 0, 0), (1, 0, 0), (0, 3, 0),
                                      (63, 7, 0), (5, 2, 2**64 - 1),
                                      (255, 8, 0x0123456789ABCDEF)])
def test_verify_counter_layout_matches_numpy(b, k, seed):
    # counter (b, k, 0, 0), key (seed, 0); b = 0 needs the borrow across
    # words in the numpy offset, which _numpy_block handles.
    assert philox.block((b, k, 0, 0), (seed, 0)) == _numpy_block((b, k, 0, 0), (seed, 0))


def test_uniforms_are_top_24_bits():
    rng = np.random.default_rng(7)
    for _ in range(100):
        b, k = int(rng.integers(0, 1000)), int(rng.integers(0, 16))
        seed = int(rng.integers(0, 2**63))
        w = _numpy_block((b, k, 0, 0), (seed, 0))
        u, u2 = philox.verify_uniforms(seed, b, k)
        assert u == (w[0] >> 40) / 2.0**24
        assert u2 == (w[1] >> 40) / 2.0**24
        assert 0.0 <= u < 1.0 and 0.0 <= u2 < 1.0
        # exact in binary32
        assert float(np.float32(u)) == u and float(np.float32(u2)) == u2


def test_uniforms_look_uniform():
    us = np.array([philox.verify_uniforms(0, b, k)[i]
                   for b in range(500) for k in range(4) for i in range(2)])
    assert abs(us.mean() - 0.5) < 5 * np.sqrt(1 / 12 / us.size)
    hist, _ = np.histogram(us, bins=10, range=(0, 1))
    from scipy.stats import chisquare
    assert chisquare(hist).pvalue > 1e-3
