"""Pins of the oracle's confidence-scheduled verify lengths: exhaustive search
over every choice of lengths on small cases (the definition evaluated
directly), the limits of a flat and of a collapsing throughput curve, the
tie order, clamping, and the binary32 survival products. None of these
calls the product path."""

import itertools

import numpy as np
import pytest

from oracle import schedule as osch


def _sps_table(rng, R, L, kind):
    B = np.arange(R * (L + 1) + 1, dtype=np.float64)
    if kind == "steps":
        # a throughput curve with steps, as when a batch spills into the next
        # hardware tile
        return 1000.0 / (1.0 + np.floor(B / 3.0)) + rng.uniform(0, 5, B.size)
    if kind == "random":
        return rng.uniform(1.0, 100.0, B.size)
    return 500.0 - 7.0 * B


@pytest.mark.parametrize("kind", ["steps", "random", "linear"])
@pytest.mark.parametrize("R,L", [(1, 4), (2, 3), (3, 3), (4, 2)])
def test_matches_exhaustive_search(kind, R, L):
    rng = np.random.default_rng(R * 10 + L)
    for _ in range(4):
        conf = rng.uniform(0.05, 1.0, (R, L)).astype(np.float32)
        sps = _sps_table(rng, R, L, kind)
        lens, best, B, _ = osch.schedule(conf, sps)
        brute = max(osch.objective(conf, sps, ls)
                    for ls in itertools.product(range(L + 1), repeat=R))
        assert best == pytest.approx(brute, rel=1e-12)
        assert osch.objective(conf, sps, lens) == pytest.approx(best, rel=1e-12)
        assert B == R + int(lens.sum())


def test_flat_curve_verifies_everything_and_collapse_verifies_nothing():
    rng = np.random.default_rng(5)
    R, L = 6, 8
    conf = rng.uniform(0.1, 0.99, (R, L)).astype(np.float32)
    flat = np.full(R * (L + 1) + 1, 50.0)
    assert np.all(osch.schedule(conf, flat)[0] == L)
    collapse = np.where(np.arange(R * (L + 1) + 1) > R, 0.0, 50.0)
    lens, best, B, _ = osch.schedule(conf, collapse)
    assert np.all(lens == 0) and B == R and best == pytest.approx(R * 50.0)


def test_equal_survivals_taken_in_index_order():
    conf = np.full((3, 2), 0.5, np.float32)
    # B = R + 2 is the best batch: the two largest survivals are three equal
    # 0.5 values; the first two in flat order are (0, 0) and (1, 0)
    sps = np.array([0, 0, 0, 10.0, 10.0, 10.0, 1.0, 1.0, 1.0, 1.0])
    lens, _, B, _ = osch.schedule(conf, sps)
    assert B == 5 and list(lens) == [1, 1, 0]


def test_selection_is_a_prefix_of_every_request():
    rng = np.random.default_rng(6)
    R, L = 40, 16
    conf = rng.uniform(0.3, 1.0, (R, L)).astype(np.float32)
    conf[::7, 3] = 1.0                                   # equal neighbours
    sps = _sps_table(rng, R, L, "steps")
    lens, _, B, theta = osch.schedule(conf, sps)
    a = osch.survivals(conf)
    t = B - R
    # the chosen survivals are exactly the t largest (ties by flat index)
    chosen = np.concatenate([a[r, :lens[r]] for r in range(R)])
    assert chosen.size == t
    assert np.isclose(np.sort(chosen)[::-1], np.sort(a.ravel())[::-1][:t]).all()
    assert theta[t] == theta.max()


def test_clamp_and_nan():
    conf = np.array([[1.5, np.nan, 0.5], [-1.0, 0.5, 0.5]], np.float32)
    a = osch.survivals(conf)
    assert list(a[0]) == [1.0, 0.0, 0.0]
    assert list(a[1]) == [0.0, 0.0, 0.0]


def test_survivals_are_binary32_left_to_right():
    rng = np.random.default_rng(7)
    conf = rng.uniform(0.0, 1.0, (5, 16)).astype(np.float32)
    a = osch.survivals(conf)
    for r in range(5):
        run = np.float32(1.0)
        for j in range(16):
            run = np.float32(run * conf[r, j])
            assert a[r, j] == run
