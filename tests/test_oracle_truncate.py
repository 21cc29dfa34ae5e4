"""Pins of the oracle's top-k / top-p truncation: the limits (top-k = 1 is
the argmax, nothing truncated when disabled), agreement with an independent
formulation of top-p (sort ascending, drop the tokens whose cumulative mass
stays within 1 - top_p), the tie order, the status of a bad top_p, and the
law of the emitted token, which must be the truncated target distribution
(exact enumeration through the verify step with truncation on)."""

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

from oracle import truncate as ot
from oracle import verify as ov

LATTICE = 4096


def _lattice():
    return (np.arange(LATTICE) + 0.5) / LATTICE


def test_top_k_one_is_the_argmax_and_disabled_keeps_all():
    rng = np.random.default_rng(1)
    s = rng.standard_normal(50)
    p, _, _, _ = ot.truncated_softmax(s, 1, 1.0)
    assert p[np.argmax(s)] == 1.0 and np.count_nonzero(p) == 1
    for k in (0, -3, 50, 77):
        p, _, _, margin = ot.truncated_softmax(s, k, 1.0)
        assert np.allclose(p, sp_softmax(s), rtol=1e-13) and margin == np.inf


def test_top_k_keeps_the_k_largest_renormalised():
    rng = np.random.default_rng(2)
    s = rng.standard_normal(40)
    p, _, _, _ = ot.truncated_softmax(s, 7, 1.0)
    top = np.argsort(-s)[:7]
    expect = np.zeros(40)
    expect[top] = sp_softmax(s[top])
    assert np.allclose(p, expect, rtol=1e-13, atol=0)


def _top_p_ascending(s, top_p):
    """Independent formulation: sort ascending, drop tokens while the
    cumulative mass from the bottom stays <= 1 - top_p (keeping the top
    token always)."""
    p = sp_softmax(np.asarray(s, dtype=np.float64))
    idx = np.argsort(p, kind="stable")
    c = np.cumsum(p[idx])
    drop = c <= 1.0 - top_p
    drop[-1] = False
    mask = np.ones_like(p, dtype=bool)
    mask[idx[drop]] = False
    return mask


@pytest.mark.parametrize("top_p", [0.05, 0.3, 0.5, 0.8, 0.95, 0.999])
def test_top_p_matches_the_ascending_formulation(top_p):
    rng = np.random.default_rng(int(top_p * 1000))
    for _ in range(20):
        s = rng.standard_normal(64) * 2
        mask, margin = ot.keep(s, 0, top_p)
        if margin < 1e-9:
            continue            # a boundary tie: the two formulations may differ
        assert np.array_equal(mask, _top_p_ascending(s, top_p))
        kept = sp_softmax(s)[mask].sum()
        assert kept >= top_p - 1e-12
        # minimal: the smallest kept token takes the mass below top_p
        assert kept - sp_softmax(s)[mask].min() < top_p


def test_top_k_then_top_p_uses_the_top_k_mass():
    s = np.log(np.array([0.4, 0.3, 0.2, 0.1]))
    # top-k = 2 keeps 0.4, 0.3 (renormalised 4/7, 3/7); top-p 0.5 of that
    # keeps only the first (4/7 >= 0.5)
    mask, _ = ot.keep(s, 2, 0.5)
    assert list(mask) == [True, False, False, False]
    mask, _ = ot.keep(s, 0, 0.5)            # without top-k: 0.4 < 0.5, keep two
    assert list(mask) == [True, True, False, False]


def test_equal_logits_kept_in_token_order():
    s = np.array([1.0, 2.0, 2.0, 2.0, 0.5])
    mask, _ = ot.keep(s, 2, 1.0)
    assert list(mask) == [False, True, True, False, False]


def test_bad_top_p_faults_the_request():
    t = np.zeros((2, 5), np.float32)
    d = np.zeros((1, 5), np.float32)
    for top_p in (0.0, -0.5, np.nan):
        out = ov.verify_request(t, d, np.array([1]), 1, 1.0, 0, 0, 1, top_p=top_p)
        assert out["status"] == ov.STATUS_BAD_TRUNCATION and out["accepted_len"] == -1


@pytest.mark.parametrize("top_k,top_p", [(2, 1.0), (0, 0.6), (3, 0.7)])
def test_emitted_law_is_the_truncated_target(top_k, top_p):
    """Exact enumeration through the verify step: y over the truncated q,
    the accept and draw uniforms over a lattice. The emitted token's law must
    be the truncated p."""
    rng = np.random.default_rng(7 + top_k)
    V = 5
    t = rng.standard_normal((2, V)).astype(np.float32)
    d = (t[:1] + rng.standard_normal((1, V))).astype(np.float32)
    p, _, _, _ = ot.truncated_softmax(t[0].astype(np.float64), top_k, top_p)
    q, _, _, _ = ot.truncated_softmax(d[0].astype(np.float64), top_k, top_p)
    law = np.zeros(V)
    for y in range(V):
        if q[y] == 0:
            continue
        acc = 0
        for u in _lattice():
            out = ov.verify_request(t, d, np.array([y]), 1, 1.0, 0, 0, 1,
                                    uniforms=lambda s, b, k, u=u: (u, 0.5),
                                    top_k=top_k, top_p=top_p)
            acc += out["accepted_len"] == 1
        p_acc = acc / LATTICE
        law[y] += q[y] * p_acc
        draws = np.zeros(V)
        for u2 in _lattice():
            out = ov.verify_request(t, d, np.array([y]), 1, 1.0, 0, 0, 1,
                                    uniforms=lambda s, b, k, u2=u2: (1 - 2.0**-24, u2),
                                    top_k=top_k, top_p=top_p)
            if out["accepted_len"] == 0:
                draws[out["tokens"][0]] += 1
        if 1 - p_acc > 0:
            law += q[y] * (1 - p_acc) * draws / LATTICE
    assert np.allclose(law, p, atol=4.0 / LATTICE)
