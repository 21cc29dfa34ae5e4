"""Pins of the decision margins the parity rules excuse mismatches by, and of
the scheduler's NaN-throughput reading.

Every excused GPU/oracle mismatch rests on a margin the oracle reports: the
accept margin |u - p/q| ("Reading Qwen Bebop and DeepSeek DSpark",
"Formulas", eq. alpha(y): accept with probability min(1, p/q)), the
inverse-CDF margin of a draw, normalised by the total weight ("Speculative
Decoding and MTP" survey, section 3: the correction is drawn from
max(0, p - q)/Z), and the top-p margin, normalised by the kept total
(survey, section 4). Each is checked here on hand-built cases whose
probabilities, cumulative weights and margins are exact binary fractions,
worked out by hand in the comments, so a margin measured on the wrong side,
against the wrong total or without its normalisation fails one of them."""

import numpy as np
import pytest

from oracle import schedule as osch
from oracle import truncate as ot
from oracle import verify as ov

Q = 2.0 ** -24  # spacing of the 24-bit uniform lattice


# ---------------------------------------------------------------- accept margin

@pytest.mark.parametrize("p_y,q_y,u,accepted,margin", [
    # r = p/q = 0.5
    (0.25, 0.5, 0.5 - 3 * Q, True, 3 * Q),
    (0.25, 0.5, 0.5 + 5 * Q, False, 5 * Q),
    (0.25, 0.5, 0.5, False, 0.0),          # strict test: u == p/q rejects
    # r = 0.75 / 0.25 = 3 > 1: every u accepts, margin 3 - u
    (0.75, 0.25, 1.0 - Q, True, 2.0 + Q),
    # r = 0: always rejects, margin u
    (0.0, 0.5, 0.125, False, 0.125),
])
def test_accept_margin_exact(p_y, q_y, u, accepted, margin):
    ok, m = ov.accept(u, p_y, q_y)
    assert ok is accepted
    assert m == margin


def test_accept_margin_infinite_when_q_is_zero():
    assert ov.accept(0.5, 0.25, 0.0) == (True, np.inf)
    assert ov.accept(0.5, 0.0, 0.0) == (False, np.inf)


def _two_token_request(u_accept, u_draw):
    """K = 2, V = 2. Target rows (0, 0): p = (1/2, 1/2) exactly. Draft row 0
    (0, -inf): q_0 = (1, 0); draft row 1 (0, 0): q_1 = (1/2, 1/2). Draft
    tokens (0, 0), so r_0 = p_0(0)/q_0(0) = 1/2 and r_1 = 1."""
    t = np.zeros((3, 2), np.float32)
    d = np.array([[0.0, -np.inf], [0.0, 0.0]], np.float32)

    def uniforms(seed, b, k):
        return u_accept[k], u_draw[k]
    return ov.verify_request(t, d, np.array([0, 0]), 2, 1.0, 0, 0, 2, uniforms=uniforms)


def test_request_reports_accept_margins_up_to_the_first_rejection():
    # accepted at 0 (u = 1/2 - 2^-20 < 1/2) and at 1 (u < 1): margins
    # 2^-20 and 1 - (1 - 2^-24) = 2^-24; the bonus comes from p_2
    out = _two_token_request([0.5 - 2.0 ** -20, 1.0 - Q, 0.0], [0.0, 0.0, 0.75])
    assert out["accepted_len"] == 2
    assert out["accept_margin"][0] == 2.0 ** -20
    assert out["accept_margin"][1] == Q
    # rejected at 0 (u = 1/2 + 2^-22): margin 2^-22, no decision at 1
    out = _two_token_request([0.5 + 2.0 ** -22, 0.0, 0.0], [0.25, 0.0, 0.0])
    assert out["accepted_len"] == 0
    assert out["accept_margin"][0] == 2.0 ** -22
    assert np.isnan(out["accept_margin"][1])


def test_request_draw_margin_is_normalised_by_the_residual_total():
    # rejected at 0: residual max(0, p_0 - q_0) = (0, 1/2), cumulative
    # (0, 1/2), target u' / 2. Token 1 is drawn for every u'; the margin is
    # min(u'/2 - 0, 1/2 - u'/2) / (1/2) = min(u', 1 - u')
    out = _two_token_request([0.5 + Q, 0.0, 0.0], [0.25, 0.0, 0.0])
    assert out["tokens"][0] == 1
    assert out["draw_margin"] == 0.25
    out = _two_token_request([0.5 + Q, 0.0, 0.0], [1.0 - 2.0 ** -10, 0.0, 0.0])
    assert out["draw_margin"] == 2.0 ** -10
    # bonus draw from p_2 = (1/2, 1/2): cumulative (1/2, 1), target u'. At
    # u' = 3/8 token 0, margin min(3/8, 1/2 - 3/8) / 1 = 1/8; at u' = 5/8
    # token 1, margin min(5/8 - 1/2, 1 - 5/8) = 1/8
    out = _two_token_request([0.0, 0.0, 0.0], [0.0, 0.0, 0.375])
    assert (out["accepted_len"], out["tokens"][2], out["draw_margin"]) == (2, 0, 0.125)
    out = _two_token_request([0.0, 0.0, 0.0], [0.0, 0.0, 0.625])
    assert (out["accepted_len"], out["tokens"][2], out["draw_margin"]) == (2, 1, 0.125)


# ---------------------------------------------------------------- draw margin

@pytest.mark.parametrize("u,token,margin", [
    # weights (1, 2, 1): cumulative (1, 3, 4), total 4, target 4u
    (0.5, 1, 0.25),                        # target 2: min(2 - 1, 3 - 2) / 4
    (0.25 + 2.0 ** -10, 1, 2.0 ** -10),    # just past the boundary at C = 1
    (0.25 - 2.0 ** -10, 0, 2.0 ** -10),    # just before it
    (0.25, 1, 0.0),                        # on it: the first C[v] > target
    (0.75 - 2.0 ** -12, 1, 2.0 ** -12),    # just before the boundary at C = 3
    (0.75 + 2.0 ** -12, 2, 2.0 ** -12),
    (0.0, 0, 0.0),
    (1.0 - Q, 2, Q),
])
def test_draw_margin_exact(u, token, margin):
    v, m = ov.draw(u, np.array([1.0, 2.0, 1.0]))
    assert v == token
    assert m == margin


def test_draw_margin_skips_zero_weights():
    # weights (0, 1, 0, 3): cumulative (0, 1, 1, 4). Target 4u = 1.5 lies in
    # token 3's interval [1, 4): margin min(1.5 - 1, 4 - 1.5) / 4 = 1/8; a
    # zero-weight token never bounds the interval from below
    v, m = ov.draw(0.375, np.array([0.0, 1.0, 0.0, 3.0]))
    assert (v, m) == (3, 0.125)


# ---------------------------------------------------------------- top-p margin

@pytest.mark.parametrize("top_p,kept,margin", [
    # four equal weights: cumulative (1, 2, 3, 4), total 4, target 4 top_p;
    # the kept prefix is the shortest whose cumulative weight reaches it
    (0.5 + 2.0 ** -6, 3, 2.0 ** -6),   # target 2 + 1/16: min(3 - t, t - 2) / 4
    (0.5 - 2.0 ** -6, 2, 2.0 ** -6),   # target 2 - 1/16: min(2 - t, t - 1) / 4
    (0.5, 2, 0.0),                     # exactly reached
    (0.125, 1, 0.125),                 # target 1/2: min(1 - 1/2, 1/2 - 0) / 4
])
def test_top_p_margin_exact(top_p, kept, margin):
    mask, m = ot.keep(np.zeros(4), 0, top_p)
    assert int(mask.sum()) == kept
    assert m == margin


def test_top_p_margin_is_normalised_by_the_top_k_total():
    # six equal logits, top-k 4 keeps tokens 0..3 (total 4, not 6); top-p
    # 0.5 + 2^-6 then keeps 3 of them with margin (1/16) / 4
    mask, m = ot.keep(np.zeros(6), 4, 0.5 + 2.0 ** -6)
    assert np.array_equal(np.flatnonzero(mask), [0, 1, 2])
    assert m == 2.0 ** -6


def test_top_p_margin_with_unequal_weights():
    # s = ln w with w = (1, 1/2, 1/4, 1/4) (exp(s - max s) gives w back up
    # to the log/exp round trip, hence the 1e-15 tolerance): cumulative
    # (1, 3/2, 7/4, 2), total 2; top_p 0.8 -> target 1.6, kept 3 (7/4 >=
    # 1.6), margin min(7/4 - 1.6, 1.6 - 3/2) / 2 = 0.05
    s = np.log(np.array([1.0, 0.5, 0.25, 0.25]))
    mask, m = ot.keep(s, 0, 0.8)
    assert np.array_equal(np.flatnonzero(mask), [0, 1, 2])
    assert m == pytest.approx(0.05, abs=1e-15)


def test_request_reports_the_closest_top_p_decision():
    # one position, V = 4, T = 1, top-p 0.5 + 2^-6 on four equal logits in
    # every row: each row's margin is 2^-6 (as above), so the request's too
    t = np.zeros((2, 4), np.float32)
    d = np.zeros((1, 4), np.float32)
    out = ov.verify_request(t, d, np.array([0]), 1, 1.0, 0, 0, 1, top_p=0.5 + 2.0 ** -6)
    assert out["trunc_margin"] == 2.0 ** -6


# ---------------------------------------------------------------- scheduler: NaN throughput

def test_schedule_never_picks_a_nan_throughput():
    # R = 2, L = 2, every confidence 1: the survivals are all 1, so verifying
    # B - R tokens yields tau = B and Theta(B) = B SPS(B). With SPS = 1 at
    # B = 2, 3, 5, NaN at B = 4 and 1/2 at B = 6: Theta = 2, 3, NaN, 5, 3.
    # B = 5 is the best number; a NaN at B = 4 must not win.
    conf = np.ones((2, 2), np.float32)
    sps = np.array([0, 0, 1.0, 1.0, np.nan, 1.0, 0.5])
    lens, best, B, theta = osch.schedule(conf, sps)
    assert B == 5
    assert best == 5.0
    assert int(lens.sum()) == 3
    assert np.array_equal(lens, [2, 1])   # equal survivals in flat index order


def test_schedule_all_nan_throughputs_verify_nothing():
    conf = np.full((3, 2), 0.5, np.float32)
    sps = np.full(3 * 3 + 1, np.nan)
    lens, best, B, _ = osch.schedule(conf, sps)
    assert B == 3
    assert np.array_equal(lens, [0, 0, 0])
