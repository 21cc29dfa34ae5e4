"""Pins of the oracle's verify step against what the pages and the
mathematics fix (identities, closed forms, exact enumeration, the worked
examples, chi-square tests and the greedy limit). None of these calls the
product path."""

import json
import os

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax
from scipy.stats import chisquare

from oracle import verify as ov

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _req(t_rows, d_rows, y, temperature=1.0, seed=0, b=0, k_b=None, uniforms=None):
    t_rows = np.asarray(t_rows, dtype=np.float32)
    d_rows = np.asarray(d_rows, dtype=np.float32)
    kmax = d_rows.shape[0]
    k_b = kmax if k_b is None else k_b
    return ov.verify_request(t_rows, d_rows, np.asarray(y), k_b, temperature,
                             seed, b, kmax, uniforms=uniforms)


def _probs(rows, temperature=1.0):
    """Reference softmax through scipy of the fp32-scaled logits."""
    s = (np.asarray(rows, dtype=np.float32) *
         (np.float32(1.0) / np.float32(temperature))).astype(np.float64)
    return sp_softmax(s, axis=-1)


# ---------------------------------------------------------------- softmax / alpha

def test_softmax_matches_scipy():
    rng = np.random.default_rng(0)
    s = rng.standard_normal(1000) * 5
    p, m, total = ov.softmax64(s)
    assert np.allclose(p, sp_softmax(s), rtol=1e-13, atol=0)
    assert m == s.max()


@pytest.mark.parametrize("temperature", [1.0, 0.6, 1.7])
def test_alpha_is_one_minus_tv(temperature):
    rng = np.random.default_rng(1)
    K, V = 3, 500
    t = rng.standard_normal((K + 1, V)) * 2
    d = t[:K] + rng.standard_normal((K, V))
    out = _req(t, d, np.zeros(K, int), temperature=temperature)
    p, q = _probs(t, temperature), _probs(d, temperature)
    for k in range(K):
        tv = 0.5 * np.sum(np.abs(p[k] - q[k]))
        assert out["alpha"][k] == pytest.approx(1 - tv, rel=1e-12, abs=1e-14)
        assert out["alpha"][k] + out["residual"][k] == pytest.approx(1.0, abs=1e-12)


def test_alpha_is_expected_acceptance_probability():
    # alpha = E_{y~q}[min(1, p(y)/q(y))], enumerated over every y
    rng = np.random.default_rng(2)
    V = 40
    t = rng.standard_normal((2, V))
    d = t[:1] + 0.7 * rng.standard_normal((1, V))
    out = _req(t, d, [0])
    p, q = _probs(t)[0], _probs(d)[0]
    expect = sum(q[y] * min(1.0, p[y] / q[y]) for y in range(V))
    assert out["alpha"][0] == pytest.approx(expect, rel=1e-12)


def test_alpha_special_cases():
    V = 16
    rng = np.random.default_rng(3)
    t = rng.standard_normal((2, V)).astype(np.float32)
    same = _req(t, t[:1], [0])
    assert same["alpha"][0] == pytest.approx(1.0, abs=1e-14)
    # disjoint supports
    t2 = np.full((2, 4), -np.inf, np.float32)
    t2[:, :2] = 0.0
    d2 = np.full((1, 4), -np.inf, np.float32)
    d2[0, 2:] = 0.0
    dis = _req(t2, d2, [2])
    assert dis["alpha"][0] == 0.0
    assert dis["status"] == 0


@pytest.mark.parametrize("x,y", [(0.7, 0.5), (0.2, 0.9), (0.5, 0.5), (0.99, 0.01)])
def test_alpha_two_token_closed_form(x, y):
    # q = (x, 1-x), p = (y, 1-y)  =>  alpha = 1 - |x - y|
    d = np.array([[0.0, np.log((1 - x) / x)]], np.float32)
    t = np.array([[0.0, np.log((1 - y) / y)], [0.0, 0.0]], np.float32)
    xh = 1.0 / (1.0 + np.exp(np.float64(d[0, 1]) - np.float64(d[0, 0])))
    yh = 1.0 / (1.0 + np.exp(np.float64(t[0, 1]) - np.float64(t[0, 0])))
    out = _req(t, d, [0])
    assert out["alpha"][0] == pytest.approx(1 - abs(xh - yh), rel=1e-12)


# ---------------------------------------------------------------- accept / draw rules

LATTICE = 4096        # u = (i + 0.5) / LATTICE, exactly representable


def _lattice():
    return (np.arange(LATTICE) + 0.5) / LATTICE


def test_accept_rule_threshold_on_the_24_bit_lattice():
    # accept iff u < p/q: on the lattice of 24-bit uniforms the accepted count
    # is exactly ceil(r * 2^24)
    for r in [0.0, 1e-7, 0.3, 0.5, 0.75, 0.999999, 1.0, 2.5]:
        p_y, q_y = r * 0.25, 0.25
        ratio = p_y / q_y
        n_acc = int(np.ceil(min(ratio, 1.0) * 2**24))
        # the threshold point and its neighbours
        for i in [n_acc - 1, n_acc, n_acc + 1]:
            if 0 <= i < 2**24:
                ok, _ = ov.accept(i * 2.0**-24, p_y, q_y)
                assert ok == (i < n_acc)
    assert ov.accept(0.0, 0.0, 0.0)[0] is False      # q = 0, p = 0: reject
    assert ov.accept(0.999, 1e-30, 0.0)[0] is True    # q = 0, p > 0: accept


def test_draw_counts_on_the_24_bit_lattice():
    rng = np.random.default_rng(4)
    w = rng.random(7)
    w[0] = 0.0            # a zero weight first: "smallest v with C[v] > target"
    w[2] = 0.0
    u = np.arange(2**24, dtype=np.float64) * 2.0**-24
    counts = np.bincount(ov.draw(u, w), minlength=len(w))
    expect = w / w.sum() * 2**24
    assert counts[0] == 0 and counts[2] == 0
    assert np.all(np.abs(counts - expect) <= 1.0)


def test_single_position_law_rebuilds_target():
    """Exact enumeration through the oracle's own code path: y over the
    vocabulary with weight q(y), the accept uniform and the draw uniform over
    a lattice. The emitted-token law must be p (accept mass min(p, q) plus
    reject mass max(0, p - q))."""
    rng = np.random.default_rng(5)
    V = 3
    t = rng.standard_normal((2, V)).astype(np.float32)
    d = (t[:1] + rng.standard_normal((1, V))).astype(np.float32)
    p, q = _probs(t)[0], _probs(d)[0]
    lat = _lattice()
    law = np.zeros(V)
    for y in range(V):
        acc = 0
        for u in lat:
            out = _req(t, d, [y], uniforms=lambda s, b, k, u=u: (u, 0.5))
            acc += out["accepted_len"] == 1
        p_acc = acc / LATTICE
        law[y] += q[y] * p_acc
        draws = np.zeros(V)
        for u2 in lat:
            out = _req(t, d, [y], uniforms=lambda s, b, k, u2=u2: (1 - 2.0**-24, u2))
            if out["accepted_len"] == 0:
                draws[out["tokens"][0]] += 1
        if (1 - p_acc) > 0:
            law += q[y] * (1 - p_acc) * draws / LATTICE
    assert np.allclose(law, p, atol=4.0 / LATTICE)


def test_scan_stops_at_first_rejection():
    rng = np.random.default_rng(6)
    K, V = 4, 30
    t = rng.standard_normal((K + 1, V)).astype(np.float32)
    d = (t[:K] + rng.standard_normal((K, V))).astype(np.float32)
    y = [3, 4, 5, 6]
    # force accept at 0, reject at 1 (u = 1 - 2^-24 rejects unless p/q >= 1 - 2^-24)
    p, q = _probs(t), _probs(d)

    def forced(s, b, k):
        return (0.0, 0.25) if k != 1 else (1 - 2.0**-24, 0.25)
    out = _req(t, d, y, uniforms=forced)
    if p[1][4] / q[1][4] < 1 - 2.0**-24:
        assert out["accepted_len"] == 1
        assert out["tokens"][0] == 3
        assert out["tokens"][1] != -1 and out["tokens"][2] == -1
        assert p[1][out["tokens"][1]] > q[1][out["tokens"][1]]
        assert np.isnan(out["accept_margin"][2])
    # alpha is reported for every position, also after the rejection
    for k in range(K):
        assert out["alpha"][k] == pytest.approx(np.minimum(p[k], q[k]).sum(), rel=1e-12)


# ---------------------------------------------------------------- statistics

def test_chi_square_emitted_law_two_positions():
    """y_k ~ q_k fresh per trial, Philox seeds vary. The first emitted token is
    distributed as p_0; given a first accept the next is distributed as p_1;
    P(accepted_len >= j) = prod_{k<j} alpha_k."""
    rng = np.random.default_rng(7)
    V, K, trials = 8, 2, 20000
    t = (1.5 * rng.standard_normal((K + 1, V))).astype(np.float32)
    d = (t[:K] + rng.standard_normal((K, V))).astype(np.float32)
    p, q = _probs(t), _probs(d)
    first = np.zeros(V)
    second = np.zeros(V)
    bonus = np.zeros(V)
    ge1 = ge2 = 0
    alpha = None
    for s in range(trials):
        y = [rng.choice(V, p=q[0]), rng.choice(V, p=q[1])]
        out = _req(t, d, y, seed=s, b=s % 5)
        alpha = out["alpha"]
        first[out["tokens"][0]] += 1
        if out["accepted_len"] >= 1:
            ge1 += 1
            second[out["tokens"][1]] += 1
        if out["accepted_len"] == 2:
            ge2 += 1
            bonus[out["tokens"][2]] += 1
    assert chisquare(first, p[0] * trials).pvalue > 1e-3
    assert chisquare(bonus, p[2] * bonus.sum()).pvalue > 1e-3
    assert chisquare(second, p[1] * second.sum()).pvalue > 1e-3
    for count, prob in [(ge1, alpha[0]), (ge2, alpha[0] * alpha[1])]:
        sd = np.sqrt(trials * prob * (1 - prob))
        assert abs(count - trials * prob) < 5 * sd


def test_plain_sampling_when_k_is_zero():
    # K_b = 0: one token drawn from p_0
    rng = np.random.default_rng(8)
    V, trials = 12, 20000
    t = (2 * rng.standard_normal((1, V))).astype(np.float32)
    d = np.zeros((1, V), np.float32)
    p = _probs(t)[0]
    counts = np.zeros(V)
    for s in range(trials):
        out = ov.verify_request(t, d, np.array([-1]), 0, 1.0, s, 3, 1)
        assert out["accepted_len"] == 0
        counts[out["tokens"][0]] += 1
    assert chisquare(counts, p * trials).pvalue > 1e-3


def _two_token_rows(alphas):
    """Target p = (0.5, 0.5); draft q = (x, 1 - x) with x = 1.5 - alpha gives
    sum min(p, q) = alpha."""
    K = len(alphas)
    t = np.zeros((K + 1, 2), np.float32)
    d = np.zeros((K, 2), np.float32)
    for k, a in enumerate(alphas):
        x = 1.5 - a
        d[k] = [np.log(x), np.log(1 - x)]
    return t, d


@pytest.mark.parametrize("example", json.load(open(GOLDEN))["expected_emitted"])
def test_worked_expected_emitted_length(example):
    alphas = example["alphas"]
    assert ov.expected_emitted(alphas) == pytest.approx(example["expected_emitted"], abs=1e-12)
    t, d = _two_token_rows(alphas)
    q = _probs(d)
    rng = np.random.default_rng(9)
    trials = 20000
    emitted = np.empty(trials)
    alpha_hat = None
    for s in range(trials):
        y = [rng.choice(2, p=q[k]) for k in range(len(alphas))]
        out = _req(t, d, y, seed=s, b=s % 7)
        emitted[s] = out["accepted_len"] + 1
        alpha_hat = out["alpha"]
    assert np.allclose(alpha_hat, alphas, atol=1e-6)
    se = emitted.std() / np.sqrt(trials)
    assert abs(emitted.mean() - example["expected_emitted"]) < 5 * se
    assert abs(emitted.mean() - ov.expected_emitted(alpha_hat)) < 5 * se


def test_speed_model_example():
    sm = json.load(open(GOLDEN))["speed_model"]
    speed = sm["expected_emitted"] * sm["t_ar_ms"] / (
        sm["t_draft_ms"] + sm["t_verify_ms"] + sm["t_overhead_ms"])
    assert speed == pytest.approx(sm["speedup_approx"], abs=0.01)
    slow = sm["expected_emitted"] * sm["t_ar_ms"] / (
        sm["t_draft_ms"] + sm["t_verify_no_gain_ms"] + sm["t_overhead_ms"])
    assert slow == pytest.approx(1.0, abs=0.05)


def test_residual_support_invariant():
    rng = np.random.default_rng(10)
    V, K = 50, 3
    t = (2 * rng.standard_normal((K + 1, V))).astype(np.float32)
    d = (t[:K] + 1.5 * rng.standard_normal((K, V))).astype(np.float32)
    p, q = _probs(t), _probs(d)
    seen = 0
    for s in range(400):
        y = [rng.choice(V, p=q[k]) for k in range(K)]
        out = _req(t, d, y, seed=s)
        j = out["accepted_len"]
        v = out["tokens"][j]
        if j < K:
            assert p[j][v] > q[j][v]
            seen += 1
        else:
            assert p[K][v] > 0
    assert seen > 50


# ---------------------------------------------------------------- greedy

def test_greedy_is_the_low_temperature_limit():
    """T = 0 compares with the target argmax. At T = 1e-3 on rows whose top
    gap is >= 0.05, p and q are one-hot in fp64 and the stochastic path must
    emit exactly what the greedy rule emits."""
    rng = np.random.default_rng(11)
    V, K = 64, 4
    checked = 0
    for trial in range(60):
        t = rng.standard_normal((K + 1, V)).astype(np.float32)
        d = (t[:K] + 0.8 * rng.standard_normal((K, V))).astype(np.float32)
        rows = np.concatenate([t, d])
        top2 = np.sort(rows, axis=1)[:, -2:]
        if np.any(top2[:, 1] - top2[:, 0] < 0.05):
            continue
        # a greedy drafter proposes its own argmax; the limit argument needs it
        y = [int(np.argmax(d[k])) for k in range(K)]
        g = _req(t, d, y, temperature=0.0)
        s = _req(t, d, y, temperature=1e-3, seed=trial)
        assert g["greedy"] and not s["greedy"]
        assert g["accepted_len"] == s["accepted_len"]
        assert np.array_equal(g["tokens"], s["tokens"])
        assert np.allclose(g["alpha"], s["alpha"], atol=1e-12)
        # literal rule: accept while y_k is the target argmax
        j = next((k for k in range(K) if y[k] != np.argmax(t[k])), K)
        assert g["accepted_len"] == j and g["tokens"][j] == np.argmax(t[j])
        checked += 1
    assert checked > 20


def test_greedy_literal_rule_with_arbitrary_tokens():
    rng = np.random.default_rng(13)
    V, K = 32, 5
    for _ in range(50):
        t = rng.standard_normal((K + 1, V)).astype(np.float32)
        d = rng.standard_normal((K, V)).astype(np.float32)
        g_t = np.argmax(t, axis=1)
        y = [int(g_t[k]) if rng.random() < 0.8 else int(rng.integers(V)) for k in range(K)]
        out = _req(t, d, y, temperature=0.0)
        j = 0
        while j < K and y[j] == g_t[j]:
            j += 1
        assert out["accepted_len"] == j
        assert list(out["tokens"][:j]) == y[:j] and out["tokens"][j] == g_t[j]
        assert np.all(out["tokens"][j + 1:] == -1)
        assert np.array_equal(out["alpha"], (g_t[:K] == np.argmax(d, axis=1)).astype(float))


def test_greedy_argmax_ties_take_lowest_index():
    t = np.array([[1.0, 3.0, 3.0, 0.0], [2.0, 2.0, 1.0, 0.0]], np.float32)
    d = np.array([[0.0, 5.0, 5.0, 1.0]], np.float32)
    out = _req(t, d, [2], temperature=0.0)
    assert out["accepted_len"] == 0 and out["tokens"][0] == 1
    out = _req(t, d, [1], temperature=0.0)
    assert out["accepted_len"] == 1 and out["tokens"][1] == 0
    assert out["alpha"][0] == 1.0


# ---------------------------------------------------------------- faults and padding

def test_status_bits():
    V, K = 10, 3
    t = np.zeros((K + 1, V), np.float32)
    d = np.zeros((K, V), np.float32)
    kmax = K
    bad_k = ov.verify_request(t, d, np.array([0, 0, 0]), 4, 1.0, 0, 0, kmax)
    assert bad_k["status"] == ov.STATUS_BAD_K and bad_k["accepted_len"] == -1
    bad_tok = ov.verify_request(t, d, np.array([0, V, 0]), 3, 1.0, 0, 0, kmax)
    assert bad_tok["status"] == ov.STATUS_BAD_TOKEN
    # tokens beyond K_b are not checked
    ok = ov.verify_request(t, d, np.array([0, V, -5]), 1, 1.0, 0, 0, kmax)
    assert ok["status"] == 0
    for temp in [-1.0, np.nan, np.inf]:
        r = ov.verify_request(t, d, np.array([0, 0, 0]), 3, temp, 0, 0, kmax)
        assert r["status"] == ov.STATUS_BAD_TEMPERATURE
        assert np.all(r["tokens"] == -1) and np.all(r["alpha"] == 0)
    nan_t = t.copy()
    nan_t[2, 5] = np.nan
    assert ov.verify_request(nan_t, d, np.array([0, 0, 0]), 3, 1.0, 0, 0, kmax)["status"] == 8
    # the NaN row is not used when K_b = 1
    assert ov.verify_request(nan_t, d, np.array([0, 0, 0]), 1, 1.0, 0, 0, kmax)["status"] == 0
    inf_d = d.copy()
    inf_d[0, 1] = np.inf
    assert ov.verify_request(t, inf_d, np.array([0, 0, 0]), 3, 0.0, 0, 0, kmax)["status"] == 8
    ninf = np.full_like(t, -np.inf)
    assert ov.verify_request(ninf, d, np.array([0, 0, 0]), 2, 1.0, 0, 0, kmax)["status"] == 8
    # overflow of the scaled logit is a fault too
    big = t.copy()
    big[0, 0] = 3e38
    assert ov.verify_request(big, d, np.array([0, 0, 0]), 2, 0.5, 0, 0, kmax)["status"] == 8


def test_alpha_zero_beyond_k():
    rng = np.random.default_rng(12)
    V, K = 20, 4
    t = rng.standard_normal((K + 1, V)).astype(np.float32)
    d = (t[:K] + rng.standard_normal((K, V))).astype(np.float32)
    out = ov.verify_request(t, d, np.array([1, 2, -1, -1]), 2, 1.0, 0, 0, K)
    assert np.all(out["alpha"][2:] == 0) and np.all(out["alpha"][:2] > 0)
    assert np.all(out["tokens"][out["accepted_len"] + 1:] == -1)


def test_scaling_is_binary32():
    x = np.array([1.1, -3.3, 7.25, 1e-3], np.float32)
    s = ov.scale(x, 0.6)
    inv = np.float32(1) / np.float32(0.6)
    assert s.dtype == np.float32
    assert np.array_equal(s, x * inv)
    assert np.array_equal(ov.scale(x, 1.0), x)


def test_batched_matches_per_request():
    from lossless_verify_tv_amd import synth
    case = synth.verify_case(3, temperature=1.0, batch=4, kmax=3, vocab=300)
    res = ov.spec_verify(case.target, case.draft, case.dtype, case.tokens,
                         case.k, case.temperature, case.seed)
    for b in range(4):
        one = ov.verify_request(ov.decode_rows(case.target[b], "bf16"),
                                ov.decode_rows(case.draft[b], "bf16"),
                                case.tokens[b], case.k[b], 1.0, 0, b, 3)
        assert res["accepted_len"][b] == one["accepted_len"]
        assert np.array_equal(res["tokens"][b], one["tokens"])
