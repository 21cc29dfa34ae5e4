"""Pins of the oracle's comparator objectives (per-step TV, CE, KL): the
one-hot case of CE (the log loss, by scipy's logsumexp and softmax), KL = 0 at
q = p and KL = CE - H(p) (scipy's entropy), Gibbs' inequality, the per-step
TV loss as half the L1 distance and its W = 1 agreement with the E2E-TV
loss, the two-token closed forms, and central finite differences of every
gradient with unnormalised target probabilities. None of these calls the
product path."""

import numpy as np
import pytest
from scipy.special import logsumexp, softmax
from scipy.stats import entropy

from oracle import bf16
from oracle import loss as ol
from oracle import objectives as ob


def _rand(rng, W, V, normalised=True, gap=1e-4):
    """fp64 logits and probabilities with |q - p| >= gap everywhere."""
    while True:
        z = rng.standard_normal((W, V))
        p = np.exp(rng.standard_normal((W, V)))
        p /= p.sum(-1, keepdims=True)
        if not normalised:
            p *= rng.uniform(0.5, 1.5, size=(W, 1))
        q = np.exp(z - z.max(-1, keepdims=True))
        q /= q.sum(-1, keepdims=True)
        if np.min(np.abs(q - p)) > gap:
            return z, p


def test_ce_one_hot_is_log_loss():
    rng = np.random.default_rng(10)
    W, V = 3, 50
    z = rng.standard_normal((W, V)) * 2
    y = rng.integers(0, V, size=W)
    p = np.zeros((W, V))
    p[np.arange(W), y] = 1.0
    loss_n, _, dz = ob.branch(z, p, 1, "ce")
    assert loss_n == pytest.approx(sum(logsumexp(z[k]) - z[k, y[k]] for k in range(W)), rel=1e-13)
    expect = softmax(z, axis=1) - p
    assert np.allclose(dz, expect, rtol=1e-12, atol=1e-15)
    # N branches: the gradient carries 1/N
    assert np.allclose(ob.branch(z, p, 4, "ce")[2], expect / 4, rtol=1e-12, atol=1e-16)


def test_kl_vanishes_at_q_equal_p():
    rng = np.random.default_rng(11)
    p = np.exp(rng.standard_normal((2, 40)))
    p /= p.sum(-1, keepdims=True)
    z = np.log(p) + 3.0                      # softmax(z) = p
    loss_n, alpha, dz = ob.branch(z, p, 1, "kl")
    assert abs(loss_n) < 1e-13
    assert np.allclose(alpha, 1.0, atol=1e-13)
    assert np.max(np.abs(dz)) < 1e-15


def test_kl_is_ce_minus_entropy_and_nonnegative():
    rng = np.random.default_rng(12)
    for _ in range(5):
        z, p = _rand(rng, 4, 30, gap=0)
        p[0, :3] = 0.0                        # zero entries: p log p = 0
        p[0] /= p[0].sum()
        ce = ob.branch(z, p, 1, "ce")[0]
        kl = ob.branch(z, p, 1, "kl")[0]
        h = sum(entropy(p[k]) for k in range(4))
        assert kl == pytest.approx(ce - h, rel=1e-12, abs=1e-12)
        q = softmax(z, axis=1)
        assert kl == pytest.approx(sum(entropy(p[k], q[k]) for k in range(4)), rel=1e-11)
        assert kl >= 0.0


def test_step_tv_is_half_l1_and_matches_e2e_at_one_position():
    rng = np.random.default_rng(13)
    z, p = _rand(rng, 5, 60)
    loss_n, alpha, _ = ob.branch(z, p, 1, "step_tv")
    q = softmax(z, axis=1)
    assert loss_n == pytest.approx(0.5 * np.abs(q - p).sum(), rel=1e-12)
    assert np.allclose(alpha, 1.0 - 0.5 * np.abs(q - p).sum(-1), atol=1e-13)
    # W = 1: the E2E-TV loss is -alpha = L_TV - 1, with the same gradient
    l1, _, dz1 = ob.branch(z[:1], p[:1], 3, "step_tv")
    le, _, _, _, dze = ol.branch(z[:1], p[:1], 3)
    assert l1 == pytest.approx(le + 1.0, abs=1e-13)
    assert np.allclose(dz1, dze, rtol=1e-13, atol=1e-17)


@pytest.mark.parametrize("x_logit,a,b", [(1.0, 0.3, 0.5), (-0.7, 0.6, 0.6), (0.2, 0.1, 0.95)])
def test_two_token_closed_forms(x_logit, a, b):
    # q = (s, 1 - s), s = sigmoid(z0 - z1); p = (a, b), not normalised.
    z = np.array([[x_logit, 0.0]])
    p = np.array([[a, b]])
    s = 1.0 / (1.0 + np.exp(-x_logit))
    ce, _, dce = ob.branch(z, p, 1, "ce")
    assert ce == pytest.approx(-a * np.log(s) - b * np.log(1 - s), rel=1e-13)
    # d/dz0 [-a log s - b log(1 - s)] = -a (1 - s) + b s
    assert dce[0, 0] == pytest.approx(-a * (1 - s) + b * s, rel=1e-12)
    assert dce[0, 1] == pytest.approx(a * (1 - s) - b * s, rel=1e-12)
    kl, _, dkl = ob.branch(z, p, 1, "kl")
    assert kl == pytest.approx(a * np.log(a / s) + b * np.log(b / (1 - s)), rel=1e-12)
    assert np.allclose(dkl, dce, rtol=1e-14)
    tv, _, dtv = ob.branch(z, p, 1, "step_tv")
    assert tv == pytest.approx(1.0 - min(s, a) - min(1 - s, b), rel=1e-13)
    # d(1 - alpha)/dz0 = -(d/dz0)(min(s, a) + min(1 - s, b)), ds/dz0 = s (1 - s)
    dmin = (s * (1 - s) if s < a else 0.0) - (s * (1 - s) if 1 - s < b else 0.0)
    assert dtv[0, 0] == pytest.approx(-dmin, rel=1e-12, abs=1e-15)


@pytest.mark.parametrize("objective", ["step_tv", "ce", "kl"])
def test_gradient_central_differences(objective):
    rng = np.random.default_rng({"step_tv": 20, "ce": 21, "kl": 22}[objective])
    N, W, V = 2, 3, 5
    zs, ps = zip(*[_rand(rng, W, V, normalised=False) for _ in range(N)])
    z, p = np.stack(zs), np.stack(ps)

    def total(zz):
        return sum(ob.branch(zz[n], p[n], N, objective)[0] for n in range(N)) / N

    dz = np.stack([ob.branch(z[n], p[n], N, objective)[2] for n in range(N)])
    h = 1e-6
    fd = np.zeros_like(z)
    for idx in np.ndindex(z.shape):
        zp, zm = z.copy(), z.copy()
        zp[idx] += h
        zm[idx] -= h
        fd[idx] = (total(zp) - total(zm)) / (2 * h)
    assert np.allclose(dz, fd, rtol=1e-6, atol=1e-9)


def test_full_tensor_wrapper_matches_branches():
    rng = np.random.default_rng(30)
    z = bf16.encode_rne(rng.standard_normal((3, 2, 17)))
    p = softmax(rng.standard_normal((3, 2, 17)), axis=-1).astype(np.float32)
    for objective in ob.OBJECTIVES:
        out = ob.draft_loss(z, p, objective)
        parts = [ob.branch(bf16.decode(z[n]), p[n], 3, objective) for n in range(3)]
        assert out["loss"] == pytest.approx(sum(x[0] for x in parts) / 3, rel=1e-14)
        assert np.array_equal(out["dlogits"], bf16.encode_rne(out["dz"]))
    e2e = ol.e2e_tv_loss(z, p)
    assert ob.draft_loss(z, p, "e2e_tv")["loss"] == e2e["loss"]
