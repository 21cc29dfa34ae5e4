"""Pins of the oracle's loss with the target given as logits and a
temperature (``oracle.objectives.draft_loss_logits``): the overlap equals the
verify step's overlap at the same temperature (the verify oracle's own
scaling, softmax and overlap, and its full spec_verify), torch fp64 autograd
of the composed function for every objective at a temperature whose scaling
is exact, central finite differences through the temperature scaling, and
the unit-temperature reduction to a probability target. None of these calls
the product path."""

import numpy as np
import pytest
import torch

from oracle import bf16
from oracle import objectives as ob
from oracle import verify as ov


def _case(seed, N, W, V, sigma=1.0):
    rng = np.random.default_rng(seed)
    t = rng.standard_normal((N, W, V)) * 2.0
    z = t + sigma * rng.standard_normal((N, W, V))
    return bf16.encode_rne(z), bf16.encode_rne(t)


@pytest.mark.parametrize("temperature", [0.6, 1.0, 1.7])
def test_alpha_is_the_verify_overlap_at_the_same_temperature(temperature):
    z, t = _case(1, 2, 3, 300)
    out = ob.draft_loss_logits(z, t, temperature, "e2e_tv")
    for n in range(2):
        for k in range(3):
            p, _, _ = ov.softmax64(ov.scale(bf16.decode(t[n, k]).astype(np.float32),
                                            temperature))
            q, _, _ = ov.softmax64(ov.scale(bf16.decode(z[n, k]).astype(np.float32),
                                            temperature))
            a, _ = ov.overlap(p, q)
            assert out["alpha"][n, k] == pytest.approx(a, rel=1e-13)


def test_alpha_matches_the_verify_oracle_output():
    """The full verify oracle on the same rows (every request verifying all
    W positions) reports the same per-position alpha."""
    N, W, V, T = 3, 4, 500, 0.8
    z, t = _case(2, N, W, V)
    target = np.concatenate([t, t[:, :1]], axis=1)       # a bonus row per request
    tokens = np.zeros((N, W), np.int32)
    res = ov.spec_verify(target, z, ov.BF16, tokens, np.full(N, W, np.int32),
                         np.full(N, T, np.float32), np.arange(N, dtype=np.uint64))
    out = ob.draft_loss_logits(z, t, T, "step_tv")
    assert np.allclose(out["alpha"], res["alpha"], rtol=1e-6)


def _torch_loss(zt, tt, inv, objective):
    s = zt * inv
    p = torch.softmax(tt * inv, -1)
    if objective in ("e2e_tv", "step_tv"):
        alpha = torch.minimum(p, torch.softmax(s, -1)).sum(-1)
        if objective == "e2e_tv":
            return -torch.cumprod(alpha, dim=1).sum(1).mean()
        return (1.0 - alpha).sum(1).mean()
    logq = torch.log_softmax(s, -1)
    per = -(p * logq).sum(-1)
    if objective == "kl":
        per = per + (p * torch.log(p)).sum(-1)
    return per.sum(1).mean()


@pytest.mark.parametrize("objective", list(ob.OBJECTIVES))
def test_matches_torch_autograd_at_an_exact_temperature(objective):
    """T = 0.5: fl32(x * 2) is exact, so the oracle and a torch fp64 graph
    of the composed function (scaling, both softmaxes, the objective) see the
    same numbers; autograd supplies the chain rule through the scaling."""
    N, W, V = 3, 5, 40
    z, t = _case(3, N, W, V)
    out = ob.draft_loss_logits(z, t, 0.5, objective)
    zt = torch.tensor(bf16.decode(z), dtype=torch.float64, requires_grad=True)
    tt = torch.tensor(bf16.decode(t), dtype=torch.float64)
    loss = _torch_loss(zt, tt, 2.0, objective)
    loss.backward()
    assert out["loss"] == pytest.approx(loss.item(), rel=1e-12)
    assert np.allclose(out["dz"], zt.grad.numpy(), rtol=1e-9, atol=1e-15)


@pytest.mark.parametrize("objective", list(ob.OBJECTIVES))
def test_gradient_central_differences_through_the_scaling(objective):
    """T = 0.7: finite differences of z -> loss(z * inv, t * inv) in fp64
    (inv = fl32(1/0.7)) against the gradient the oracle returns for those
    scaled logits; the chain factor inv is part of what is checked."""
    rng = np.random.default_rng(4)
    N, W, V = 2, 3, 5
    z = rng.standard_normal((N, W, V))
    t = rng.standard_normal((N, W, V))
    inv = float(np.float32(1.0) / np.float32(0.7))

    def total(zz):
        return sum(ob.branch_scaled(zz[n] * inv, t[n] * inv, inv, N, objective)[0]
                   for n in range(N)) / N

    dz = np.stack([ob.branch_scaled(z[n] * inv, t[n] * inv, inv, N, objective)[2]
                   for n in range(N)])
    h = 1e-6
    fd = np.zeros_like(z)
    for idx in np.ndindex(z.shape):
        zp, zm = z.copy(), z.copy()
        zp[idx] += h
        zm[idx] -= h
        fd[idx] = (total(zp) - total(zm)) / (2 * h)
    assert np.allclose(dz, fd, rtol=1e-6, atol=1e-9)


@pytest.mark.parametrize("objective", list(ob.OBJECTIVES))
def test_unit_temperature_is_the_probability_target(objective):
    """At T = 1 the target enters as softmax(t): the probability-target loss
    fed fp32(softmax(t)) agrees up to that fp32 rounding."""
    z, t = _case(5, 2, 3, 200)
    out = ob.draft_loss_logits(z, t, 1.0, objective)
    t64 = bf16.decode(t)
    p = np.exp(t64 - t64.max(-1, keepdims=True))
    p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
    ref = ob.draft_loss(z, p, objective)
    assert out["loss"] == pytest.approx(ref["loss"], rel=1e-6, abs=1e-7)
    assert np.allclose(out["alpha"], ref["alpha"], rtol=1e-6)
    assert np.allclose(out["dz"], ref["dz"], rtol=1e-4, atol=1e-9)


@pytest.mark.parametrize("temperature", [0.0, -1.0, float("nan"), float("inf"), 1e-39])
def test_bad_temperature_is_refused(temperature):
    z, t = _case(6, 1, 1, 8)
    with pytest.raises(ValueError):
        ob.draft_loss_logits(z, t, temperature, "e2e_tv")
