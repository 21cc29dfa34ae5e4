"""Per-position comparators of the E2E-TV objective, plain fp64 (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The pages set three per-position objectives against the end-to-end one
("Reading Qwen Bebop and DeepSeek DSpark", section "Bebop's solution":
cross-entropy CE = -sum_y p(y) log q(y), the divergence
KL(p || q) = sum_y p(y) log(p(y) / q(y)), and the per-step TV loss
L_TV = d_TV(p, q) = 1 - sum_y min(p(y), q(y)); the "SpecOPD" summary's
ablation, Figure 8, compares the E2E-TV objective with CE). The readings
taken here, the same for every objective:

* q_k = softmax(z_k) of the draft logits (no temperature); the target
  probabilities p_k are used as given, without renormalisation;
* a branch's loss is the sum of the per-position losses over its W
  positions, and the reported loss is the mean over the N branches (as for
  the E2E-TV loss, whose oracle is ``oracle/loss.py``);
* in KL, p log p is 0 where p = 0;
* only the draft logits are differentiated; p is a constant.

Gradients, written out from the definitions (no autograd):

* per-step TV: d(1 - alpha_k)/dz(u) = -q(u) ([q(u) < p(u)] - S_k), with
  S_k = sum_{q<p} q and the subgradient of min at q = p taken as 0 (the
  E2E-TV oracle's reading); evaluated as -q(u) S'_k where the bit is set and
  q(u) S_k elsewhere (S'_k = sum_{q>=p} q);
* CE and KL (they differ by the constant sum p log p):
  d/dz(u) of -sum_v p(v) log q(v) = q(u) sum_v p(v) - p(u).

Every gradient carries the 1/N of the mean over branches.
"""

from __future__ import annotations

import numpy as np

from . import bf16
from . import loss as e2e

OBJECTIVES = {"e2e_tv": 0, "step_tv": 1, "ce": 2, "kl": 3}


def _softmax_rows(z64):
    return np.stack([e2e.softmax64(z64[k]) for k in range(z64.shape[0])])


def _log_softmax_rows(z64):
    m = np.max(z64, axis=1, keepdims=True)
    return z64 - m - np.log(np.sum(np.exp(z64 - m), axis=1, keepdims=True))


def branch(z64, p64, n_branches, objective):
    """One branch in fp64 under ``objective`` (a key of OBJECTIVES).

    ``z64`` [W, V] draft logits, ``p64`` [W, V] target probabilities. Returns
    (L_n, alpha [W], dz [W, V]); alpha_k = sum min(q_k, p_k) for every
    objective, dz carries the 1/N of the mean over branches.
    """
    if objective == "e2e_tv":
        loss_n, alpha, _, _, dz = e2e.branch(z64, p64, n_branches)
        return loss_n, alpha, dz
    z64 = np.asarray(z64, dtype=np.float64)
    p64 = np.asarray(p64, dtype=np.float64)
    q = _softmax_rows(z64)
    alpha = np.sum(np.minimum(q, p64), axis=1)
    if objective == "step_tv":
        below = q < p64
        s_below = np.sum(np.where(below, q, 0.0), axis=1)[:, None]
        s_above = np.sum(np.where(below, 0.0, q), axis=1)[:, None]
        loss_n = float(np.sum(1.0 - alpha))
        dz = np.where(below, -q * s_above, q * s_below) / n_branches
        return loss_n, alpha, dz
    if objective in ("ce", "kl"):
        logq = _log_softmax_rows(z64)
        ce = -np.sum(p64 * logq, axis=1)
        if objective == "kl":
            plogp = np.where(p64 > 0, p64 * np.log(np.where(p64 > 0, p64, 1.0)), 0.0)
            per_pos = ce + np.sum(plogp, axis=1)
        else:
            per_pos = ce
        loss_n = float(np.sum(per_pos))
        dz = (q * np.sum(p64, axis=1, keepdims=True) - p64) / n_branches
        return loss_n, alpha, dz
    raise ValueError(f"unknown objective {objective!r}")


def draft_loss(draft_logits_bf16, target_probs, objective):
    """Full loss over [N, W, V] under ``objective``.

    ``draft_logits_bf16`` uint16 bfloat16 patterns, ``target_probs`` float32.
    Returns a dict: ``loss`` (mean over branches), ``alpha`` [N, W], ``dz``
    fp64 [N, W, V] and ``dlogits`` uint16 [N, W, V] (bfloat16,
    round-to-nearest-even directly from fp64).
    """
    n_br, width, vocab = draft_logits_bf16.shape
    alpha = np.zeros((n_br, width))
    dz = np.zeros((n_br, width, vocab))
    total = 0.0
    for n in range(n_br):
        l_n, alpha[n], dz[n] = branch(bf16.decode(draft_logits_bf16[n]), target_probs[n], n_br,
                                      objective)
        total += l_n
    return {"loss": total / n_br, "alpha": alpha, "dz": dz, "dlogits": bf16.encode_rne(dz)}


# ---------------------------------------------------------------------------
# Target given as logits, with a temperature.
#
# The verify step compares p and q after one temperature transform applied to
# both sides ("Speculative Decoding and MTP" survey, section 4), and the
# overlap the loss drives up is that same alpha ("Reading Qwen Bebop and
# DeepSeek DSpark", section "Formulas", eq. alpha_RS; "SpecOPD" summary,
# prerequisite on the E2E-TV objective). Readings taken here, where the
# pages are silent:
#
# * both logit rows are scaled by the verify step's transform,
#   s = fl32(x * fl32(1/T)) (``oracle.verify.scale``); p_k = softmax(s_target),
#   q_k = softmax(s_draft), both in fp64;
# * T > 0 only (a greedy target has no gradient), with fl32(1/T) finite;
# * the gradient is taken with respect to the raw draft logits through the
#   linear map s = x * fl32(1/T), i.e. d/dx = fl32(1/T) * d/ds (the rounding
#   of s is not differentiated);
# * p is a constant (SpecOPD, method step (6)).
# ---------------------------------------------------------------------------

def branch_scaled(s_z, s_t, inv_t, n_branches, objective):
    """One branch from fp64 scaled logits ``s_z`` [W, V] (draft) and ``s_t``
    [W, V] (target), with the chain factor ``inv_t`` = fl32(1/T). Returns
    (L_n, alpha [W], dz [W, V]), dz with respect to the raw draft logits."""
    s_t = np.asarray(s_t, dtype=np.float64)
    p = np.stack([e2e.softmax64(s_t[k]) for k in range(s_t.shape[0])])
    loss_n, alpha, ds = branch(s_z, p, n_branches, objective)
    return loss_n, alpha, float(inv_t) * ds


def scaled_logits(raw_bf16, temperature):
    """fp64 copy of fl32(x * fl32(1/T)) for bfloat16 logits."""
    from . import verify as ov
    return ov.scale(bf16.decode(raw_bf16).astype(np.float32), temperature).astype(np.float64)


def draft_loss_logits(draft_logits_bf16, target_logits_bf16, temperature, objective):
    """Full loss over [N, W, V] with the target given as bfloat16 logits and
    the temperature ``temperature`` > 0 on both sides. Returns a dict as
    ``draft_loss``."""
    with np.errstate(over="ignore", divide="ignore"):
        inv32 = np.float32(1.0) / np.float32(temperature)
    if not (np.isfinite(temperature) and temperature > 0 and np.isfinite(inv32)):
        raise ValueError("the temperature must be finite and > 0, with fl32(1/T) finite")
    n_br, width, vocab = draft_logits_bf16.shape
    inv_t = float(inv32)
    alpha = np.zeros((n_br, width))
    dz = np.zeros((n_br, width, vocab))
    total = 0.0
    for n in range(n_br):
        l_n, alpha[n], dz[n] = branch_scaled(scaled_logits(draft_logits_bf16[n], temperature),
                                             scaled_logits(target_logits_bf16[n], temperature),
                                             inv_t, n_br, objective)
        total += l_n
    return {"loss": total / n_br, "alpha": alpha, "dz": dz, "dlogits": bf16.encode_rne(dz)}
