"""E2E-TV prefix-product loss and its gradient, plain fp64 (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Definition (cites by page title and section):

* Per-position overlap alpha_k = sum_v min(q_k(v), p_k(v)) = 1 - TV(q_k, p_k)
  ("SpecOPD" summary, prerequisites, "Acceptance length and the E2E-TV
  objective"; "Reading Qwen Bebop and DeepSeek DSpark", section "Bebop's
  solution", alpha_k = 1 - d_TV(p_k, q_k)).
* Prefix survival P(tau >= j) = prod_{k<=j} alpha_k, and the end-to-end
  objective sum_j prod_{k<=j} alpha_k (same Bebop section, eq. E[tau]); the
  loss is its negative. SpecOPD, method step (6): the prefix products of the
  per-position overlaps give the loss, only the draft probabilities are
  differentiated, and the samples and the target distribution are constants.
* Reduction over branches: the pages give the per-branch sum over W
  positions and are silent across branches; this build takes the mean over
  the N branches.
* q_k = softmax(z_k) of the draft logits, no temperature (the pages are
  silent; T = 1 reading). target_probs are used as given, without
  renormalisation.

Gradient (written out, no autograd): with R_{W-1} = 1,
R_k = 1 + alpha_{k+1} R_{k+1} and P_{-1} = 1, dL_n/dalpha_k = -P_{k-1} R_k
(no division by alpha). The subgradient of min at q = p is taken as 0, so
dalpha/dq(v) = [q(v) < p(v)], and the softmax Jacobian gives
dalpha/dz(u) = q(u) ([q(u) < p(u)] - S) with S = sum_{q<p} q. This is
evaluated as q(u) S' when the indicator is 1 and -q(u) S when it is 0, with
S' = sum_{q>=p} q = 1 - S, so that neither side needs the cancellation 1 - S.

Parity: pinned by the worked examples (constant overlaps 0.8 over four
positions give -2.3616; 0.9/0.8/0.7/0.6 give -2.4264), the W = 1 special case
(-alpha, the per-step TV loss shifted by a constant), central finite
differences, torch fp64 autograd, the V = 2 closed form and the zero-sum
invariant of the logit gradient; see ``tests/test_oracle_loss.py``.
"""

from __future__ import annotations

import numpy as np

from . import bf16


def softmax64(z):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - np.max(z))
    return e / np.sum(e)


def branch(z64, p64, n_branches):
    """One branch in fp64.

    ``z64`` [W, V] draft logits, ``p64`` [W, V] target probabilities. Returns
    (L_n, alpha [W], S [W], S' [W], dz [W, V]) where dz already carries the
    1/N of the mean over branches.
    """
    z64 = np.asarray(z64, dtype=np.float64)
    p64 = np.asarray(p64, dtype=np.float64)
    width = z64.shape[0]
    q = np.stack([softmax64(z64[k]) for k in range(width)])
    below = q < p64                              # [q(v) < p(v)]
    alpha = np.sum(np.minimum(q, p64), axis=1)
    s_below = np.sum(np.where(below, q, 0.0), axis=1)
    s_above = np.sum(np.where(below, 0.0, q), axis=1)

    prefix = np.cumprod(alpha)                    # P_j
    loss_n = -float(np.sum(prefix))

    suffix = np.ones(width)                       # R_k
    for k in range(width - 2, -1, -1):
        suffix[k] = 1.0 + alpha[k + 1] * suffix[k + 1]
    prev = np.concatenate(([1.0], prefix[:-1]))   # P_{k-1}
    g = -prev * suffix                            # dL_n / dalpha_k

    coef = (g / n_branches)[:, None]
    dz = np.where(below, coef * q * s_above[:, None], -coef * q * s_below[:, None])
    return loss_n, alpha, s_below, s_above, dz


def e2e_tv_loss(draft_logits_bf16, target_probs):
    """Full loss over [N, W, V].

    ``draft_logits_bf16`` uint16 bfloat16 patterns, ``target_probs`` float32.
    Returns a dict: ``loss`` (mean over branches), ``alpha`` [N, W], ``S``,
    ``S_prime`` [N, W], ``dz`` fp64 [N, W, V] and ``dlogits`` uint16 [N, W, V]
    (bfloat16, round-to-nearest-even directly from fp64).
    """
    n_br, width, vocab = draft_logits_bf16.shape
    alpha = np.zeros((n_br, width))
    s_b = np.zeros((n_br, width))
    s_a = np.zeros((n_br, width))
    dz = np.zeros((n_br, width, vocab))
    total = 0.0
    for n in range(n_br):
        l_n, alpha[n], s_b[n], s_a[n], dz[n] = branch(
            bf16.decode(draft_logits_bf16[n]), target_probs[n], n_br)
        total += l_n
    return {
        "loss": total / n_br,
        "alpha": alpha,
        "S": s_b,
        "S_prime": s_a,
        "dz": dz,
        "dlogits": bf16.encode_rne(dz),
    }


def loss_from_alphas(alphas):
    """-sum_j prod_{k<=j} alpha_k for one branch."""
    return -float(np.sum(np.cumprod(np.asarray(alphas, dtype=np.float64))))
