"""Speculative-sampling verify step, plain fp64 restatement (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What is computed, per request b with K_b draft positions (all cites by page
title and section):

0. Temperature transform, the same for target and draft ("Speculative
   Decoding and MTP" survey, section 4: p and q are computed after the same
   temperature transform). The pages do not fix the arithmetic; this build's
   reading: scaled logit s = fl32(x * fl32(1 / T)), an IEEE binary32 divide
   and multiply, then promoted exactly to fp64. At T = 1 this is the
   identity. T = 0 selects the greedy rule (step 7).
1. p_k = softmax(s_target[k]) for k = 0..K_b, q_k = softmax(s_draft[k]) for
   k < K_b, in fp64 (the distributions p(y) and q(y) of "Reading Qwen Bebop
   and DeepSeek DSpark", section "Formulas").
2. Overlap alpha_k = sum_v min(p_k(v), q_k(v)) (same section, eq. alpha_RS,
   which also states alpha = 1 - d_TV) and residual mass
   Z_k = sum_v max(0, p_k(v) - q_k(v)) (survey, section 3). Both are computed
   for every k < K_b, also after the first rejection.
3. Uniforms from Philox4x64-10 keyed on (seed_b; b, k): see ``philox``.
4. Accept scan in order: draft token y_k is accepted with probability
   min(1, p_k(y_k)/q_k(y_k)) (P1 "Formulas", eq. alpha(y); survey section 3),
   read as "accept iff u_k < p/q" with u_k in [0, 1); when q_k(y_k) = 0 the
   token is accepted iff p_k(y_k) > 0. The first rejection ends the scan and
   voids every later position (survey, section 2). j = first rejected
   position, or K_b if none.
5. Correction: if j < K_b, draw from the residual max(0, p_j - q_j) / Z_j
   (survey, section 3; the formula itself is lost from the extracted text,
   and the surrounding proof that accept mass min(p, q) plus reject mass
   max(0, p - q) rebuilds p fixes it). Bonus: if j = K_b, draw from p_{K_b}
   (survey, section 2: the bonus distribution available when every draft is
   accepted). Draws are inverse-CDF in ascending token id: the smallest v
   whose cumulative weight exceeds u' times the total.
6. Emit y_0..y_{j-1}, then the drawn token; pad with -1.
7. Greedy (T = 0; survey section 4): compare each draft token with the target
   argmax (first maximal index), emit the target argmax at the first
   mismatch, or the bonus argmax. alpha_k is then the indicator
   [argmax target_k == argmax draft_k], the T -> 0 limit of the overlap of
   two one-hot distributions (this build's reading; the pages are silent).

Per-request status bits (data faults found on the device without a host
sync; this build's convention): 1 = K_b outside [0, Kmax]; 2 = a draft token
outside [0, V); 4 = temperature negative, NaN or infinite; 8 = a used row
holds a NaN or +inf, or is entirely -inf (after scaling). A faulted request
gets accepted_len = -1, all tokens -1 and alpha 0. Bit 1 is checked only with
a valid K_b; bit 8 only with valid K_b and temperature.

Parity: overlap pinned by the TV identity, exact enumeration and closed forms;
accept rule and draws pinned by exact enumeration over the 24-bit uniform
lattice; the sampler's law pinned by chi-square tests and the worked
expected-length examples; greedy pinned by the T -> 0 limit of the stochastic
path. The RNG contract itself (which token a given seed yields) is fixed by no
page: parity unpinned except by agreement of the two implementations. See
``tests/test_oracle_verify.py``.
"""

from __future__ import annotations

import numpy as np

from . import bf16, philox, truncate

F32 = "f32"
BF16 = "bf16"

STATUS_BAD_K = 1
STATUS_BAD_TOKEN = 2
STATUS_BAD_TEMPERATURE = 4
STATUS_NONFINITE = 8
STATUS_BAD_TRUNCATION = 16


def decode_rows(raw, dtype):
    """Stored logits (float32 array, or uint16 bfloat16 patterns) -> float32."""
    if dtype == F32:
        return np.asarray(raw, dtype=np.float32)
    if dtype == BF16:
        return bf16.decode(raw).astype(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def scale(x32, temperature):
    """Step 0: fl32(x * fl32(1/T)) with binary32 round-to-nearest-even."""
    inv_t = np.float32(1.0) / np.float32(temperature)
    with np.errstate(over="ignore", invalid="ignore"):
        return (np.asarray(x32, dtype=np.float32) * inv_t).astype(np.float32)


def softmax64(s):
    """fp64 softmax of one row. Returns (probabilities, max, sum)."""
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s)
    e = np.exp(s - m)
    total = np.sum(e)
    return e / total, m, total


def overlap(p, q):
    """(alpha, Z) = (sum min(p, q), sum max(0, p - q))."""
    return float(np.sum(np.minimum(p, q))), float(np.sum(np.maximum(0.0, p - q)))


def accept(u, p_y, q_y):
    """Accept decision for one draft token and its margin |u - p/q|."""
    if q_y == 0.0:
        return bool(p_y > 0.0), np.inf
    r = p_y / q_y
    return bool(u < r), abs(u - r)


def draw(u, w):
    """Inverse-CDF draw over weights ``w`` in ascending index.

    Returns (index, normalised CDF margin). ``u`` may be an array (the
    vectorised form is used by the enumeration tests); the margin is then
    omitted.
    """
    c = np.cumsum(np.asarray(w, dtype=np.float64))
    total = c[-1]
    target = np.asarray(u, dtype=np.float64) * total
    v = np.searchsorted(c, target, side="right")
    if np.ndim(u) != 0:
        return v
    v = int(v)
    if v >= len(c):                       # not reachable in fp64; kept total
        v = int(np.flatnonzero(np.asarray(w) > 0)[-1])
    below = c[v - 1] if v > 0 else 0.0
    margin = min(float(target) - below, c[v] - float(target)) / total
    return v, margin


def _row_fault(s):
    """True if a row holds NaN or +inf, or is entirely -inf."""
    if np.isnan(s).any():
        return True
    m = np.max(s)
    return bool(np.isinf(m))


def verify_request(t_rows, d_rows, y, k_b, temperature, seed, b, kmax,
                   uniforms=None, top_k=0, top_p=1.0):
    """Verify one request.

    ``t_rows`` float32 [>= K_b+1, V], ``d_rows`` float32 [>= K_b, V] (decoded
    stored logits), ``y`` int [>= K_b]. Returns a dict with ``accepted_len``,
    ``tokens`` (length kmax+1), ``alpha`` (length kmax), ``status`` and the
    diagnostics used by the parity rules: ``accept_margin`` (length kmax, NaN
    where no decision was taken), ``draw_margin``, ``residual`` (Z_k),
    ``greedy``. ``uniforms(seed, b, k) -> (u_accept, u_draw)`` defaults to
    the Philox mapping; the enumeration tests substitute lattice values.
    ``top_k`` / ``top_p`` truncate p and q first (``truncate``; the defaults
    keep every token); ``trunc_margin`` then reports the closest top-p
    decision of the request's rows. A top_p that is NaN or <= 0 faults the
    request with status 16.
    """
    if uniforms is None:
        uniforms = philox.verify_uniforms
    out = {
        "accepted_len": -1,
        "tokens": np.full(kmax + 1, -1, dtype=np.int64),
        "alpha": np.zeros(kmax, dtype=np.float64),
        "residual": np.zeros(kmax, dtype=np.float64),
        "accept_margin": np.full(kmax, np.nan),
        "draw_margin": np.nan,
        "status": 0,
        "greedy": False,
        "trunc_margin": np.inf,
    }
    status = 0
    if not (float(np.float32(top_p)) > 0.0):
        status |= STATUS_BAD_TRUNCATION
    t_val = float(np.float32(temperature))
    if not (t_val >= 0.0) or np.isinf(t_val):
        status |= STATUS_BAD_TEMPERATURE
    k_b = int(k_b)
    if k_b < 0 or k_b > kmax:
        status |= STATUS_BAD_K
    else:
        vocab = t_rows.shape[-1]
        for k in range(k_b):
            if not (0 <= int(y[k]) < vocab):
                status |= STATUS_BAD_TOKEN
                break
    if status & (STATUS_BAD_K | STATUS_BAD_TEMPERATURE) == 0:
        if t_val == 0.0:
            rows = [t_rows[k] for k in range(k_b + 1)] + [d_rows[k] for k in range(k_b)]
        else:
            rows = [scale(t_rows[k], t_val) for k in range(k_b + 1)] + \
                   [scale(d_rows[k], t_val) for k in range(k_b)]
        if any(_row_fault(r) for r in rows):
            status |= STATUS_NONFINITE
    out["status"] = status
    if status:
        return out

    if t_val == 0.0:
        return _greedy(out, t_rows, d_rows, y, k_b)

    s_t = [scale(t_rows[k], t_val) for k in range(k_b + 1)]
    s_d = [scale(d_rows[k], t_val) for k in range(k_b)]
    top_p = float(np.float32(top_p))
    pt = [truncate.truncated_softmax(s, top_k, top_p) for s in s_t]
    qt = [truncate.truncated_softmax(s, top_k, top_p) for s in s_d]
    p = [x[0] for x in pt]
    q = [x[0] for x in qt]
    out["trunc_margin"] = min([x[3] for x in pt + qt] + [np.inf])

    for k in range(k_b):
        out["alpha"][k], out["residual"][k] = overlap(p[k], q[k])

    j = k_b
    for k in range(k_b):
        u_acc, _ = uniforms(seed, b, k)
        ok, margin = accept(u_acc, p[k][int(y[k])], q[k][int(y[k])])
        out["accept_margin"][k] = margin
        if not ok:
            j = k
            break

    _, u_draw = uniforms(seed, b, j)
    if j < k_b:
        w = np.maximum(0.0, p[j] - q[j])
        if not np.sum(w) > 0.0:            # p_j == q_j: fall back to p_j
            w = p[j]
    else:
        w = p[k_b]
    v, margin = draw(u_draw, w)
    out["draw_margin"] = margin
    out["accepted_len"] = j
    out["tokens"][:j] = np.asarray(y[:j], dtype=np.int64)
    out["tokens"][j] = v
    return out


def _greedy(out, t_rows, d_rows, y, k_b):
    out["greedy"] = True
    g = [int(np.argmax(t_rows[k])) for k in range(k_b + 1)]
    h = [int(np.argmax(d_rows[k])) for k in range(k_b)]
    for k in range(k_b):
        out["alpha"][k] = 1.0 if g[k] == h[k] else 0.0
    j = k_b
    for k in range(k_b):
        if int(y[k]) != g[k]:
            j = k
            break
    out["accepted_len"] = j
    out["tokens"][:j] = np.asarray(y[:j], dtype=np.int64)
    out["tokens"][j] = g[j]
    return out


def spec_verify(target_logits, draft_logits, dtype, draft_tokens, k_per_req,
                temperature, seed, top_k=None, top_p=None):
    """Batched verify.

    ``target_logits`` [B, Kmax+1, V] and ``draft_logits`` [B, Kmax, V] stored
    as float32 (dtype "f32") or uint16 bfloat16 patterns (dtype "bf16");
    ``draft_tokens`` int [B, Kmax]; ``k_per_req`` int [B]; ``temperature``
    float [B]; ``seed`` uint64 [B]; ``top_k`` int [B] and ``top_p`` float
    [B] are optional (``truncate``; omitted: every token kept). Returns a dict
    of stacked per-request results (see ``verify_request``).
    """
    batch = target_logits.shape[0]
    kmax = draft_logits.shape[1]
    res = [verify_request(decode_rows(target_logits[b], dtype),
                          decode_rows(draft_logits[b], dtype),
                          draft_tokens[b], k_per_req[b], temperature[b],
                          int(seed[b]), b, kmax,
                          top_k=0 if top_k is None else int(top_k[b]),
                          top_p=1.0 if top_p is None else float(top_p[b]))
           for b in range(batch)]
    return {
        "accepted_len": np.array([r["accepted_len"] for r in res], dtype=np.int64),
        "tokens": np.stack([r["tokens"] for r in res]),
        "alpha": np.stack([r["alpha"] for r in res]),
        "residual": np.stack([r["residual"] for r in res]),
        "accept_margin": np.stack([r["accept_margin"] for r in res]),
        "draw_margin": np.array([r["draw_margin"] for r in res]),
        "status": np.array([r["status"] for r in res], dtype=np.int64),
        "greedy": np.array([r["greedy"] for r in res]),
        "trunc_margin": np.array([r["trunc_margin"] for r in res]),
    }


def expected_emitted(alphas):
    """Expected tokens emitted per cycle, bonus / correction included:
    1 + sum_j prod_{k<=j} alpha_k (survey, section 6; the formula is lost
    from the extracted text and the section's worked example fixes it).
    "Reading Qwen Bebop and DeepSeek DSpark", section "Formulas", writes the
    same sum without the leading 1 (accepted drafts only)."""
    total, prod = 1.0, 1.0
    for a in alphas:
        prod *= float(a)
        total += prod
    return total
