"""Top-k / top-p truncation of the verify step's distributions, plain fp64
(oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The "Speculative Decoding and MTP" survey, section 4, requires p and q to be
computed after the agreed temperature and top-p/top-k transforms, the same
for both. The pages do not spell the transforms out; this build takes the
usual sampling ones, applied to each distribution on its own (the target's
top set for p, the draft's for q):

* order the tokens by scaled logit s (the temperature transform of
  ``verify.scale``) from largest to smallest, lower token id first among
  equal s;
* top-k: keep the first k tokens (k <= 0 or k >= V: keep all);
* top-p: among the tokens top-k kept, with weights w = exp(s - max s), keep
  the shortest prefix whose weight reaches top_p times their total (at least
  one token; top_p >= 1 keeps them all; top_p must be > 0);
* renormalise the kept weights; every other token has probability 0.

The verify step then runs unchanged on the truncated p and q. Which prefix
top-p keeps is decided by floating point; ``keep`` reports how close the
decision was (the distance, relative to the total, between top_p times the
total and the cumulative weights on either side of the boundary), and the
parity rules excuse a request whose decision lies within 1e-6.
"""

from __future__ import annotations

import numpy as np


def order(s):
    """Token ids by s descending, id ascending among equal s."""
    s = np.asarray(s, dtype=np.float64)
    return np.lexsort((np.arange(s.size), -s))


def keep(s, top_k, top_p):
    """Kept-token mask of one row and the top-p decision margin (inf when
    top-p keeps everything top-k kept)."""
    s = np.asarray(s, dtype=np.float64)
    V = s.size
    idx = order(s)
    k = int(top_k)
    m = k if 1 <= k < V else V
    margin = np.inf
    if float(top_p) < 1.0:
        w = np.exp(s[idx[:m]] - np.max(s))
        c = np.cumsum(w)
        target = float(top_p) * c[-1]
        n = int(np.searchsorted(c, target, side="left")) + 1   # first c[n-1] >= target
        n = min(max(n, 1), m)
        below = c[n - 2] if n >= 2 else 0.0
        margin = min(abs(c[n - 1] - target), abs(target - below)) / c[-1]
        m = n
    mask = np.zeros(V, dtype=bool)
    mask[idx[:m]] = True
    return mask, margin


def truncated_softmax(s, top_k, top_p):
    """(p', max s, kept weight, margin): p' is the softmax over the kept
    tokens, 0 elsewhere."""
    s = np.asarray(s, dtype=np.float64)
    mask, margin = keep(s, top_k, top_p)
    mx = np.max(s)
    e = np.where(mask, np.exp(s - mx), 0.0)
    total = np.sum(e)
    return e / total, mx, total, margin
