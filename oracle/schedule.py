"""Confidence-scheduled verify lengths, plain numpy (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Definition ("Reading Qwen Bebop and DeepSeek DSpark", section "DSpark's
second piece: confidence-scheduled verify length"): request r has per-
position confidences c_{r,j} (the chance that draft token j survives given
that every earlier one did; the pages' soft label is 1 - d_TV, i.e. the
verify step's alpha). The prefix survival is a_{r,j} = prod_{i<=j} c_{r,i}.
Verifying l_r tokens of request r puts B = sum_r (1 + l_r) tokens through the
target model and yields tau = sum_r (1 + sum_{j<=l_r} a_{r,j}) tokens in
expectation; with SPS(B) the engine's decode steps per second at batch size
B, the scheduler picks the l_r that maximise Theta = tau * SPS(B).

Algorithm (the plainest one the definition supports): a_{r,j} does not grow
with j, so for a fixed B the best choice takes the B - R largest survivals,
which form a prefix of every request; Theta is therefore evaluated for every
B from R to R (1 + L) on the sorted survivals and the best B is kept.

Readings (the pages are silent on them):
* confidences are clamped to [0, 1], NaN read as 0;
* the survivals are products in binary32, left to right (the kernel's
  precision, since they decide an integer: the order);
* equal survivals are taken in flat index order r * L + j (so every
  request's selection stays a prefix);
* tau and Theta are fp64; among equal Theta the smallest B wins, and a NaN
  Theta (a NaN throughput) never wins.
"""

from __future__ import annotations

import numpy as np


def survivals(conf):
    """a_{r,j} = prod_{i<=j} c_{r,i} in binary32, left to right."""
    c = np.asarray(conf, dtype=np.float32)
    c = np.where(np.isnan(c), np.float32(0.0), np.clip(c, np.float32(0.0), np.float32(1.0)))
    a = np.empty_like(c)
    run = np.ones(c.shape[0], dtype=np.float32)
    for j in range(c.shape[1]):
        run = (run * c[:, j]).astype(np.float32)
        a[:, j] = run
    return a


def schedule(conf, sps):
    """Returns (l [R] int, Theta at the optimum, B at the optimum, theta [N+1])
    where theta[t] is Theta for B = R + t and N = R L. ``sps`` is indexed by
    the batch size B and has at least R (L + 1) + 1 entries."""
    a = survivals(conf)
    R, L = a.shape
    flat = a.ravel()
    order = np.lexsort((np.arange(flat.size), -flat.astype(np.float64)))
    s = np.concatenate(([0.0], np.cumsum(flat[order].astype(np.float64))))
    sps = np.asarray(sps, dtype=np.float64)
    theta = (R + s) * sps[R + np.arange(flat.size + 1)]
    theta = np.where(np.isnan(theta), -np.inf, theta)   # a NaN never wins
    t = int(np.argmax(theta))
    taken = order[:t]
    lens = np.zeros(R, dtype=np.int64)
    np.maximum.at(lens, taken // L, taken % L + 1)
    return lens, float(theta[t]), R + t, theta


def objective(conf, sps, lens):
    """Theta of an explicit choice of lengths, straight from the definition."""
    a = survivals(conf).astype(np.float64)
    lens = np.asarray(lens)
    tau = sum(1.0 + a[r, :lens[r]].sum() for r in range(a.shape[0]))
    return tau * float(np.asarray(sps, dtype=np.float64)[int(np.sum(1 + lens))])
