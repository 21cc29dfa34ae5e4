"""Parity rules between the HIP path and the oracle.

Verify (per request):
  * status must be equal; a faulted request must have accepted_len -1, all
    tokens -1 and alpha 0;
  * greedy requests (T = 0): accepted_len, tokens and alpha bit-exact;
  * stochastic requests: find the first decision where the two differ: an
    accept bit at k = min(j_gpu, j_oracle) if the accepted lengths differ,
    otherwise the drawn token. The request is excused if the oracle's margin
    at that decision is below 1e-6 (|u - p/q| for an accept bit, the
    normalised CDF margin for a draw); otherwise it fails. Excused requests
    are counted and reported;
  * alpha_k within 1e-5 relative for every k < K_b (also for excused
    requests), exactly 0 for K_b <= k < Kmax.

Loss:
  * loss and alpha within 1e-5 relative;
  * bfloat16 dlogits equal to the oracle's round-to-nearest-even of its fp64
    gradient, except (i) +-1 bf16 ulp where the fp64 value lies within 1e-5
    relative of a rounding midpoint, (ii) elements whose q and p are within
    1e-6 relative of each other (the [q < p] indicator is then a coin flip
    of rounding). Values below the fp32 minimum normal compare as 0. Both
    exemptions are counted.
  * a near-tie also moves q(u) between S and S' for its whole row, so the
    row's other gradients shift by about q(u)/S. The pages leave the
    subgradient of min at q = p open (either side is a valid one), so for a
    row holding near-ties the GPU row must match the oracle's row for one of
    the tie choices: the oracle is rerun with p nudged across q at the tie
    elements (by 1e-12 relative, which moves alpha by less than 1e-11), so
    that its own indicator takes the other side.
"""

from __future__ import annotations

import numpy as np

MARGIN = 1e-6
ALPHA_RTOL = 1e-5
LOSS_RTOL = 1e-5
MIDPOINT_RTOL = 1e-5
TIE_RTOL = 1e-6
FP32_MIN_NORMAL = 1.1754943508222875e-38


def compare_verify(gpu, orc, k_per_req, kmax):
    """gpu: dict of numpy arrays accepted_len, tokens, alpha, status.
    orc: the oracle's batched dict. Returns a report dict; report["failures"]
    lists (request, reason)."""
    rep = {"requests": 0, "greedy": 0, "stochastic": 0, "faulted": 0,
           "excused_accept": 0, "excused_draw": 0, "failures": []}
    B = len(k_per_req)
    for b in range(B):
        rep["requests"] += 1
        kb = int(k_per_req[b])
        st_g, st_o = int(gpu["status"][b]), int(orc["status"][b])
        if st_g != st_o:
            rep["failures"].append((b, f"status {st_g} != {st_o}"))
            continue
        if st_o:
            rep["faulted"] += 1
            if gpu["accepted_len"][b] != -1 or np.any(gpu["tokens"][b] != -1) \
                    or np.any(gpu["alpha"][b] != 0):
                rep["failures"].append((b, "faulted request outputs not cleared"))
            continue
        a_g = np.asarray(gpu["alpha"][b], dtype=np.float64)
        a_o = np.asarray(orc["alpha"][b], dtype=np.float64)
        if kb < kmax and np.any(a_g[kb:] != 0):
            rep["failures"].append((b, "alpha beyond K_b not zero"))
        if kb > 0:
            err = np.abs(a_g[:kb] - a_o[:kb])
            bad = err > ALPHA_RTOL * np.abs(a_o[:kb])
            if orc["greedy"][b]:
                bad = err != 0
            if np.any(bad):
                k = int(np.flatnonzero(bad)[0])
                rep["failures"].append((b, f"alpha[{k}] {a_g[k]!r} vs {a_o[k]!r}"))
        j_g, j_o = int(gpu["accepted_len"][b]), int(orc["accepted_len"][b])
        t_g, t_o = np.asarray(gpu["tokens"][b]), np.asarray(orc["tokens"][b])
        if orc["greedy"][b]:
            rep["greedy"] += 1
            if j_g != j_o or not np.array_equal(t_g, t_o):
                rep["failures"].append((b, f"greedy mismatch j {j_g} vs {j_o}"))
            continue
        rep["stochastic"] += 1
        if j_g != j_o:
            k = min(j_g, j_o)
            margin = orc["accept_margin"][b][k] if 0 <= k < kb else np.inf
            if margin < MARGIN:
                rep["excused_accept"] += 1
            else:
                rep["failures"].append((b, f"accepted_len {j_g} vs {j_o}, margin {margin:.3g}"))
            continue
        if not np.array_equal(t_g, t_o):
            if np.array_equal(t_g[:j_o], t_o[:j_o]) and np.all(t_g[j_o + 1:] == -1) \
                    and orc["draw_margin"][b] < MARGIN:
                rep["excused_draw"] += 1
            else:
                rep["failures"].append(
                    (b, f"token at {j_o}: {t_g[j_o]} vs {t_o[j_o]}, "
                        f"margin {orc['draw_margin'][b]:.3g}"))
    return rep


def bf16_bits_to_f64(u16):
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)) \
        .view(np.float32).astype(np.float64)


def near_bf16_midpoint(d64, rtol=MIDPOINT_RTOL):
    """True where the fp64 value lies within rtol (relative) of the midpoint
    between two adjacent bf16 values."""
    d = np.abs(np.asarray(d64, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(d > 0, d, 1.0)))
    e = np.maximum(e, -126)
    quantum = np.ldexp(1.0, (e - 7).astype(np.int64))
    frac = d / quantum - np.floor(d / quantum)
    return (np.abs(frac - 0.5) * quantum <= rtol * d) & (d > 0)


def compare_dlogits(gpu_u16, orc_u16, orc_dz64, q64, p64):
    """Element-wise bf16 gradient comparison. Returns (n_bad, n_midpoint,
    n_tie, first_bad_index or None)."""
    g = np.asarray(gpu_u16, dtype=np.uint16)
    o = np.asarray(orc_u16, dtype=np.uint16)
    gv = bf16_bits_to_f64(g)
    ov = bf16_bits_to_f64(o)
    tiny = (np.abs(orc_dz64) < FP32_MIN_NORMAL) & (np.abs(gv) < FP32_MIN_NORMAL)
    equal = (g == o) | tiny | (gv == ov)
    mismatch = ~equal
    tie = mismatch & (np.abs(q64 - p64) <= TIE_RTOL * np.maximum(q64, p64))
    rest = mismatch & ~tie
    gi = g.astype(np.int64) & 0x7FFF
    oi = o.astype(np.int64) & 0x7FFF
    same_sign = (g >> 15) == (o >> 15)
    one_ulp = same_sign & (np.abs(gi - oi) == 1)
    mid = rest & one_ulp & near_bf16_midpoint(orc_dz64)
    bad = rest & ~mid
    first = int(np.flatnonzero(bad.ravel())[0]) if bad.any() else None
    return int(bad.sum()), int(mid.sum()), int(tie.sum()), first


# Bounds on the exemptions, as shares of the elements compared.
#  * Midpoint: the oracle's fp64 value must lie within MIDPOINT_RTOL of a
#    rounding midpoint. bf16 midpoints are 2^-7 of a value's binade apart,
#    so at most 2 * 1.5 * MIDPOINT_RTOL / 2^-7 = 3.84e-3 of uniformly spread
#    values lie that close; 4e-3 bounds the exempted share.
#  * Tie: |q - p| <= TIE_RTOL max(q, p). With a draft that is the target plus
#    Gaussian noise of sigma >= 0.3 (in log space), the density of
#    log(q / p) is at most about 1.4 near 0, so the share of such elements
#    is about 2 TIE_RTOL * 1.4 < 3e-6; 1e-5 bounds it.
#    The same bound holds for every element inside the tie window, whether
#    or not the GPU's element differs.
#  * Rows matched on the other tie side: at most one per tie-window element
#    of the rows compared.
MIDPOINT_SHARE_MAX = 4e-3
TIE_SHARE_MAX = 1e-5


def check_exemption_bounds(n_mid, n_tie, n_alt_rows, n_window, n_elems, tag=""):
    """n_window: elements of the compared rows inside the tie window."""
    assert n_mid <= MIDPOINT_SHARE_MAX * n_elems, (tag, "midpoint exemptions", n_mid, n_elems)
    cap = max(2, TIE_SHARE_MAX * n_elems)
    assert n_window <= cap, (tag, "elements in the tie window", n_window, n_elems)
    assert n_tie <= n_window, (tag, "tie exemptions", n_tie, n_window)
    assert n_alt_rows <= n_window, (tag, "rows on the other tie side", n_alt_rows, n_window)


# Verify: an excused mismatch needs an oracle margin below MARGIN, which a
# uniform accept or draw variate gives with probability about 2 MARGIN per
# decision; the GPU's rounding must then also carry it across. At most one
# excused request per call, or 1e-3 of the stochastic requests, is allowed.
def check_excused_bound(rep, tag=""):
    excused = rep["excused_accept"] + rep["excused_draw"]
    assert excused <= max(1, 1e-3 * rep["stochastic"]), (tag, "excused requests", excused, rep)


def rel_close(a, b, rtol):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.abs(a - b) <= rtol * np.abs(b)


def compare_branch(gpu_u16, z_u16, p32, n_branches, grad=None):
    """Compare the GPU gradient rows of one branch ([W, V] bf16) with the
    oracle, with the tie alternatives described in the module docstring.
    ``grad(z64, p64)`` gives the oracle's fp64 gradient of the branch
    ([W, V]); the default is the E2E-TV loss's (the per-step TV loss passes
    its own). Returns (n_bad, n_midpoint, n_tie, n_rows_on_alternative,
    first_bad, n_tie_window), the last the number of elements inside the
    tie window whether or not they differ."""
    from oracle import bf16 as obf16
    from oracle import loss as ol

    if grad is None:
        def grad(zz, pp):
            return ol.branch(zz, pp, n_branches)[4]
    return _compare_tv_rows(gpu_u16, obf16.decode(z_u16), np.asarray(p32, dtype=np.float64),
                            grad)


def _compare_tv_rows(gpu_u16, z64, p64, grad):
    """compare_branch on fp64 (scaled) draft logits z64 and probabilities
    p64; q = softmax(z64)."""
    from oracle import bf16 as obf16

    dz = grad(z64, p64)
    q = np.exp(z64 - z64.max(-1, keepdims=True))
    q /= q.sum(-1, keepdims=True)
    tie = np.abs(q - p64) <= TIE_RTOL * np.maximum(q, p64)
    tot_bad = tot_mid = tot_tie = alt_rows = 0
    first = None
    for k in range(z64.shape[0]):
        cands = [dz[k]]
        idx = np.flatnonzero(tie[k])
        if idx.size:
            subsets = [idx] if idx.size > 4 else [
                idx[[bool(m >> i & 1) for i in range(idx.size)]]
                for m in range(1, 1 << idx.size)]
            for sub in subsets:
                p_alt = p64.copy()
                below = q[k, sub] < p64[k, sub]
                p_alt[k, sub] = np.where(below, q[k, sub] * (1 - 1e-12), q[k, sub] * (1 + 1e-12))
                cands.append(grad(z64, p_alt)[k])
        best = None
        for ci, cand in enumerate(cands):
            res = compare_dlogits(gpu_u16[k], obf16.encode_rne(cand), cand, q[k], p64[k])
            if best is None or res[0] < best[0][0]:
                best = (res, ci)
        (bad, mid, nt, fb), ci = best
        tot_bad += bad
        tot_mid += mid
        tot_tie += nt
        alt_rows += ci > 0
        if first is None and fb is not None:
            first = (k, fb)
    return tot_bad, tot_mid, tot_tie, alt_rows, first, int(tie.sum())


XENT_QTOL = 4e-6


def compare_xent_branch(gpu_u16, z_u16, p32, n_branches, objective):
    """Gradient rows of one branch under CE or KL: dz = (q sum p - p) / N.

    The GPU evaluates q in fp32 from an exponent whose reference is rounded
    (about 1e-6 relative in q) and forms q sum p - p with one fused
    multiply-add, which cancels where q sum p is close to p. A GPU value
    passes when it is the bf16 round-to-nearest-even of some value within
    XENT_QTOL (q sum p + p) / N of the oracle's fp64 gradient (that bound
    covers both effects), or equal to the oracle's rounding. Returns (n_bad,
    n_within_bound_but_unequal, first_bad)."""
    from oracle import bf16 as obf16
    from oracle import objectives as ob

    z64 = obf16.decode(z_u16)
    p64 = np.asarray(p32, dtype=np.float64)
    dz = ob.branch(z64, p64, n_branches, objective)[2]
    return _compare_xent_rows(gpu_u16, z64, p64, dz, n_branches, 1.0)


def _compare_xent_rows(gpu_u16, z64, p64, dz, n_branches, scale):
    """compare_xent_branch on fp64 (scaled) draft logits z64 and
    probabilities p64, with the oracle's gradient dz already formed and
    carrying the chain factor ``scale``."""
    from oracle import bf16 as obf16

    q = np.exp(z64 - z64.max(-1, keepdims=True))
    q /= q.sum(-1, keepdims=True)
    err = XENT_QTOL * scale * (q * p64.sum(-1, keepdims=True) + p64) / n_branches
    g = np.asarray(gpu_u16, dtype=np.uint16)
    exact = g == obf16.encode_rne(dz)
    lo = bf16_bits_to_f64(obf16.encode_rne(dz - err))
    hi = bf16_bits_to_f64(obf16.encode_rne(dz + err))
    gv = bf16_bits_to_f64(g)
    within = (gv >= np.minimum(lo, hi)) & (gv <= np.maximum(lo, hi))
    tiny = (np.abs(dz) < FP32_MIN_NORMAL) & (np.abs(gv) < FP32_MIN_NORMAL)
    bad = ~(exact | within | tiny)
    first = None
    if bad.any():
        i = int(np.flatnonzero(bad.ravel())[0])
        first = (np.unravel_index(i, bad.shape), float(gv.ravel()[i]), float(dz.ravel()[i]))
    return int(bad.sum()), int((within & ~exact).sum()), first


def compare_branch_logits(gpu_u16, z_u16, t_u16, temperature, n_branches, objective):
    """Gradient rows of one branch of draft_loss_logits_fwd_bwd: the oracle
    works on the scaled logits s = fl32(x fl32(1/T)) of both rows, with
    p = softmax(s_target), and its gradient carries the chain factor
    fl32(1/T). The TV objectives follow compare_branch's rules (ties
    included), CE and KL compare_xent_branch's, with the tolerance scaled by
    fl32(1/T); both q and p are formed on the GPU here, and those bounds
    cover an error of that size in either. Returns (n_bad, n_excused,
    first_bad)."""
    from oracle import objectives as ob

    s_z = ob.scaled_logits(z_u16, temperature)
    s_t = ob.scaled_logits(t_u16, temperature)
    inv = float(np.float32(1.0) / np.float32(temperature))
    e = np.exp(s_t - s_t.max(-1, keepdims=True))
    p64 = e / e.sum(-1, keepdims=True)
    if objective in ("ce", "kl"):
        dz = inv * ob.branch(s_z, p64, n_branches, objective)[2]
        return _compare_xent_rows(gpu_u16, s_z, p64, dz, n_branches, inv)

    def grad(zz, pp):
        return inv * ob.branch(zz, pp, n_branches, objective)[2]
    bad, mid, tie, _, first, _ = _compare_tv_rows(gpu_u16, s_z, p64, grad)
    return bad, mid + tie, first
