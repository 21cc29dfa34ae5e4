"""GPU parity of draft_loss_fwd_bwd (the E2E-TV loss and its per-position
comparators: per-step TV, CE, KL) against the oracle, through the C ABI.

Small and ragged shapes are compared element by element. At the full
workload (N=512, W=7, V=151936) the loss and every alpha are compared with
the oracle run over all 512 branches, the gradient on 32 branches. Every
comparator runs on the single-read kernel and, forced through the debug
entry point, on the multi-pass pipeline; the single-read kernel's repair
launch gives the same bits. CE and KL write the gradient in the kernel's
pass over p where a row's coefficient (sum p)/N rounds to 1/N's binary32,
and from a second read of p elsewhere; forcing the second read on every
row gives the same bits. Gradient rules: tests/parity.py."""

import numpy as np
import pytest

from lossless_verify_tv_amd import synth
from oracle import bf16 as obf16
from oracle import objectives as ob

from .gpu_util import (announce, full_loss_case, oracle_loss_all, run_debug_loss,
                       run_draft_loss, run_loss)
from .parity import (ALPHA_RTOL, LOSS_RTOL, check_exemption_bounds, compare_branch,
                     compare_xent_branch,
                     rel_close)

pytestmark = pytest.mark.gpu

COMPARATORS = ("step_tv", "ce", "kl")


# CE and KL: gradient elements that differ from the oracle's rounding but lie
# within the cancellation bound of compare_xent_branch. The bound is absolute
# (4e-6 (q sum p + p) / N) on a value q sum p - p that cancels where q is
# close to p, so its relative width is not small for those elements; this
# caps their share.
XENT_WITHIN_SHARE_MAX = 5e-2


def _check_branches(gpu, z, p, objective, branches, tag):
    N = z.shape[0]
    tot = np.zeros(5, dtype=np.int64)
    for n in branches:
        if objective in ("ce", "kl"):
            bad, within, first = compare_xent_branch(gpu["dlogits"][n], z[n], p[n], N, objective)
            tot += (bad, within, 0, 0, 0)
        else:
            bad, mid, tie, alt, first, window = compare_branch(
                gpu["dlogits"][n], z[n], p[n], N,
                grad=lambda zz, pp: ob.branch(zz, pp, N, objective)[2])
            tot += (bad, mid, tie, alt, window)
        assert bad == 0, (tag, n, first)
    elems = len(branches) * z.shape[1] * z.shape[2]
    announce(f"{tag}: bad {tot[0]}, excused (midpoint or bound) {tot[1]}, ties {tot[2]}, "
             f"rows on the other tie side {tot[3]}, tie-window elements {tot[4]} of {elems}")
    if objective in ("ce", "kl"):
        assert tot[1] <= XENT_WITHIN_SHARE_MAX * elems, (tag, tot[1], elems)
    else:
        check_exemption_bounds(tot[1], tot[2], tot[3], tot[4], elems, tag)


def _check_small(z, p, objective, tag, path=None):
    announce(f"{tag} shape={z.shape}")
    gpu = (run_draft_loss(z, p, objective) if path is None else
           run_debug_loss(z, p, objective, path=path))
    orc = ob.draft_loss(z, p, objective)
    assert rel_close(gpu["loss"], orc["loss"], LOSS_RTOL), (gpu["loss"], orc["loss"])
    assert np.all(rel_close(gpu["alpha"], orc["alpha"], ALPHA_RTOL))
    _check_branches(gpu, z, p, objective, range(z.shape[0]), tag)
    return gpu


@pytest.mark.parametrize("objective", COMPARATORS)
@pytest.mark.parametrize("vocab", [20000, 1001, 3])
def test_comparators_shrunk(objective, vocab):
    c = synth.loss_case(n_branches=5, width=7, vocab=vocab)
    _check_small(c.draft_logits, c.target_probs, objective, f"{objective} N=5 W=7 V={vocab}")


@pytest.mark.parametrize("objective", COMPARATORS)
def test_comparators_on_both_paths(objective):
    c = synth.loss_case(n_branches=4, width=5, vocab=24000)
    fused = _check_small(c.draft_logits, c.target_probs, objective, f"{objective} single-read",
                         path="auto")
    multi = _check_small(c.draft_logits, c.target_probs, objective, f"{objective} multi-pass",
                         path="multi-pass")
    assert rel_close(fused["loss"], multi["loss"], 1e-6)
    assert np.all(rel_close(fused["alpha"], multi["alpha"], 1e-6))


@pytest.mark.parametrize("objective", COMPARATORS)
@pytest.mark.parametrize("vocab", [30000, 20001])
def test_comparators_forced_repair_is_bit_identical(objective, vocab):
    c = synth.loss_case(n_branches=3, width=7, vocab=vocab)
    normal = run_draft_loss(c.draft_logits, c.target_probs, objective)
    announce(f"{objective} forced repair V={vocab}")
    forced = run_debug_loss(c.draft_logits, c.target_probs, objective, spin_limit=0)
    assert normal["loss"] == forced["loss"]
    assert np.array_equal(normal["alpha"], forced["alpha"])
    assert np.array_equal(normal["dlogits"], forced["dlogits"])


def test_e2e_objective_is_the_e2e_call():
    c = synth.loss_case(n_branches=4, width=7, vocab=12000)
    a = run_draft_loss(c.draft_logits, c.target_probs, "e2e_tv")
    b = run_loss(c.draft_logits, c.target_probs)
    assert a["loss"] == b["loss"]
    assert np.array_equal(a["alpha"], b["alpha"])
    assert np.array_equal(a["dlogits"], b["dlogits"])


def test_ce_and_kl_differ_by_the_entropy_of_p():
    """Same gradient; the losses differ by the mean over branches of
    sum_k sum_v p log p, computed here from the inputs alone."""
    c = synth.loss_case(n_branches=3, width=4, vocab=5000)
    ce = run_draft_loss(c.draft_logits, c.target_probs, "ce")
    kl = run_draft_loss(c.draft_logits, c.target_probs, "kl")
    assert np.array_equal(ce["dlogits"], kl["dlogits"])
    p = c.target_probs.astype(np.float64)
    plogp = np.where(p > 0, p * np.log(np.where(p > 0, p, 1.0)), 0.0).sum() / p.shape[0]
    assert kl["loss"] - ce["loss"] == pytest.approx(plogp, rel=1e-4, abs=1e-5)


@pytest.mark.parametrize("objective", COMPARATORS)
def test_comparators_full_workload_against_the_oracle(objective):
    c = full_loss_case()
    announce(f"{objective} full workload")
    gpu = run_draft_loss(c.draft_logits, c.target_probs, objective)
    N = c.draft_logits.shape[0]
    loss_o, alpha_o = oracle_loss_all(c.draft_logits, c.target_probs, objective)
    assert rel_close(gpu["loss"], loss_o, LOSS_RTOL), (objective, gpu["loss"], loss_o)
    assert np.all(rel_close(gpu["alpha"], alpha_o, ALPHA_RTOL)), objective
    announce(f"{objective} full workload: loss {gpu['loss']!r} vs {loss_o!r}")
    sample = list(range(0, N, 16))
    _check_branches(gpu, c.draft_logits, c.target_probs, objective, sample,
                    f"{objective} full, 32 branches")


def _targets_on_both_routes(c):
    """The case's targets with rows that certainly take each CE / KL route:
    row (0, 0) one-hot and row (0, 1) uniform over a power-of-two count of
    tokens (their sums are exactly one in any order: the gradient is written
    in the pass over p), row (1, 0) scaled by 1.001 and row (1, 1) by 0.5
    (their coefficients round elsewhere: the second read rewrites them)."""
    p = c.target_probs.copy()
    V = p.shape[2]
    p[0, 0] = 0.0
    p[0, 0, V // 3] = 1.0
    k = 1 << (V.bit_length() - 2)
    p[0, 1] = 0.0
    p[0, 1, :k] = np.float32(1.0 / k)
    p[1, 0] *= np.float32(1.001)
    p[1, 1] *= np.float32(0.5)
    return p


@pytest.mark.parametrize("objective", ["ce", "kl"])
@pytest.mark.parametrize("shape", [(4, 7, 24000), (3, 5, 100000), (2, 3, 151936),
                                   (5, 2, 155648), (3, 4, 20001)])
def test_xent_gradient_in_one_pass_equals_the_second_read(objective, shape):
    """One workgroup a row (V=24000), halves that skip groups (V=100000),
    halves with every group (V=151936, V=155648), an unaligned row length
    (V=20001: always the second read); N not a power of two, so 1/N is not
    exact. Every output bit-identical, the fp32 gradient too."""
    N, W, V = shape
    c = synth.loss_case(n_branches=N, width=W, vocab=V)
    p = _targets_on_both_routes(c)
    announce(f"{objective} one pass vs second read shape={shape}")
    one = run_debug_loss(c.draft_logits, p, objective, path="auto", want_f32=True)
    two = run_debug_loss(c.draft_logits, p, objective, path="reread", want_f32=True)
    assert one["loss"] == two["loss"]
    assert np.array_equal(one["alpha"], two["alpha"])
    assert np.array_equal(one["dlogits"], two["dlogits"])
    assert np.array_equal(one["dlogits_f32"].view(np.uint32), two["dlogits_f32"].view(np.uint32))


@pytest.mark.parametrize("objective", ["ce", "kl"])
@pytest.mark.parametrize("vocab", [24000, 151936])
def test_xent_targets_on_both_routes_against_the_oracle(objective, vocab):
    c = synth.loss_case(n_branches=3, width=4, vocab=vocab)
    _check_small(c.draft_logits, _targets_on_both_routes(c), objective,
                 f"{objective} one-hot, dyadic and scaled targets V={vocab}")
