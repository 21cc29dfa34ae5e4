"""GPU parity of draft_loss_logits_fwd_bwd (every objective with the target
given as bf16 logits and a temperature on both rows) against the oracle,
through the C ABI.

Shrunk and ragged shapes are compared element by element; the full workload
(N=512, W=7, V=151936) on sampled branches plus properties that hold at any
size. Gradient rules: tests/parity.py (compare_branch_logits)."""

import numpy as np
import pytest

from lossless_verify_tv_amd import synth
from oracle import objectives as ob

from .gpu_util import (announce, oracle_loss_all, run_debug_loss, run_draft_loss,
                       run_loss_logits)
from .parity import ALPHA_RTOL, LOSS_RTOL, compare_branch_logits, rel_close

pytestmark = pytest.mark.gpu

OBJECTIVES = ("e2e_tv", "step_tv", "ce", "kl")


def _check(z, t, T, objective, tag, branches=None, path=None):
    announce(f"{tag} shape={z.shape} T={T}")
    gpu = (run_loss_logits(z, t, T, objective) if path is None else
           run_debug_loss(z, t, objective, temperature=T, path=path))
    N = z.shape[0]
    if branches is None:
        orc = ob.draft_loss_logits(z, t, T, objective)
        assert rel_close(gpu["loss"], orc["loss"], LOSS_RTOL), (gpu["loss"], orc["loss"])
        assert np.all(rel_close(gpu["alpha"], orc["alpha"], ALPHA_RTOL))
        branches = range(N)
    tot = np.zeros(2, dtype=np.int64)
    for n in branches:
        bad, exc, first = compare_branch_logits(gpu["dlogits"][n], z[n], t[n], T, N, objective)
        tot += (bad, exc)
        assert bad == 0, (tag, n, first)
    announce(f"{tag}: bad {tot[0]}, excused {tot[1]}")
    return gpu


@pytest.mark.parametrize("objective", OBJECTIVES)
@pytest.mark.parametrize("vocab,T", [(20000, 0.6), (1001, 1.0), (3, 1.5), (8192, 0.35),
                                     (9, 0.8), (8200, 1.2)])
def test_logits_target_shrunk(objective, vocab, T):
    c = synth.loss_logits_case(n_branches=5, width=7, vocab=vocab)
    _check(c.draft_logits, c.target_logits, T, objective, f"{objective} V={vocab}")


@pytest.mark.parametrize("objective", ["e2e_tv", "step_tv"])
def test_both_paths_agree(objective):
    c = synth.loss_logits_case(n_branches=4, width=5, vocab=24000)
    a = _check(c.draft_logits, c.target_logits, 0.8, objective, f"{objective} default path")
    b = _check(c.draft_logits, c.target_logits, 0.8, objective, f"{objective} multi-pass",
               path="multi-pass")
    assert rel_close(a["loss"], b["loss"], 1e-6)
    assert np.all(rel_close(a["alpha"], b["alpha"], 1e-6))


@pytest.mark.parametrize("objective", ["e2e_tv", "step_tv"])
def test_forced_repair_is_bit_identical(objective):
    c = synth.loss_logits_case(n_branches=3, width=7, vocab=30000)
    normal = run_loss_logits(c.draft_logits, c.target_logits, 0.7, objective)
    announce(f"{objective} logits target, forced repair")
    forced = run_debug_loss(c.draft_logits, c.target_logits, objective, temperature=0.7,
                            spin_limit=0)
    assert normal["loss"] == forced["loss"]
    assert np.array_equal(normal["alpha"], forced["alpha"])
    assert np.array_equal(normal["dlogits"], forced["dlogits"])


def test_unit_temperature_is_close_to_the_probability_target():
    """At T = 1 the fused target softmax must give what the probability
    entry gives for p = fp32(softmax(t)), up to the rounding of p."""
    c = synth.loss_logits_case(n_branches=3, width=7, vocab=12000)
    t64 = (c.target_logits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    e = np.exp(t64 - t64.max(-1, keepdims=True))
    p = (e / e.sum(-1, keepdims=True)).astype(np.float32)
    a = run_loss_logits(c.draft_logits, c.target_logits, 1.0, "e2e_tv")
    b = run_draft_loss(c.draft_logits, p, "e2e_tv")
    assert rel_close(a["loss"], b["loss"], 1e-5)
    assert np.all(rel_close(a["alpha"], b["alpha"], 1e-5))


def test_unaligned_rows_take_the_element_path():
    """V not a multiple of 8 (rows not 16-byte aligned) against the oracle."""
    c = synth.loss_logits_case(n_branches=3, width=4, vocab=9999)
    _check(c.draft_logits, c.target_logits, 0.9, "e2e_tv", "e2e_tv V=9999")


@pytest.fixture(scope="module")
def full_case():
    return synth.loss_logits_case(workers=16)


@pytest.mark.parametrize("objective,T", [("e2e_tv", 1.0), ("e2e_tv", 0.7), ("kl", 0.7)])
def test_full_workload_against_the_oracle(objective, T, full_case):
    """The loss and every alpha against the oracle over all 512 branches;
    the gradient element by element on four branches."""
    c = full_case
    N = c.draft_logits.shape[0]
    sample = (0, 1, 257, N - 1)
    gpu = _check(c.draft_logits, c.target_logits, T, objective, f"{objective} full", sample)
    loss_o, alpha_o = oracle_loss_all(c.draft_logits, c.target_logits, objective, temperature=T)
    assert rel_close(gpu["loss"], loss_o, LOSS_RTOL), (objective, T, gpu["loss"], loss_o)
    assert np.all(rel_close(gpu["alpha"], alpha_o, ALPHA_RTOL)), (objective, T)


@pytest.mark.parametrize("objective", ["e2e_tv", "kl"])
def test_vocab_above_the_single_read_limit(objective):
    """V = 160000 exceeds what a half workgroup holds: the multi-pass
    pipeline serves it."""
    c = synth.loss_logits_case(n_branches=2, width=3, vocab=160000)
    _check(c.draft_logits, c.target_logits, 0.8, objective, f"{objective} V=160000")


@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 16, 5), (2, 1, 40000)])
def test_edge_shapes(shape):
    """A single token, the widest branch (W = 16) and a single position."""
    N, W, V = shape
    c = synth.loss_logits_case(n_branches=N, width=W, vocab=V)
    for obj in ("e2e_tv", "step_tv", "ce"):
        _check(c.draft_logits, c.target_logits, 1.3, obj, f"{obj} N={N} W={W} V={V}")


def test_target_row_of_one_hot_logits():
    """A target row with one finite logit and the rest -inf (p one-hot):
    alpha is q at that token, as the oracle computes it."""
    c = synth.loss_logits_case(n_branches=2, width=2, vocab=3000)
    t = c.target_logits.copy()
    t[:, :, :] = 0xFF80                      # -inf
    t[:, :, 17] = synth.to_bf16(np.float32([2.0]))[0]
    _check(c.draft_logits, t, 0.9, "e2e_tv", "one-hot target")
