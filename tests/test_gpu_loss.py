"""GPU parity of e2e_tv_loss_fwd_bwd against the oracle, through the C ABI.

Small and ragged shapes are compared element by element; the full workload
(N=512, W=7, V=151936) is compared on sampled branches, and on properties
that hold at any size (the loss equals -mean_n sum_j prod alpha of the
returned alphas; gradient rows sum to ~0)."""

import numpy as np
import pytest

from lossless_verify_tv_amd import synth
from oracle import bf16 as obf16
from oracle import loss as ol

from .gpu_util import announce, run_loss
from .parity import ALPHA_RTOL, LOSS_RTOL, compare_branch, rel_close

pytestmark = pytest.mark.gpu


def _check_branches(gpu, z, p, branches, tag):
    N = z.shape[0]
    totals = np.zeros(4, dtype=np.int64)
    for n in branches:
        bad, mid, tie, alt, first = compare_branch(gpu["dlogits"][n], z[n], p[n], N)
        totals += (bad, mid, tie, alt)
        assert bad == 0, (tag, n, first)
    announce(f"loss {tag}: midpoint-exempt {totals[1]}, tie-exempt {totals[2]}, "
             f"rows on the other tie side {totals[3]}, bad {totals[0]}")


def _check_small(z, p, tag):
    announce(f"loss {tag} shape={z.shape}")
    gpu = run_loss(z, p)
    orc = ol.e2e_tv_loss(z, p)
    assert rel_close(gpu["loss"], orc["loss"], LOSS_RTOL), (gpu["loss"], orc["loss"])
    assert np.all(rel_close(gpu["alpha"], orc["alpha"], ALPHA_RTOL))
    _check_branches(gpu, z, p, range(z.shape[0]), tag)
    return gpu, orc


@pytest.mark.parametrize("vocab", [20000, 20001, 8192, 1001, 3])
def test_loss_shrunk(vocab):
    c = synth.loss_case(n_branches=5, width=7, vocab=vocab)
    _check_small(c.draft_logits, c.target_probs, f"N=5 W=7 V={vocab}")


def test_loss_single_position_and_branch():
    c = synth.loss_case(n_branches=1, width=1, vocab=5000)
    gpu, orc = _check_small(c.draft_logits, c.target_probs, "N=1 W=1")
    assert gpu["loss"] == pytest.approx(-float(gpu["alpha"][0, 0]), rel=1e-6)


def test_loss_width_16():
    c = synth.loss_case(n_branches=3, width=16, vocab=4096)
    _check_small(c.draft_logits, c.target_probs, "W=16")


def test_loss_full_workload_sampled():
    announce("loss full workload N=512 W=7 V=151936 (generating)")
    c = synth.loss_case(workers=16)
    gpu = run_loss(c.draft_logits, c.target_probs)
    N, W, _ = c.draft_logits.shape
    # the loss is the mean prefix-product sum of the returned alphas
    a = gpu["alpha"].astype(np.float64)
    assert rel_close(gpu["loss"], -np.cumprod(a, axis=1).sum(1).mean(), 1e-6)
    sample = [0, 1, 2, 255, 511]
    for n in sample:
        _, alpha, _, _, _ = ol.branch(obf16.decode(c.draft_logits[n]), c.target_probs[n], N)
        assert np.all(rel_close(gpu["alpha"][n], alpha, ALPHA_RTOL)), n
    _check_branches(gpu, c.draft_logits, c.target_probs, sample, "full workload (sampled)")
    g = obf16.decode(gpu["dlogits"][:8])
    assert np.all(np.abs(g.sum(-1)) <= 4e-3 * np.abs(g).sum(-1) + 1e-30)


def test_loss_bit_identical_reruns():
    c = synth.loss_case(n_branches=4, width=7, vocab=30000)
    first = run_loss(c.draft_logits, c.target_probs)
    for _ in range(2):
        again = run_loss(c.draft_logits, c.target_probs)
        assert first["loss"] == again["loss"]
        assert np.array_equal(first["alpha"], again["alpha"])
        assert np.array_equal(first["dlogits"], again["dlogits"])


@pytest.mark.parametrize("path", ["fused", "multi-pass"])
def test_loss_both_paths_against_oracle(path, monkeypatch):
    """The single-read kernel and the multi-pass pipeline (the one large V
    uses) both match the oracle."""
    monkeypatch.setenv("LVTV_LOSS_PATH", path)
    c = synth.loss_case(n_branches=4, width=7, vocab=24000)
    _check_small(c.draft_logits, c.target_probs, f"{path} N=4 W=7 V=24000")


def test_loss_vocab_beyond_register_capacity():
    """V above what one workgroup holds in registers takes the multi-pass
    pipeline."""
    c = synth.loss_case(n_branches=2, width=3, vocab=160000)
    _check_small(c.draft_logits, c.target_probs, "N=2 W=3 V=160000")


def test_loss_forced_recompute_is_bit_identical(monkeypatch):
    """With a spin limit of 0 every row gives up waiting for its branch at
    once and recomputes the other rows' overlaps from the inputs; the
    outputs must be bit-identical to the normal path."""
    for shape in ((3, 7, 30000), (2, 16, 4096), (4, 1, 5000)):
        c = synth.loss_case(n_branches=shape[0], width=shape[1], vocab=shape[2])
        normal = run_loss(c.draft_logits, c.target_probs)
        monkeypatch.setenv("LVTV_SPIN_LIMIT", "0")
        announce(f"loss forced recompute shape={shape}")
        forced = run_loss(c.draft_logits, c.target_probs)
        monkeypatch.delenv("LVTV_SPIN_LIMIT")
        assert normal["loss"] == forced["loss"]
        assert np.array_equal(normal["alpha"], forced["alpha"])
        assert np.array_equal(normal["dlogits"], forced["dlogits"])


def test_loss_workspace_reuse_across_shapes():
    """One cached workspace serves calls of different shapes in a row (the
    exchange words of one call are never mistaken for the next call's)."""
    shapes = [(4, 7, 30000), (2, 3, 9000), (4, 7, 30000), (6, 5, 12000)]
    for rnd in range(2):
        for shape in shapes:
            c = synth.loss_case(n_branches=shape[0], width=shape[1], vocab=shape[2])
            _check_small(c.draft_logits, c.target_probs, f"reuse round {rnd} {shape}")
