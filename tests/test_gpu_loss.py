"""GPU parity of e2e_tv_loss_fwd_bwd against the oracle, through the C ABI.

Small and ragged shapes are compared element by element. At the full
workload (N=512, W=7, V=151936) the loss and every alpha are compared with
the oracle run over all 512 branches, and the bf16 gradient element by
element on 32 branches spread over the three draft-noise levels; the
exemptions the parity rules allow are counted and bounded."""

import numpy as np
import pytest
import torch

import lossless_verify_tv_amd as lv
from lossless_verify_tv_amd import synth
from oracle import bf16 as obf16
from oracle import loss as ol

from .gpu_util import (announce, device, full_loss_case, loss_to_device, oracle_loss_all,
                       run_debug_loss, run_loss)
from .parity import (ALPHA_RTOL, LOSS_RTOL, check_exemption_bounds, compare_branch,
                     rel_close)

pytestmark = pytest.mark.gpu


def _check_branches(gpu, z, p, branches, tag):
    N = z.shape[0]
    totals = np.zeros(5, dtype=np.int64)
    for n in branches:
        bad, mid, tie, alt, first, window = compare_branch(gpu["dlogits"][n], z[n], p[n], N)
        totals += (bad, mid, tie, alt, window)
        assert bad == 0, (tag, n, first)
    elems = len(branches) * z.shape[1] * z.shape[2]
    announce(f"loss {tag}: midpoint-exempt {totals[1]}, tie-exempt {totals[2]}, "
             f"rows on the other tie side {totals[3]}, tie-window elements {totals[4]}, "
             f"bad {totals[0]} of {elems} elements")
    check_exemption_bounds(totals[1], totals[2], totals[3], totals[4], elems, tag)


def _check_small(z, p, tag, path=None):
    announce(f"loss {tag} shape={z.shape}")
    gpu = run_loss(z, p) if path is None else run_debug_loss(z, p, path=path)
    orc = ol.e2e_tv_loss(z, p)
    assert rel_close(gpu["loss"], orc["loss"], LOSS_RTOL), (gpu["loss"], orc["loss"])
    assert np.all(rel_close(gpu["alpha"], orc["alpha"], ALPHA_RTOL))
    _check_branches(gpu, z, p, range(z.shape[0]), tag)
    return gpu, orc


@pytest.mark.parametrize("vocab", [20000, 20001, 8192, 1001, 3])
def test_loss_shrunk(vocab):
    c = synth.loss_case(n_branches=5, width=7, vocab=vocab)
    _check_small(c.draft_logits, c.target_probs, f"N=5 W=7 V={vocab}")


@pytest.mark.parametrize("vocab", [8, 9, 15, 16, 17, 4104, 8200, 77825, 155647])
def test_loss_half_split_edges(vocab):
    """A row's halves meet at ceil(V/2) rounded up to a group of 8: rows of
    one group (the second half empty), a second half of one token, halves
    whose last group holds a single group's tokens for one thread, V just
    past the largest half, and V near the largest (every group used, the
    last one partial)."""
    c = synth.loss_case(n_branches=3, width=4, vocab=vocab)
    _check_small(c.draft_logits, c.target_probs, f"N=3 W=4 V={vocab}")


def _offset_copy(t, offset):
    """The values of `t` stored `offset` elements past a fresh allocation's
    start: rows whose base is not 16-byte aligned."""
    flat = torch.empty(t.numel() + offset, dtype=t.dtype, device=t.device)
    view = flat[offset:].view(t.shape)
    view.copy_(t)
    return view


@pytest.mark.parametrize("objective", ["e2e_tv", "step_tv", "ce", "kl"])
def test_unaligned_bases_match_aligned(objective):
    """Inputs whose rows are not 16-byte aligned take the unaligned loads
    (one unaligned vector load per group inside a row, the row's last group
    token by token); outputs must be bit-identical to those from aligned
    copies, whose rows take 16-byte loads."""
    dev = device()
    c = synth.loss_case(n_branches=3, width=7, vocab=30000)
    z, p = loss_to_device(c.draft_logits, c.target_probs, dev)
    announce(f"loss unaligned bases objective={objective}")
    ref = lv.draft_loss_fwd_bwd(z, p, objective)
    got = lv.draft_loss_fwd_bwd(_offset_copy(z, 1), _offset_copy(p, 3), objective)
    torch.cuda.synchronize(dev)
    assert ref[0].item() == got[0].item()
    assert torch.equal(ref[1], got[1])
    assert torch.equal(ref[2].view(torch.int16), got[2].view(torch.int16))


def test_loss_most_branches():
    """The largest branch count (N = 65535, W = 1, V = 8; one workgroup a
    row): the loss and every alpha against the oracle, the gradient element
    by element on 256 branches spread over the batch."""
    c = synth.loss_case(n_branches=65535, width=1, vocab=8)
    z, p = c.draft_logits, c.target_probs
    announce(f"loss most branches shape={z.shape}")
    gpu = run_loss(z, p)
    orc = ol.e2e_tv_loss(z, p)
    assert rel_close(gpu["loss"], orc["loss"], LOSS_RTOL), (gpu["loss"], orc["loss"])
    assert np.all(rel_close(gpu["alpha"], orc["alpha"], ALPHA_RTOL))
    _check_branches(gpu, z, p, range(0, 65535, 257), "N=65535")


@pytest.mark.parametrize("vocab", [1 << 20, 1000003])
def test_loss_large_vocabulary(vocab):
    """V far above the single-read limit (155648): the multi-pass kernels."""
    c = synth.loss_case(n_branches=2, width=3, vocab=vocab)
    _check_small(c.draft_logits, c.target_probs, f"N=2 W=3 V={vocab}")


def test_loss_single_position_and_branch():
    c = synth.loss_case(n_branches=1, width=1, vocab=5000)
    gpu, orc = _check_small(c.draft_logits, c.target_probs, "N=1 W=1")
    assert gpu["loss"] == pytest.approx(-float(gpu["alpha"][0, 0]), rel=1e-6)


def test_loss_width_16():
    c = synth.loss_case(n_branches=3, width=16, vocab=4096)
    _check_small(c.draft_logits, c.target_probs, "W=16")


def test_loss_full_workload_against_the_oracle():
    c = full_loss_case()
    gpu = run_loss(c.draft_logits, c.target_probs)
    N, W, _ = c.draft_logits.shape
    announce("loss full workload: oracle over all 512 branches")
    loss_o, alpha_o = oracle_loss_all(c.draft_logits, c.target_probs, "e2e_tv")
    assert rel_close(gpu["loss"], loss_o, LOSS_RTOL), (gpu["loss"], loss_o)
    ok = rel_close(gpu["alpha"], alpha_o, ALPHA_RTOL)
    assert np.all(ok), (np.argwhere(~ok)[:5], gpu["alpha"][~ok][:5], alpha_o[~ok][:5])
    announce(f"loss full workload: loss {gpu['loss']!r} vs {loss_o!r}, max alpha rel. error "
             f"{np.max(np.abs(gpu['alpha'] - alpha_o) / alpha_o):.3g}")
    # 32 branches, n = 0, 16, ..., 496: every draft-noise level (n mod 3)
    sample = list(range(0, N, 16))
    assert {n % 3 for n in sample} == {0, 1, 2}
    _check_branches(gpu, c.draft_logits, c.target_probs, sample, "full workload, 32 branches")
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


@pytest.mark.parametrize("path", ["auto", "multi-pass"])
def test_loss_both_paths_against_oracle(path):
    """The single-read kernel and the multi-pass pipeline (the one large V
    uses) both match the oracle."""
    c = synth.loss_case(n_branches=4, width=7, vocab=24000)
    _check_small(c.draft_logits, c.target_probs, f"{path} N=4 W=7 V=24000", path=path)


def test_loss_vocab_beyond_register_capacity():
    """V above what one workgroup holds in registers takes the multi-pass
    pipeline."""
    c = synth.loss_case(n_branches=2, width=3, vocab=160000)
    _check_small(c.draft_logits, c.target_probs, "N=2 W=3 V=160000")


def test_loss_forced_recompute_is_bit_identical():
    """With a spin limit of 0 every row gives up waiting for its branch at
    once and recomputes the other rows' overlaps from the inputs; the
    outputs must be bit-identical to the normal path."""
    for shape in ((3, 7, 30000), (2, 16, 4096), (4, 1, 5000)):
        c = synth.loss_case(n_branches=shape[0], width=shape[1], vocab=shape[2])
        normal = run_loss(c.draft_logits, c.target_probs)
        announce(f"loss forced recompute shape={shape}")
        forced = run_debug_loss(c.draft_logits, c.target_probs, spin_limit=0)
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
