"""GPU checks of the loss through the debug entry point and of its workspace
rules, through the C ABI.

* The fp32 gradient before its bf16 rounding (lvtv_debug_draft_loss's
  dlogits_f32) against the oracle's fp64 gradient at 1e-5 relative, on
  shrunk shapes (every branch) and on 16 branches of the full workload.
  Elements inside the tie window |q - p| <= 1e-6 max(q, p) are left out (the
  subgradient of min at q = p is open: "SpecOPD", method step (6)); a row
  holding such elements may match the oracle rerun with the tie taken on
  the other side, as in the bf16 rule.
* The bf16 output of the same call equals the product call's.
* A workspace that held anything (words that look fresh under the
  workspace's current epoch, or a greedy verify call's records) gives the
  same loss as a fresh one.
"""

import numpy as np
import pytest
import torch

import lossless_verify_tv_amd as lv
from lossless_verify_tv_amd import synth
from oracle import bf16 as obf16
from oracle import loss as ol
from oracle import objectives as ob

from .gpu_util import (announce, device, full_loss_case, loss_to_device, run_debug_loss,
                       run_loss, verify_inputs)
from .parity import FP32_MIN_NORMAL, TIE_RTOL, TIE_SHARE_MAX

pytestmark = pytest.mark.gpu

GRAD_RTOL = 1e-5


def _row_ok(g32, dz, window):
    """fp32 row against an fp64 row: within GRAD_RTOL relative outside the
    tie window; values below the fp32 minimum normal compare as 0."""
    tiny = (np.abs(dz) < FP32_MIN_NORMAL) & (np.abs(g32) < FP32_MIN_NORMAL)
    close = np.abs(g32 - dz) <= GRAD_RTOL * np.abs(dz)
    return (close | tiny | window), np.abs(g32 - dz) / np.maximum(np.abs(dz), FP32_MIN_NORMAL)


def _check_f32_branch(g32, z_u16, p32, n_branches, objective="e2e_tv"):
    """Returns (bad elements, rows matched on the other tie side, tie-window
    elements, largest relative error outside the window)."""
    z64 = obf16.decode(z_u16)
    p64 = np.asarray(p32, dtype=np.float64)

    def grad(pp):
        return ob.branch(z64, pp, n_branches, objective)[2]

    dz = grad(p64)
    q = np.exp(z64 - z64.max(-1, keepdims=True))
    q /= q.sum(-1, keepdims=True)
    tie = np.abs(q - p64) <= TIE_RTOL * np.maximum(q, p64)
    bad = alt = 0
    worst = 0.0
    for k in range(z64.shape[0]):
        ok, rel = _row_ok(g32[k], dz[k], tie[k])
        if not ok.all() and tie[k].any():
            idx = np.flatnonzero(tie[k])
            p_alt = p64.copy()
            below = q[k, idx] < p64[k, idx]
            p_alt[k, idx] = np.where(below, q[k, idx] * (1 + 1e-12), q[k, idx] * (1 - 1e-12))
            ok2, rel2 = _row_ok(g32[k], grad(p_alt)[k], tie[k])
            if ok2.sum() > ok.sum():
                ok, rel = ok2, rel2
                alt += 1
        bad += int((~ok).sum())
        worst = max(worst, float(np.max(np.where(tie[k], 0.0, rel))))
    return bad, alt, int(tie.sum()), worst


@pytest.mark.parametrize("objective", ["e2e_tv", "step_tv"])
@pytest.mark.parametrize("shape", [(5, 7, 20000), (3, 4, 20001), (2, 16, 4096), (4, 1, 3)])
@pytest.mark.parametrize("path", ["auto", "multi-pass"])
def test_fp32_gradient_against_the_oracle(objective, shape, path):
    c = synth.loss_case(n_branches=shape[0], width=shape[1], vocab=shape[2])
    announce(f"fp32 gradient {objective} {path} shape={shape}")
    dbg = run_debug_loss(c.draft_logits, c.target_probs, objective, path=path, want_f32=True)
    N = shape[0]
    tot = np.zeros(3, dtype=np.int64)
    worst = 0.0
    for n in range(N):
        bad, alt, window, w = _check_f32_branch(dbg["dlogits_f32"][n], c.draft_logits[n],
                                                c.target_probs[n], N, objective)
        tot += (bad, alt, window)
        worst = max(worst, w)
    announce(f"fp32 gradient {objective} {path} {shape}: bad {tot[0]}, other tie side rows "
             f"{tot[1]}, tie-window elements {tot[2]}, worst rel. error {worst:.3g}")
    assert tot[0] == 0
    assert tot[1] <= tot[2]
    # the bf16 output is the nearest-even rounding of the fp32 one (normal
    # values; torch's CPU cast rounds to nearest even), and equals the
    # product call's
    g32 = dbg["dlogits_f32"]
    r = torch.from_numpy(g32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    normal = np.abs(g32) >= FP32_MIN_NORMAL
    assert np.array_equal(r[normal], dbg["dlogits"][normal])
    if objective == "e2e_tv" and path == "auto":
        prod = run_loss(c.draft_logits, c.target_probs)
        assert np.array_equal(prod["dlogits"], dbg["dlogits"])
        assert prod["loss"] == dbg["loss"]


def test_fp32_gradient_full_workload_sampled():
    c = full_loss_case()
    dbg = run_debug_loss(c.draft_logits, c.target_probs, want_f32=True)
    prod = run_loss(c.draft_logits, c.target_probs)
    assert np.array_equal(prod["dlogits"], dbg["dlogits"])
    N = c.draft_logits.shape[0]
    tot = np.zeros(3, dtype=np.int64)
    worst = 0.0
    sample = list(range(5, N, 32))          # 16 branches, every n mod 3
    for n in sample:
        bad, alt, window, w = _check_f32_branch(dbg["dlogits_f32"][n], c.draft_logits[n],
                                                c.target_probs[n], N)
        tot += (bad, alt, window)
        worst = max(worst, w)
    elems = len(sample) * c.draft_logits.shape[1] * c.draft_logits.shape[2]
    announce(f"fp32 gradient full workload, 16 branches: bad {tot[0]}, other tie side rows "
             f"{tot[1]}, tie-window elements {tot[2]} of {elems}, worst rel. error {worst:.3g}")
    assert tot[0] == 0
    assert tot[2] <= max(2, TIE_SHARE_MAX * elems) and tot[1] <= tot[2]


def _loss_of(z, p, ws):
    loss, alpha, dl = lv.e2e_tv_loss_fwd_bwd(z, p, workspace=ws)
    torch.cuda.synchronize()
    return float(loss.cpu()[0]), alpha.cpu().numpy(), dl.view(torch.int16).cpu().numpy()


def test_loss_ignores_words_left_in_the_workspace():
    """Every 64-bit word of the workspace carries the tag of the epoch the
    control block holds, as a fresh word of this call would: the call must
    not take any of them for a partner's statistics or parts."""
    dev = device()
    c = synth.loss_case(n_branches=4, width=7, vocab=30000)
    z, p = loss_to_device(c.draft_logits, c.target_probs, dev)
    nbytes = lv.e2e_tv_loss_workspace_bytes(4, 7, 30000)
    fresh = lv.new_workspace(nbytes, dev)
    want = _loss_of(z, p, fresh)
    orc = ol.e2e_tv_loss(c.draft_logits, c.target_probs)
    assert want[0] == pytest.approx(orc["loss"], rel=1e-5)
    for epoch in (0, 5, 0x7FFFFFFF):
        tag = ((epoch & 0x7FFFFFFF) << 1) | 1
        ws = lv.new_workspace(nbytes, dev)
        words = ws[: (ws.numel() // 8) * 8].view(torch.int64)
        pattern = (tag << 32) | 0x3F800000                  # tag | 1.0f
        words.fill_(pattern - (1 << 64) if pattern >= 1 << 63 else pattern)
        ws[:4].view(torch.int32).fill_(epoch)
        announce(f"loss on a workspace of stale tagged words, epoch {epoch}")
        got = _loss_of(z, p, ws)
        assert got[0] == want[0]
        assert np.array_equal(got[1], want[1]) and np.array_equal(got[2], want[2])


def test_verify_and_loss_share_one_workspace():
    """A greedy verify call (whose row records hold argmax token ids and NaN
    flags) and the loss alternate on one workspace."""
    dev = device()
    vcase = synth.verify_case(3, temperature=0.0, batch=8, vocab=30000)
    c = synth.loss_case(n_branches=4, width=7, vocab=30000)
    z, p = loss_to_device(c.draft_logits, c.target_probs, dev)
    nbytes = max(lv.e2e_tv_loss_workspace_bytes(4, 7, 30000),
                 lv.spec_verify_workspace_bytes(8, 7, 30000))
    ref = _loss_of(z, p, lv.new_workspace(nbytes, dev))
    ws = lv.new_workspace(nbytes, dev)
    vin = verify_inputs(vcase, dev)
    for rnd in range(3):
        announce(f"greedy verify then loss on one workspace, round {rnd}")
        acc, toks, alpha, status = lv.spec_verify(**vin, workspace=ws)
        torch.cuda.synchronize()
        assert int(status.abs().sum().cpu()) == 0
        got = _loss_of(z, p, ws)
        assert got[0] == ref[0]
        assert np.array_equal(got[1], ref[1]) and np.array_equal(got[2], ref[2])


@pytest.mark.parametrize("objective", ["ce", "kl"])
@pytest.mark.parametrize("shape", [(4, 7, 20000), (3, 5, 20001)])
@pytest.mark.parametrize("path", ["auto", "multi-pass"])
def test_fp32_xent_gradient_against_the_oracle(objective, shape, path):
    """CE / KL: the fp32 gradient q sum p - p (over N) against the oracle's
    fp64 one, within 4e-6 (q sum p + p) / N: q carries about 1e-6 relative
    error from the fp32 exponent reference, and q sum p - p cancels where q
    is close to p, so the bound is absolute in the size of the two terms."""
    c = synth.loss_case(n_branches=shape[0], width=shape[1], vocab=shape[2])
    announce(f"fp32 gradient {objective} {path} shape={shape}")
    dbg = run_debug_loss(c.draft_logits, c.target_probs, objective, path=path, want_f32=True)
    N = shape[0]
    worst = 0.0
    for n in range(N):
        z64 = obf16.decode(c.draft_logits[n])
        p64 = np.asarray(c.target_probs[n], dtype=np.float64)
        dz = ob.branch(z64, p64, N, objective)[2]
        q = np.exp(z64 - z64.max(-1, keepdims=True))
        q /= q.sum(-1, keepdims=True)
        bound = 4e-6 * (q * p64.sum(-1, keepdims=True) + p64) / N
        err = np.abs(dbg["dlogits_f32"][n] - dz)
        worst = max(worst, float(np.max(err / np.maximum(bound, 1e-300))))
        assert np.all(err <= bound + FP32_MIN_NORMAL), (n, float(err.max()))
    announce(f"fp32 gradient {objective} {path}: largest error / bound {worst:.3g}")
