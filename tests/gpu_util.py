"""Helpers for the GPU tests: move seeded inputs to the device, call the
library through its binding (which calls the C ABI), run the oracle on the
same inputs."""

from __future__ import annotations

import functools
import os
import sys
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import torch

import lossless_verify_tv_amd as lv
from oracle import verify as ov


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a HIP device (run them on the MI355X box)")
    return torch.device("cuda:0")


def announce(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def logits_to_device(arr, dtype, dev):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(dev)


def verify_inputs(case, dev):
    return dict(
        target_logits=logits_to_device(case.target, case.dtype, dev),
        draft_logits=logits_to_device(case.draft, case.dtype, dev),
        draft_tokens=torch.from_numpy(np.ascontiguousarray(case.tokens, dtype=np.int32)).to(dev),
        k_per_req=torch.from_numpy(np.ascontiguousarray(case.k, dtype=np.int32)).to(dev),
        temperature=torch.from_numpy(np.ascontiguousarray(case.temperature, dtype=np.float32)).to(dev),
        seed=torch.from_numpy(np.ascontiguousarray(case.seed, dtype=np.uint64).view(np.int64)).to(dev),
    )


def run_verify(case, dev=None, inputs=None):
    dev = dev or device()
    inputs = inputs or verify_inputs(case, dev)
    acc, toks, alpha, status = lv.spec_verify(**inputs)
    torch.cuda.synchronize(dev)
    return {"accepted_len": acc.cpu().numpy(), "tokens": toks.cpu().numpy(),
            "alpha": alpha.cpu().numpy(), "status": status.cpu().numpy()}


def run_oracle_verify(case):
    return ov.spec_verify(case.target, case.draft, case.dtype, case.tokens, case.k,
                          case.temperature, case.seed)


def loss_to_device(z_u16, p_f32, dev):
    z = torch.from_numpy(np.ascontiguousarray(z_u16).view(np.int16)).view(torch.bfloat16).to(dev)
    p = torch.from_numpy(np.ascontiguousarray(p_f32, dtype=np.float32)).to(dev)
    return z, p


def run_loss(z_u16, p_f32, dev=None):
    dev = dev or device()
    z, p = loss_to_device(z_u16, p_f32, dev)
    loss, alpha, dl = lv.e2e_tv_loss_fwd_bwd(z, p)
    torch.cuda.synchronize(dev)
    return {"loss": float(loss.cpu().numpy()[0]), "alpha": alpha.cpu().numpy(),
            "dlogits": dl.view(torch.int16).cpu().numpy().view(np.uint16)}


def run_draft_loss(z_u16, p_f32, objective, dev=None):
    dev = dev or device()
    z, p = loss_to_device(z_u16, p_f32, dev)
    loss, alpha, dl = lv.draft_loss_fwd_bwd(z, p, objective)
    torch.cuda.synchronize(dev)
    return {"loss": float(loss.cpu().numpy()[0]), "alpha": alpha.cpu().numpy(),
            "dlogits": dl.view(torch.int16).cpu().numpy().view(np.uint16)}


def run_loss_logits(z_u16, t_u16, temperature, objective, dev=None):
    dev = dev or device()
    z = torch.from_numpy(np.ascontiguousarray(z_u16).view(np.int16)).view(torch.bfloat16).to(dev)
    t = torch.from_numpy(np.ascontiguousarray(t_u16).view(np.int16)).view(torch.bfloat16).to(dev)
    loss, alpha, dl = lv.draft_loss_logits_fwd_bwd(z, t, temperature, objective)
    torch.cuda.synchronize(dev)
    return {"loss": float(loss.cpu().numpy()[0]), "alpha": alpha.cpu().numpy(),
            "dlogits": dl.view(torch.int16).cpu().numpy().view(np.uint16)}


def run_debug_loss(z_u16, target, objective="e2e_tv", temperature=None, path="auto",
                   spin_limit=1 << 16,
                   want_f32=False, dev=None):
    """The loss through lvtv_debug_draft_loss: ``target`` is fp32
    probabilities, or (with ``temperature``) bf16 logits patterns."""
    dev = dev or device()
    z = torch.from_numpy(np.ascontiguousarray(z_u16).view(np.int16)).view(torch.bfloat16).to(dev)
    if temperature is None:
        tp = torch.from_numpy(np.ascontiguousarray(target, dtype=np.float32)).to(dev)
        loss, alpha, dl, d32 = lv.debug_draft_loss(z, target_probs=tp, objective=objective,
                                                   path=path, spin_limit=spin_limit,
                                                   want_f32=want_f32)
    else:
        tl = torch.from_numpy(np.ascontiguousarray(target).view(np.int16)).view(
            torch.bfloat16).to(dev)
        loss, alpha, dl, d32 = lv.debug_draft_loss(z, target_logits=tl, temperature=temperature,
                                                   objective=objective, path=path,
                                                   spin_limit=spin_limit, want_f32=want_f32)
    torch.cuda.synchronize(dev)
    out = {"loss": float(loss.cpu().numpy()[0]), "alpha": alpha.cpu().numpy(),
           "dlogits": dl.view(torch.int16).cpu().numpy().view(np.uint16)}
    if d32 is not None:
        out["dlogits_f32"] = d32.cpu().numpy()
    return out


@functools.lru_cache(maxsize=1)
def full_loss_case():
    """The loss workload at full size (N=512 W=7 V=151936), generated once
    per test session."""
    from lossless_verify_tv_amd import synth
    announce("loss full workload N=512 W=7 V=151936 (generating)")
    return synth.loss_case(workers=min(16, os.cpu_count() or 1))


_POOL_INPUTS = {}


def _oracle_branches(task):
    """Worker: the oracle's (L_n, alpha_n) for branches [n0, n1) of the arrays
    the parent set before forking."""
    from oracle import bf16 as obf16
    from oracle import objectives as ob
    n0, n1, objective, temperature = task
    z, p = _POOL_INPUTS["z"], _POOL_INPUTS["p"]
    N = z.shape[0]
    out = []
    for n in range(n0, n1):
        if temperature is None:
            l_n, alpha, _ = ob.branch(obf16.decode(z[n]), p[n], N, objective)
        else:
            inv_t = float(np.float32(1.0) / np.float32(temperature))
            l_n, alpha, _ = ob.branch_scaled(ob.scaled_logits(z[n], temperature),
                                             ob.scaled_logits(p[n], temperature), inv_t, N,
                                             objective)
        out.append((l_n, alpha))
    return out


def oracle_loss_all(z_u16, target, objective="e2e_tv", temperature=None, workers=16, chunk=8):
    """The oracle's loss (mean over branches of L_n, summed in branch order)
    and alpha [N, W] over every branch, computed branch by branch in a pool
    of processes (the arrays reach the workers by fork, not by pickling).
    ``target``: fp32 probabilities, or (with ``temperature``) bf16 logits."""
    N = z_u16.shape[0]
    _POOL_INPUTS["z"], _POOL_INPUTS["p"] = z_u16, target
    tasks = [(n0, min(N, n0 + chunk), objective, temperature) for n0 in range(0, N, chunk)]
    try:
        with ProcessPoolExecutor(max_workers=min(workers, os.cpu_count() or 1)) as pool:
            parts = list(pool.map(_oracle_branches, tasks))
    finally:
        _POOL_INPUTS.clear()
    res = [r for part in parts for r in part]
    total = 0.0
    for l_n, _ in res:
        total += l_n
    return total / N, np.stack([a for _, a in res])
