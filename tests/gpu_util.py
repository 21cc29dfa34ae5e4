"""Helpers for the GPU tests: move seeded inputs to the device, call the
library through its binding (which calls the C ABI), run the oracle on the
same inputs."""

from __future__ import annotations

import sys

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
