"""GPU parity of spec_verify_packed (the variable-length layout: rows back to
back, one offsets array) through the C ABI: against the oracle on ragged
inputs, bit-identical to the padded call on the same requests (the ragged
workload at full size, bf16 and fp32), and the fault of every request when
the offsets are bad."""

import numpy as np
import pytest
import torch

import lossless_verify_tv_amd as lv
from lossless_verify_tv_amd import synth

from .gpu_util import announce, device, logits_to_device, run_oracle_verify, run_verify, \
    verify_inputs
from .parity import check_excused_bound, compare_verify

pytestmark = pytest.mark.gpu


def _pack(case):
    """Packed host arrays of a padded case: offsets, target rows, draft rows,
    draft tokens."""
    k = np.asarray(case.k, dtype=np.int64)
    B = k.size
    off = np.zeros(B + 1, dtype=np.int32)
    off[1:] = np.cumsum(k + 1)
    tgt = np.concatenate([case.target[b, :k[b] + 1] for b in range(B)])
    drf = [case.draft[b, :k[b]] for b in range(B)]
    drf = np.concatenate(drf) if int(k.sum()) else case.draft[:0, 0]
    tok = np.concatenate([case.tokens[b, :k[b]] for b in range(B)]).astype(np.int32)
    return off, tgt, drf, tok


def _run_packed(case, dev, off=None):
    o, tgt, drf, tok = _pack(case)
    off = o if off is None else off
    acc, toks, alpha, status = lv.spec_verify_packed(
        logits_to_device(tgt, case.dtype, dev), logits_to_device(drf, case.dtype, dev),
        torch.from_numpy(tok).to(dev), torch.from_numpy(off).to(dev),
        torch.from_numpy(np.ascontiguousarray(case.temperature, dtype=np.float32)).to(dev),
        torch.from_numpy(np.ascontiguousarray(case.seed, dtype=np.uint64).view(np.int64)).to(dev))
    torch.cuda.synchronize(dev)
    return (acc.cpu().numpy(), toks.cpu().numpy(), alpha.cpu().numpy(), status.cpu().numpy(), o)


def _unpack(case, acc, toks, alpha, status, off):
    """Padded outputs (spec_verify's shapes) from packed ones."""
    B, K1 = case.target.shape[:2]
    k = np.asarray(case.k)
    t = np.full((B, K1), -1, dtype=np.int32)
    a = np.zeros((B, K1 - 1), dtype=np.float32)
    for b in range(B):
        t[b, :k[b] + 1] = toks[off[b]:off[b + 1]]
        a[b, :k[b]] = alpha[off[b] - b:off[b + 1] - b - 1]
    return {"accepted_len": acc, "tokens": t, "alpha": a, "status": status}


def test_packed_against_oracle():
    dev = device()
    for case, tag in ((synth.verify_case(5, batch=24, vocab=9000), "ragged bf16"),
                      (synth.verify_case(2, batch=6, vocab=9000, k_values=[0, 4, 1, 0, 2, 3]),
                       "with K_b = 0"),
                      (synth.verify_case(1, temperature=1.0), "fp32")):
        announce(f"packed vs oracle: {tag} shape={case.shape}")
        acc, toks, alpha, status, off = _run_packed(case, dev)
        gpu = _unpack(case, acc, toks, alpha, status, off)
        rep = compare_verify(gpu, run_oracle_verify(case), case.k, case.shape[1])
        assert not rep["failures"], (tag, rep["failures"][:5])
        check_excused_bound(rep, tag)


@pytest.mark.parametrize("which", ["workload5_full", "workload3_T0.6", "ragged_V9001"])
def test_packed_equals_padded(which):
    """Packed rows give the same outputs as padded ones; at V = 9001 the
    packed rows (and all padded rows after the first) are not 16-byte
    aligned."""
    dev = device()
    if which == "workload5_full":
        case = synth.verify_case(5)
    elif which == "ragged_V9001":
        case = synth.verify_case(5, batch=40, vocab=9001)
    else:
        case = synth.verify_case(3, temperature=0.6, batch=16)
    announce(f"packed vs padded: {which} shape={case.shape}")
    padded = run_verify(case, dev)
    acc, toks, alpha, status, off = _run_packed(case, dev)
    packed = _unpack(case, acc, toks, alpha, status, off)
    for key in ("accepted_len", "status", "tokens", "alpha"):
        assert np.array_equal(packed[key], padded[key]), key


def test_bad_offsets_fault_every_request():
    dev = device()
    case = synth.verify_case(2, batch=6, vocab=3000, k_values=[2, 1, 3, 0, 2, 1])
    o, _, _, _ = _pack(case)
    bad = o.copy()
    bad[3], bad[4] = bad[4], bad[3]          # a request with a negative row count
    acc, toks, alpha, status, _ = _run_packed(case, dev, off=bad)
    assert np.all(acc == -1)
    assert np.all(status == lv.STATUS_BAD_K)
    # total rows that do not match the offsets
    short = o.copy()
    short[-1] -= 1
    acc, _, _, status, _ = _run_packed(case, dev, off=short)
    assert np.all(acc == -1) and np.all(status == lv.STATUS_BAD_K)
