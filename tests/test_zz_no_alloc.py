"""GPU check of spec_verify_noalloc, the verify entry point that allocates
nothing (its scratch is the library's static per-GPU array), through the C
ABI: two calls in a row, the second with a smaller input, each against
spec_verify with a workspace on the same inputs (bit-identical outputs), and
sizes beyond the scratch rejected before anything is enqueued."""

import numpy as np
import pytest
import torch

import lossless_verify_tv_amd as lv
from lossless_verify_tv_amd import synth

from .gpu_util import announce, device, verify_inputs

pytestmark = pytest.mark.gpu


def _outs(B, Kmax, dev):
    return (torch.full((B,), -7, dtype=torch.int32, device=dev),
            torch.full((B, Kmax + 1), -7, dtype=torch.int32, device=dev),
            torch.full((B, max(Kmax, 0)), -7.0, dtype=torch.float32, device=dev),
            torch.full((B,), -7, dtype=torch.int32, device=dev))


def _np(out):
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def test_noalloc_matches_spec_verify_on_two_calls():
    dev = device()
    cases = [synth.verify_case(5, batch=64, vocab=129280),                  # ragged, mixed T
             synth.verify_case(3, temperature=0.6, batch=6, vocab=20001)]   # smaller, ragged V
    for i, case in enumerate(cases):
        B, Kmax, V = case.shape
        announce(f"noalloc call {i} shape={case.shape}")
        inp = verify_inputs(case, dev)
        want = _np(lv.spec_verify(**inp))
        got = _np(lv.spec_verify_noalloc(**inp, out=_outs(B, Kmax, dev)))
        for name, a, b in zip(("accepted_len", "tokens", "alpha", "status"), want, got):
            assert np.array_equal(a, b), (i, name)
        assert np.all(got[3] == 0)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    dev = device()
    lib = lv.load_library()
    # B = 4096, Kmax = 16, V = 151936 needs far more than 16 MiB of scratch
    need = lv.spec_verify_workspace_bytes(4096, 16, 151936)
    assert need > lv.NOALLOC_SCRATCH_BYTES
    fake = torch.empty(16, dtype=torch.int32, device=dev)
    p = fake.data_ptr()
    code = lib.spec_verify_noalloc(p, p, 1, p, p, p, p, 4096, 16, 151936, p, p, p, p, None)
    assert code == -9
