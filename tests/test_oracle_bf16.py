"""Pins of the oracle's bfloat16 decode / encode."""

import numpy as np
import torch

from oracle import bf16


def _torch_bits(x32):
    t = torch.from_numpy(np.asarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_decode_known_patterns():
    assert bf16.decode(np.uint16(0x3F80)) == 1.0
    assert bf16.decode(np.uint16(0xC000)) == -2.0
    assert bf16.decode(np.uint16(0x0001)) == 2.0 ** -133
    assert np.isinf(bf16.decode(np.uint16(0x7F80)))


def test_encode_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-38).astype(np.float32),   # subnormals
        (rng.standard_normal(5000) * 1e30).astype(np.float32),
        (rng.standard_normal(5000) * 1e-6).astype(np.float32),
        np.array([0.0, -0.0, 3.3895314e38, 3.39e38, -3.4e38], dtype=np.float32),
    ])
    ours = bf16.encode_rne(vals.astype(np.float64))
    assert np.array_equal(ours, _torch_bits(vals))


def test_ties_round_to_even():
    one = np.float64(1.0)
    assert bf16.encode_rne(one + 2.0**-8) == 0x3F80          # tie -> even (1.0)
    assert bf16.encode_rne(one + 3 * 2.0**-8) == 0x3F82      # tie -> even (1 + 2^-6)
    assert bf16.encode_rne(-(one + 2.0**-8)) == 0xBF80


def test_no_double_rounding_from_fp64():
    # 1 + 2^-8 + 2^-30 lies just above the midpoint between 1 and 1 + 2^-7.
    # Via binary32 it would first round to the midpoint and then to even (1.0);
    # rounding directly from fp64 must give 1 + 2^-7.
    x = np.float64(1.0) + 2.0**-8 + 2.0**-30
    assert bf16.encode_rne(x) == 0x3F81


def test_roundtrip_of_representable_values():
    pats = np.arange(0, 0x7F80, 37, dtype=np.uint16)
    assert np.array_equal(bf16.encode_rne(bf16.decode(pats)), pats)
    neg = pats | np.uint16(0x8000)
    assert np.array_equal(bf16.encode_rne(bf16.decode(neg)), neg)
