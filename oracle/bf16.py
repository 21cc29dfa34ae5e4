"""bfloat16 decode / encode for the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

bfloat16 keeps the sign, the 8-bit exponent and the top 7 fraction bits of an
IEEE binary32. Decoding is exact. Encoding from fp64 rounds to nearest, ties
to even, directly from the fp64 value (no intermediate fp32 rounding, so no
double rounding); the gradient output of the loss is defined this way (no
page fixes the rounding; round-to-nearest-even is this build's reading).

Parity: pinned against torch's CPU float32 -> bfloat16 cast on
fp32-representable inputs, and on hand-built ties and double-rounding cases,
in ``tests/test_oracle_bf16.py``.
"""

from __future__ import annotations

import numpy as np

_MIN_NORMAL_EXP = -126       # smallest normal exponent (same as binary32)
_FRAC_BITS = 7               # stored fraction bits
_MAX_FINITE = float.fromhex("0x1.fep127")


def decode(u16):
    """uint16 bit patterns -> float64 values (exact)."""
    bits = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return bits.view(np.float32).astype(np.float64)


def encode_rne(x):
    """float64 values -> uint16 bfloat16 bit patterns, round half to even.

    The value is split as m * 2^e with m in [1, 2); the representable grid at
    that binade has spacing 2^(e-7), or 2^(-126-7) below the normal range.
    The value is divided by that spacing (exact in fp64: a power of two),
    rounded to the nearest integer with ties to even (``numpy.rint``), and
    scaled back. Values that round above the largest finite bfloat16 become
    infinities. NaN maps to a quiet NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    ax = np.abs(np.where(finite, x, 0.0))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    # correct log2 rounding at binade edges
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > ax, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= ax, e + 1, e)
    e = np.maximum(e, _MIN_NORMAL_EXP)
    quantum_exp = (e - _FRAC_BITS).astype(np.int64)
    scaled = np.ldexp(ax, -quantum_exp)          # exact
    rounded = np.ldexp(np.rint(scaled), quantum_exp)
    rounded = np.where(rounded > _MAX_FINITE, np.inf, rounded)
    out[...] = np.copysign(rounded, np.where(finite, x, 1.0))
    out = np.where(finite, out, x)
    bits = out.astype(np.float32).view(np.uint32)   # exact: on the bf16 grid
    u16 = (bits >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if np.any(nan):
        u16 = np.where(nan, np.uint16(0x7FC0), u16)
    return u16
