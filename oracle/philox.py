"""Philox4x64-10, written from its published definition (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Definition: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
1, 2, 3", SC'11, section 3.3 ("Philox"). A 4x64 Philox round multiplies the
counter words 0 and 2 by two fixed odd multipliers, keeps the high and low
halves of the 128-bit products, permutes the words and xors the high halves
with the neighbouring counter words and the round key. Between rounds the key
is bumped by two Weyl constants (the golden ratio and sqrt(3)-1 scaled to 64
bits). Ten rounds.

How the verify step consumes it (no page fixes this, so it is this build's
reading, shared by both implementations): one block per (request b, position
k), with key = (seed_b, 0) and counter = (b, k, 0, 0). Word 0 gives the accept
uniform, word 1 the draw uniform, each as the top 24 bits times 2^-24, which
is exact in fp32 and fp64. The pages only warn that the order in which random
numbers are consumed makes outputs differ between implementations (P3, section
4) and that consuming extra randomness on the reject path is a bug (P3,
section 23); keying by (b, k) makes consumption independent of the accept
path.

Parity: pinned against ``numpy.random.Philox`` (an independent implementation
of Philox4x64-10) in ``tests/test_oracle_philox.py``.
"""

from __future__ import annotations

_MASK64 = (1 << 64) - 1

# Round multipliers and key increments of Philox4x64 (SC'11, table 2 and
# section 3.3).
_MULT_A = 0xD2E7470EE14C6C93
_MULT_B = 0xCA5A826395121157
_WEYL_A = 0x9E3779B97F4A7C15
_WEYL_B = 0xBB67AE8584CAA73B

ROUNDS = 10


def block(counter, key):
    """Return the 4x64-bit output block of Philox4x64-10.

    ``counter`` is four 64-bit words, ``key`` two. Pure Python integers, so
    the 64x64->128-bit products are exact.
    """
    c0, c1, c2, c3 = (int(w) & _MASK64 for w in counter)
    k0, k1 = (int(w) & _MASK64 for w in key)
    for _ in range(ROUNDS):
        prod_a = _MULT_A * c0
        prod_b = _MULT_B * c2
        hi_a, lo_a = prod_a >> 64, prod_a & _MASK64
        hi_b, lo_b = prod_b >> 64, prod_b & _MASK64
        c0, c1, c2, c3 = hi_b ^ c1 ^ k0, lo_b, hi_a ^ c3 ^ k1, lo_a
        k0 = (k0 + _WEYL_A) & _MASK64
        k1 = (k1 + _WEYL_B) & _MASK64
    return c0, c1, c2, c3


def unit24(word):
    """Top 24 bits of a 64-bit word as a float in [0, 1 - 2^-24]."""
    return float(int(word) >> 40) * (2.0 ** -24)


def verify_uniforms(seed, b, k):
    """(accept uniform, draw uniform) for request ``b``, position ``k``."""
    w = block((b, k, 0, 0), (seed, 0))
    return unit24(w[0]), unit24(w[1])
