"""Philox4x64-10 and the Exp(1) noise of the exponential race.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Philox is the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel random numbers: as easy as 1, 2, 3" (SC'11). Philox4x64-10 maps a
256-bit counter (four 64-bit words) and a 128-bit key (two words) through 10
rounds. One round multiplies counter words 0 and 2 by two fixed odd
multipliers into 128-bit products and mixes their halves with words 1 and 3
and the key; between rounds the key is bumped by two Weyl constants (the
golden-ratio and sqrt(3)-1 fractions). Written here with Python integers, one
block at a time, so every step can be read off directly.

Noise of the race: counter = (vocab id, stream, index, row), key = (seed, 0);
the first output word x gives u = ((x >> 12) + 1/2) * 2^-52, an exact double
strictly inside (0, 1) (with 53 bits the top value would round to 1.0); E =
-ln(u) is evaluated in double and rounded once to float32.
"""
from __future__ import annotations

import math

import numpy as np

MASK64 = (1 << 64) - 1
M0 = 0xD2E7470EE14C6C93
M1 = 0xCA5A826395121157
W0 = 0x9E3779B97F4A7C15
W1 = 0xBB67AE8584CAA73B


def _mulhilo(a: int, b: int):
    p = a * b
    return (p >> 64) & MASK64, p & MASK64


def philox4x64_10(counter, key):
    """One Philox4x64-10 block: 4 counter words, 2 key words -> 4 words."""
    c0, c1, c2, c3 = (int(x) & MASK64 for x in counter)
    k0, k1 = (int(x) & MASK64 for x in key)
    for r in range(10):
        if r > 0:
            k0 = (k0 + W0) & MASK64
            k1 = (k1 + W1) & MASK64
        hi0, lo0 = _mulhilo(M0, c0)
        hi1, lo1 = _mulhilo(M1, c2)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniform_open(x: int) -> float:
    """52 high bits of a 64-bit word -> exact double in the open interval (0,1)."""
    return ((x >> 12) + 0.5) * (2.0 ** -52)


def noise_from_word(x: int) -> np.float32:
    """E = -ln u of the uniform that the 64-bit word x maps to, rounded once to float32."""
    return np.float32(-math.log(uniform_open(x)))


def exp_noise(seed: int, row: int, stream: int, index: int, vocab_id: int) -> np.float32:
    """E ~ Exp(1) for one vocabulary id of one selection."""
    return noise_from_word(philox4x64_10((vocab_id, stream, index, row), (seed, 0))[0])
