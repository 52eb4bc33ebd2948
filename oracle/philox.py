"""Philox-4x64-10 counter-based generator (oracle's own implementation).

The sampling mode draws one uniform per (sequence, KV head, token) from a
counter-based integer hash of (seed, head, index), as the workload
description asks ("Philox-style hash").  The pages fix no generator; this
build uses Philox-4x64 with 10 rounds as published by Salmon, Moraes, Dror
and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11): each round
multiplies words 0 and 2 by two odd 64-bit constants, swaps and XORs the
high halves with the other words and a Weyl-sequence key, and the key is
bumped by two further constants between rounds.

Token j of (sequence s, KV head h) takes output word j mod 4 of the block
with counter (floor(j / 4), h, s, 0) and key (seed, 0): the tokens of one
head read the generator's output stream in order, four words per block.
u = ((x >> 11) + 0.5) * 2^-53 is strictly inside (0, 1), where x is that
word.

Pinned against numpy.random.Philox (numpy's independent library
implementation of the same generator) and by a chi-square uniformity test.
"""
from __future__ import annotations

import numpy as np

_M0 = np.uint64(0xD2E7470EE14C6C93)
_M1 = np.uint64(0xCA5A826395121157)
_W0 = np.uint64(0x9E3779B97F4A7C15)
_W1 = np.uint64(0xBB67AE8584CAA73B)
_MASK32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a: np.uint64, b: np.ndarray):
    """(high, low) 64-bit halves of the 128-bit product a*b (b an array)."""
    a_lo, a_hi = a & _MASK32, a >> _S32
    b_lo, b_hi = b & _MASK32, b >> _S32
    ll = a_lo * b_lo
    lh = a_lo * b_hi
    hl = a_hi * b_lo
    hh = a_hi * b_hi
    mid = (ll >> _S32) + (lh & _MASK32) + (hl & _MASK32)
    hi = hh + (lh >> _S32) + (hl >> _S32) + (mid >> _S32)
    lo = a * b  # wraps modulo 2^64
    return hi, lo


def philox4x64_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox-4x64-10 block: counters and key as uint64 arrays or
    scalars (broadcast).  Returns the four 64-bit output words."""
    with np.errstate(over="ignore"):
        c0 = np.asarray(c0, dtype=np.uint64)
        c1 = np.asarray(c1, dtype=np.uint64)
        c2 = np.asarray(c2, dtype=np.uint64)
        c3 = np.asarray(c3, dtype=np.uint64)
        k0 = np.asarray(k0, dtype=np.uint64)
        k1 = np.asarray(k1, dtype=np.uint64)
        for rnd in range(10):
            if rnd:
                k0 = k0 + _W0
                k1 = k1 + _W1
            hi0, lo0 = _mulhilo(_M0, c0)
            hi1, lo1 = _mulhilo(_M1, c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        return c0, c1, c2, c3


def uniform53(seed: int, s: int, h: int, j: np.ndarray) -> np.ndarray:
    """u_j in (0, 1) for tokens j of (sequence s, KV head h): word j mod 4 of
    the block of counter (floor(j / 4), h, s, 0)."""
    j = np.asarray(j, dtype=np.uint64)
    words = philox4x64_10(j >> np.uint64(2), np.uint64(h), np.uint64(s), np.uint64(0),
                          np.uint64(seed), np.uint64(0))
    x = np.choose((j & np.uint64(3)).astype(np.intp), words)
    return ((x >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0 ** -53


def uniform53_draws(seed: int, s: int, h: int, k: np.ndarray) -> np.ndarray:
    """u_k in (0, 1) for the with-replacement draws k of (sequence s, KV
    head h): the same generator on the counter (k, h, s, 1)."""
    k = np.asarray(k, dtype=np.uint64)
    x0, _, _, _ = philox4x64_10(k, np.uint64(h), np.uint64(s), np.uint64(1),
                                np.uint64(seed), np.uint64(0))
    return ((x0 >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0 ** -53
