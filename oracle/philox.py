"""Philox4xW-R counter-based generator (oracle side) -- test infrastructure.

Written from the definition in Salmon, Moraes, Dror, Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3" (SC'11), section 3.2 (the Philox S-box and
its multipliers) and Table 2 (constants):

* state: a counter of four W-bit words (c0, c1, c2, c3) and a key (k0, k1);
* one round: with (hi0, lo0) = M0 * c0 and (hi1, lo1) = M1 * c2 as full
  2W-bit products, the new counter is
  (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0);
* between rounds the key is bumped by the Weyl constants (k0 += W0, k1 += W1);
* Philox4x32-10 and Philox4x64-10 run 10 rounds.

``philox4`` is the scalar, width-generic textbook form (Python integers);
``philox4x32`` is the same map vectorised over numpy uint64 arrays.
``uniform24`` turns one 32-bit output word into a uniform in (0, 1) that is
exactly representable in fp32: U = (2*(w >> 9) + 1) * 2**-24.
"""

from __future__ import annotations

import numpy as np

# (M0, M1) multipliers and (W0, W1) key-schedule constants, per word width.
PHILOX_CONSTANTS = {
    32: dict(M0=0xD2511F53, M1=0xCD9E8D57, W0=0x9E3779B9, W1=0xBB67AE85),
    64: dict(M0=0xD2E7470EE14C6C93, M1=0xCA5A826395121157,
             W0=0x9E3779B97F4A7C15, W1=0xBB67AE8584CAA73B),
}


def philox4(ctr, key, width: int = 32, rounds: int = 10):
    """Philox4x{width}-{rounds} of a 4-word counter under a 2-word key (Python ints)."""
    cst = PHILOX_CONSTANTS[width]
    mask = (1 << width) - 1
    c0, c1, c2, c3 = (int(x) & mask for x in ctr)
    k0, k1 = (int(x) & mask for x in key)
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + cst["W0"]) & mask
            k1 = (k1 + cst["W1"]) & mask
        p0 = cst["M0"] * c0
        p1 = cst["M1"] * c2
        hi0, lo0 = p0 >> width, p0 & mask
        hi1, lo1 = p1 >> width, p1 & mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return (c0, c1, c2, c3)


def _mulhilo32(a: int, b: np.ndarray):
    p = np.uint64(a) * b.astype(np.uint64)       # < 2**64, exact in uint64
    return (p >> np.uint64(32)), (p & np.uint64(0xFFFFFFFF))


def philox4x32(c0, c1, c2, c3, k0, k1, rounds: int = 10):
    """Vectorised Philox4x32: broadcastable integer arrays in, four uint64 arrays (< 2**32) out."""
    m = np.uint64(0xFFFFFFFF)
    cst = PHILOX_CONSTANTS[32]
    arrs = np.broadcast_arrays(*(np.asarray(x, dtype=np.uint64) & m
                                 for x in (c0, c1, c2, c3, k0, k1)))
    c0, c1, c2, c3, k0, k1 = (a.copy() for a in arrs)
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + np.uint64(cst["W0"])) & m
            k1 = (k1 + np.uint64(cst["W1"])) & m
        hi0, lo0 = _mulhilo32(cst["M0"], c0)
        hi1, lo1 = _mulhilo32(cst["M1"], c2)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def seed_key(seed: int):
    """Split a 64-bit seed into the Philox4x32 key (low word, high word)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32


def uniform24(word):
    """(2*(w >> 9) + 1) * 2**-24: a uniform in (0,1) with 24 significant bits, as float64."""
    w = np.asarray(word, dtype=np.uint64)
    return ((w >> np.uint64(9)).astype(np.float64) * 2.0 + 1.0) * (2.0 ** -24)
