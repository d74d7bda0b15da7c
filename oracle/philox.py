"""Philox4x32-10 counter-based generator and the integer -> Gumbel transform.

Test infrastructure (see the package docstring): never imported by the HIP path.

Philox4x32-10 is taken from its published definition: J. Salmon, M. Moraes,
R. Dror, D. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11,
section 3 (the Philox S-box built from two 32x32->64 multiplies, the Weyl key
schedule, 10 rounds).  The pages fix only that sampling is seeded and that the
Philox offset advances between steps ("core.inference.sampling.flashinfer_sampling",
class description), and that each request carries its own 64-bit seed and an
offset (TokenSpeed Triton backend page: seed pool and offsets pool).  The
stream layout below is the reading this implementation takes:

    key     = (seed mod 2^32, seed >> 32)
    counter = (j >> 2, r, off mod 2^32, off >> 32)
    word    = output word (j & 3)

where j is the vocabulary index, r the output row index and off the per-call
step offset.  u, E and g are then

    u = (floor(w / 2^9) + 1/2) * 2^-23          (exact in fp32 and fp64)
    E = -ln u          (= -log1p(-(1 - u)) for u > 1/2, where 1 - u is exact)
    g = -ln E          (a standard Gumbel variate)

Everything is vectorised over numpy uint32 / float64 arrays.
"""

from __future__ import annotations

import numpy as np

# Multipliers and Weyl increments of Philox4x32 (Salmon et al., SC'11, section 3).
PHILOX_M0 = np.uint64(0xD2511F53)
PHILOX_M1 = np.uint64(0xCD9E8D57)
PHILOX_W0 = np.uint32(0x9E3779B9)
PHILOX_W1 = np.uint32(0xBB67AE85)

_MASK32 = np.uint64(0xFFFFFFFF)


def _mul_hi_lo(m: np.uint64, a: np.ndarray):
    """Full 64-bit product of a 32-bit constant and a uint32 array -> (hi, lo)."""
    prod = a.astype(np.uint64) * m
    return (prod >> np.uint64(32)).astype(np.uint32), (prod & _MASK32).astype(np.uint32)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox4x32 rounds on counter (c0..c3) with key (k0, k1).

    All arguments broadcast as uint32 arrays.  One round maps
    (c0, c1, c2, c3) to (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0));
    between rounds the key is bumped by the Weyl constants (W0, W1).
    Returns the four output words as uint32 arrays.
    """
    c0, c1, c2, c3, k0, k1 = np.broadcast_arrays(
        *(np.asarray(v, dtype=np.uint32) for v in (c0, c1, c2, c3, k0, k1)))
    c0, c1, c2, c3 = c0.copy(), c1.copy(), c2.copy(), c3.copy()
    k0, k1 = k0.copy(), k1.copy()
    with np.errstate(over="ignore"):
        for rnd in range(10):
            if rnd > 0:
                k0 = (k0 + PHILOX_W0).astype(np.uint32)
                k1 = (k1 + PHILOX_W1).astype(np.uint32)
            hi0, lo0 = _mul_hi_lo(PHILOX_M0, c0)
            hi1, lo1 = _mul_hi_lo(PHILOX_M1, c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def noise_words(seed: int, row: int, step_offset: int, j) -> np.ndarray:
    """The 32-bit noise word of vocabulary indices ``j`` in output row ``row``.

    key = 64-bit seed, counter = (j >> 2, row, offset lo, offset hi), word j & 3.
    """
    j = np.asarray(j, dtype=np.int64)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    off = int(step_offset) & 0xFFFFFFFFFFFFFFFF
    c0 = (j >> 2).astype(np.uint32)
    out = philox4x32_10(c0, np.uint32(row & 0xFFFFFFFF), np.uint32(off & 0xFFFFFFFF),
                        np.uint32(off >> 32), np.uint32(seed & 0xFFFFFFFF), np.uint32(seed >> 32))
    words = np.stack(out, axis=0)                     # [4, len(j)]
    return words[(j & 3), np.arange(j.size)].reshape(j.shape)


def uniform_from_words(w) -> np.ndarray:
    """u = (floor(w / 2^9) + 1/2) * 2^-23, so u lies in [2^-24, 1 - 2^-24]."""
    w = np.asarray(w, dtype=np.uint64)
    return ((w >> np.uint64(9)).astype(np.float64) + 0.5) * 2.0 ** -23


def gumbel_from_uniform(u) -> np.ndarray:
    """g = -ln(-ln u); the inner log is taken as -log1p(-(1 - u)) for u > 1/2."""
    u = np.asarray(u, dtype=np.float64)
    e = np.where(u > 0.5, -np.log1p(-(1.0 - u)), -np.log(np.minimum(u, 0.5)))
    return -np.log(e)
