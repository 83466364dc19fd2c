"""Philox4x32-10 counter-based generator, written from its published
definition (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
1, 2, 3", SC 2011): a 4 x 32-bit counter and a 2 x 32-bit key; each of the 10
rounds multiplies counter words 0 and 2 by two fixed multipliers, takes the
high and low 32-bit halves of the products, mixes them with the other two
counter words and the key, and the key is bumped by two fixed Weyl increments
between rounds.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.  The HIP library has
its own implementation of the same published definition; nothing is shared.
"""

from __future__ import annotations

import numpy as np

__all__ = ["philox4x32_10", "dropout_keep"]

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint64(0x9E3779B9)
_W1 = np.uint64(0xBB67AE85)
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10.  All arguments are arrays (or scalars) of
    values in [0, 2^32); returns four uint64 arrays holding 32-bit words."""
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & _MASK for x in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint64) & _MASK
    k1 = np.asarray(k1, dtype=np.uint64) & _MASK
    for r in range(10):
        if r:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
        p0 = _M0 * c0  # < 2^64: exact in uint64
        p1 = _M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def dropout_keep(rows, cols, head, seed, offset, p):
    """Keep-mask of attention dropout for query rows x key columns of one
    query head (global head index b * H + h).

    For query i and key j, one Philox call with counter
    (j >> 2, i >> 2, head, offset) and key (seed mod 2^32, seed >> 32) gives
    16 bytes covering the 4 x 4 block of (query, key) pairs; pair (i, j) uses
    byte (j & 3) of word (i & 3).  The weight is kept iff that byte is at
    least floor(256 p), so the drop probability is p truncated to a multiple
    of 1/256; kept weights are scaled by 256 / (256 - floor(256 p)).
    Returns (bool keep[len(rows), len(cols)], scale).
    """
    t8 = int(np.floor(p * 256.0))
    rows = np.asarray(rows, dtype=np.int64)[:, None]
    cols = np.asarray(cols, dtype=np.int64)[None, :]
    words = philox4x32_10(cols >> 2, rows >> 2, np.int64(head), np.int64(offset),
                          np.uint64(seed) & _MASK, np.uint64(seed) >> np.uint64(32))
    wsel = (rows & 3).astype(np.uint64)
    w = np.where(wsel == 0, words[0], np.where(wsel == 1, words[1],
                 np.where(wsel == 2, words[2], words[3])))
    byte = (w >> (np.uint64(8) * (cols & 3).astype(np.uint64))) & np.uint64(0xFF)
    keep = byte >= np.uint64(t8)
    return keep, 256.0 / (256.0 - t8)
