"""Philox4x32-10 and the dropout keep mask (oracle side; test infrastructure only).

Philox is written from its published definition: J. K. Salmon, M. A. Moraes,
R. O. Dror, D. E. Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11,
section 3 (the Philox S-box built from one 32x32->64-bit multiply per pair of
words, the Weyl key schedule, and the 4x32 permutation).  Constants are the
multipliers and key increments that paper gives for Philox4x32.

The pages use a fixed dropout realisation xi in {0,1} that multiplies each
attention weight by xi/(1-rho) and must be replayed in the reverse pass
(alphabetamath.cc, "A different dropout mask changes the reverse result").  They
do not say how xi is drawn; this library draws it from Philox4x32-10 with

  key     = (seed mod 2^32, seed div 2^32)
  counter = (j div 8, i, b*H + h, 0)          (i = query row, j = key column)
  u       = 16-bit half (j mod 2) of output word (j mod 8) div 2
            (the low half for even j, the high half for odd j)
  xi      = 0 if u < floor(rho * 2^16) else 1

so one Philox call covers eight adjacent keys of one query row, and the rate
is resolved in steps of 2^-16 (at rho = 0.1 a weight is kept with probability
1 - 6553/65536).  The GPU library implements the same written rule
independently.

PARITY: pinned at test time against an independent Philox4x32-10 (PyTorch's
header-only C++ engine, compiled by the test), and on the GPU bit for bit.
"""

import numpy as np

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def _mulhilo(a, b):
    """Full 64-bit product of two 32-bit words, split into (hi, lo)."""
    p = a.astype(np.uint64) * b
    return (p >> np.uint64(32)) & _MASK32, p & _MASK32


def philox4x32_10(counter, key):
    """Ten Philox4x32 rounds.

    counter: four arrays (broadcastable) of uint32 words (c0, c1, c2, c3)
    key:     two python ints (k0, k1), each < 2^32
    returns: four uint32 arrays (x0, x1, x2, x3)
    """
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & _MASK32 for c in counter)
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    for _ in range(10):
        hi0, lo0 = _mulhilo(c0, _M0)
        hi1, lo1 = _mulhilo(c2, _M1)
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0)
        k0 = (k0 + _W0) & 0xFFFFFFFF
        k1 = (k1 + _W1) & 0xFFFFFFFF
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def drop_threshold(rho):
    """Integer threshold floor(rho * 2^16): a 16-bit draw below it drops the weight."""
    if not (0.0 <= rho < 1.0):
        raise ValueError("dropout rate must lie in [0, 1)")
    return int(np.floor(np.float64(rho) * 65536.0))


def keep_mask(seed, rho, lane, rows, cols):
    """xi for one (batch, head) lane: bool array [len(rows), len(cols)].

    lane = b*H + h; rows/cols are integer index arrays of query rows i and key
    columns j.  True means the weight is kept (xi = 1).
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    thr = drop_threshold(rho)
    key = (int(seed) & 0xFFFFFFFF, (int(seed) >> 32) & 0xFFFFFFFF)
    ii = rows[:, None]
    jj = cols[None, :]
    x = philox4x32_10((jj // 8, ii, np.int64(lane), 0), key)
    w = (jj % 8) // 2
    word = np.select([w == 0, w == 1, w == 2], [x[0], x[1], x[2]], x[3]).astype(np.uint64)
    u = np.where(jj % 2 == 0, word & np.uint64(0xFFFF), word >> np.uint64(16))
    return u >= np.uint64(thr)
