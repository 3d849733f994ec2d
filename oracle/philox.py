"""Philox4xW-10 counter-based random numbers, the uniform mapping and Gumbel(0,1).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Philox is defined in Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers:
As Easy as 1, 2, 3" (SC'11), section on the Philox S-box: each round multiplies
words 0 and 2 of the counter by the round multipliers M0, M1, splits every
product into its high and low half, and forms the new counter as
(hi(M1*x2) ^ x1 ^ k0, lo(M1*x2), hi(M0*x0) ^ x3 ^ k1, lo(M0*x0)); between rounds
the key is bumped by the Weyl constants (W0, W1) modulo 2^W.

The same code serves both word sizes: for W=32 the words live in uint64 numpy
arrays (a 32x32-bit product is exact there); for W=64 they are numpy object
arrays of Python ints (exact 128-bit products).  The W=64 instantiation is
pinned against ``numpy.random.Philox`` and the W=32 instantiation against the
rocRAND Philox4x32-10 engine compiled for the host (tests/test_oracle_philox.py).

Keyformer's noise (Keyformer blog page, section on the Gumbel distribution)
is y_i = x_i + zeta_i with zeta ~ Gumbel(0,1).  The pages name no generator; the
reading used here (and by the GPU, independently) is:

* X   = word (j mod 4) of Philox4x32-10 with key (seed mod 2^32, seed >> 32)
        and counter (floor(j/4), p_i, h, 0), p_i the absolute position of the
        window query, h the query head, j the absolute key position;
* u   = (2 * floor(X / 2^9) + 1) * 2^-24, strictly inside (0, 1);
* zeta = -ln(-ln u).
"""

import numpy as np

# Round multipliers and Weyl key increments, from the SC'11 paper (Philox4x32
# and Philox4x64 parameter sets).
CONSTANTS = {
    32: {"M": (0xD2511F53, 0xCD9E8D57), "W": (0x9E3779B9, 0xBB67AE85)},
    64: {"M": (0xD2E7470EE14C6C93, 0xCA5A826395121157),
         "W": (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)},
}


def _as_words(a, width):
    if width == 32:
        return np.asarray(a, dtype=np.uint64) & np.uint64(0xFFFFFFFF)
    return np.asarray(a, dtype=object)


def philox4(counter, key, width=32, rounds=10):
    """Philox4xW-R bijection.

    counter: sequence of 4 arrays (or scalars) of W-bit words (broadcastable).
    key:     sequence of 2 W-bit words.
    Returns a tuple of 4 arrays of W-bit words.
    """
    mask = (1 << width) - 1
    m0, m1 = CONSTANTS[width]["M"]
    w0, w1 = CONSTANTS[width]["W"]
    x0, x1, x2, x3 = (_as_words(c, width) for c in counter)
    x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
    k0, k1 = int(key[0]) & mask, int(key[1]) & mask
    if width == 32:
        m0, m1 = np.uint64(m0), np.uint64(m1)
        sh, msk = np.uint64(32), np.uint64(mask)
    else:
        sh, msk = 64, mask
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + w0) & mask
            k1 = (k1 + w1) & mask
        p0 = m0 * x0
        p1 = m1 * x2
        hi0, lo0 = p0 >> sh, p0 & msk
        hi1, lo1 = p1 >> sh, p1 & msk
        if width == 32:
            kk0, kk1 = np.uint64(k0), np.uint64(k1)
        else:
            kk0, kk1 = k0, k1
        x0, x1, x2, x3 = hi1 ^ x1 ^ kk0, lo1, hi0 ^ x3 ^ kk1, lo0
    return x0, x1, x2, x3


def keyformer_words(seed, head, pos, j):
    """Word (j mod 4) of Philox4x32-10(key=seed, counter=(j//4, pos, head, 0)).

    head: int; pos: array of absolute query positions (broadcast against j);
    j: array of absolute key positions.  Returns uint64 array of 32-bit words.
    """
    seed = int(seed)
    pos = np.asarray(pos, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    pos, j = np.broadcast_arrays(pos, j)
    out = philox4((j // 4, pos, np.full(j.shape, head, dtype=np.int64), np.zeros(j.shape, np.int64)),
                  (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF), width=32)
    lane = (j % 4)
    words = np.stack(out, axis=0)
    return np.take_along_axis(words, lane[None, ...].astype(np.int64), axis=0)[0]


def uniform_open(words):
    """u = (2*floor(X/2^9) + 1) * 2^-24: the top 23 bits of X, centred, in (0,1)."""
    x = np.asarray(words, dtype=np.uint64) >> np.uint64(9)
    return (2.0 * x.astype(np.float64) + 1.0) * 2.0 ** -24


def gumbel(u):
    """zeta = -ln(-ln u) for u in (0,1); -ln u is taken as -log1p(u-1) (u-1 exact)."""
    u = np.asarray(u, dtype=np.float64)
    return -np.log(-np.log1p(u - 1.0))


def keyformer_noise(seed, head, pos, j):
    """Gumbel(0,1) noise for query head ``head`` at query positions ``pos`` and keys ``j``."""
    return gumbel(uniform_open(keyformer_words(seed, head, pos, j)))
