"""Philox4x32-10 and the uniform streams the oracle's sampler draws.

Test infrastructure (see the package docstring): only tests, the smoke check
and the benchmark's CPU-baseline leg may use this module.

Generator: Philox4x32 with 10 rounds, as defined by Salmon, Moraes, Dror and
Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), section 3.2.
A 128-bit counter (four 32-bit words) and a 64-bit key (two words) map to four
32-bit output words.  One round multiplies counter words 0 and 2 by two fixed
32-bit multipliers, keeping both halves of each 64-bit product, and mixes the
high halves with the other two words and the round key; between rounds the key
is advanced by two Weyl increments.  The pages do not name a generator: that it
is Philox, and the counter layout below, are readings where the pages are
silent.

Counter layout (word0, word1, word2, word3) of each stream, key = (seed low
32 bits, seed high 32 bits):

* accept uniform of request b, draft position i:  (0, i, b, 0), output word 0
* level-1 Gumbel of request b, sampled row a, block c:  (c >> 2, a, b, 1), word c & 3
* level-2 Gumbel of request b, row a, token j:  (j >> 2, a, b, 2), word j & 3

Uniform maps (both exact in float32 and float64):

* accept:  u = (w >> 8) * 2**-24, in [0, 1)
* Gumbel:  u = (2 * (w >> 9) + 1) * 2**-24, in (0, 1)
"""

import numpy as np

# Multipliers of Philox4x32 (SC'11, Table 2).
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
# Weyl key increments: the fractional parts of the golden ratio and of sqrt(3),
# scaled by 2**32 and truncated (SC'11, section 3.2).
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
ROUNDS = 10

_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter, key):
    """Philox4x32-10 of many counters under one key.

    counter: integer array of shape (..., 4) holding 32-bit words.
    key: pair of 32-bit integers (k0, k1).
    Returns a uint32 array of shape (..., 4).
    """
    ctr = np.asarray(counter, dtype=np.uint64) & _MASK32
    c0, c1, c2, c3 = (ctr[..., n].copy() for n in range(4))
    k0 = np.uint64(int(key[0]) & 0xFFFFFFFF)
    k1 = np.uint64(int(key[1]) & 0xFFFFFFFF)
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    for r in range(ROUNDS):
        if r > 0:  # the key is bumped before every round but the first
            k0 = np.uint64((int(k0) + PHILOX_W0) & 0xFFFFFFFF)
            k1 = np.uint64((int(k1) + PHILOX_W1) & 0xFFFFFFFF)
        p0 = m0 * c0  # exact: both factors < 2**32
        p1 = m1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def key_of_seed(seed):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return (seed & 0xFFFFFFFF, seed >> 32)


def uniform_accept(word):
    """[0, 1) uniform from the top 24 bits of a 32-bit word."""
    w = np.asarray(word, dtype=np.uint64)
    return (w >> np.uint64(8)).astype(np.float64) * 2.0**-24


def uniform_open(word):
    """(0, 1) uniform on the odd multiples of 2**-24 from the top 23 bits."""
    w = np.asarray(word, dtype=np.uint64)
    return ((w >> np.uint64(9)).astype(np.float64) * 2.0 + 1.0) * 2.0**-24


def u_accept(seed, b, i):
    """Accept uniforms of request b at draft positions i (array-like)."""
    i = np.atleast_1d(np.asarray(i, dtype=np.uint64))
    ctr = np.zeros(i.shape + (4,), dtype=np.uint64)
    ctr[..., 1] = i
    ctr[..., 2] = b
    return uniform_accept(philox4x32_10(ctr, key_of_seed(seed))[..., 0])


def u_block(seed, b, a, c):
    """Level-1 Gumbel uniforms of request b, sampled row a, blocks c."""
    c = np.atleast_1d(np.asarray(c, dtype=np.uint64))
    ctr = np.zeros(c.shape + (4,), dtype=np.uint64)
    ctr[..., 0] = c >> np.uint64(2)
    ctr[..., 1] = a
    ctr[..., 2] = b
    ctr[..., 3] = 1
    words = philox4x32_10(ctr, key_of_seed(seed))
    lane = (c & np.uint64(3)).astype(np.int64)
    return uniform_open(np.take_along_axis(words, lane[..., None], axis=-1)[..., 0])


def u_token(seed, b, a, j):
    """Level-2 Gumbel uniforms of request b, sampled row a, tokens j."""
    j = np.atleast_1d(np.asarray(j, dtype=np.uint64))
    ctr = np.zeros(j.shape + (4,), dtype=np.uint64)
    ctr[..., 0] = j >> np.uint64(2)
    ctr[..., 1] = a
    ctr[..., 2] = b
    ctr[..., 3] = 2
    words = philox4x32_10(ctr, key_of_seed(seed))
    lane = (j & np.uint64(3)).astype(np.int64)
    return uniform_open(np.take_along_axis(words, lane[..., None], axis=-1)[..., 0])


def gumbel(u):
    """Standard Gumbel variate -ln(-ln u) for u in (0, 1)."""
    return -np.log(-np.log(np.asarray(u, dtype=np.float64)))
