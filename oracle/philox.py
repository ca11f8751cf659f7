"""Philox-4x32-10 counter-based generator, written from its published definition.

Reference: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel
Random Numbers: As Easy as 1, 2, 3", SC'11.  Philox-4x32 keeps a 128-bit
counter (four 32-bit words) and a 64-bit key (two words).  One round
multiplies counter words 0 and 2 by two fixed odd constants, splits each
64-bit product into its high and low halves, and rebuilds the counter from
those halves XOR-ed with the other two words and the round key.  The key is
advanced between rounds by two Weyl constants (golden-ratio and sqrt(3)
derived).  Ten rounds make Philox-4x32-10.

None of the three pages names a generator; the verify step only needs
reproducible uniforms.  The counter layout used by the verify step is:

    key     = (seed & 0xffffffff, seed >> 32)
    counter = (slot, row_id, step & 0xffffffff, step >> 32)
    u_acc   = (x0 >> 8) * 2**-24      # acceptance of the token in this slot
    u_smp   = (x1 >> 8) * 2**-24      # inverse-CDF draw made after this slot

A slot is a position in the verified sequence: slot 0 is the last committed
token; in the linear verify draft d_i occupies slot i+1; in a token tree the
slot is the node index (node 0 = root).  Words x2 and x3 are unused.  Both
uniforms are exact in float32 and float64 and lie in [0, 1 - 2**-24].

This module is part of the oracle (test infrastructure).
"""

import numpy as np

# Round multipliers and Weyl key increments of Philox-4x32 (Salmon et al.).
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85

_MASK32 = np.uint64(0xFFFFFFFF)


def _mulhilo(a, m):
    """High and low 32-bit halves of the 64-bit product a * m (a: uint64 array)."""
    prod = a * np.uint64(m)
    return prod >> np.uint64(32), prod & _MASK32


def philox4x32_10(counters, key):
    """Apply Philox-4x32 with 10 rounds.

    counters: integer array of shape [..., 4] (each word < 2**32).
    key:      pair (k0, k1) of 32-bit integers.
    Returns a uint32 array of the same shape.
    """
    c = np.asarray(counters, dtype=np.uint64)
    if c.shape[-1] != 4:
        raise ValueError("counters must have a trailing dimension of 4")
    c0, c1, c2, c3 = (c[..., i].copy() for i in range(4))
    k0 = np.uint64(int(key[0]) & 0xFFFFFFFF)
    k1 = np.uint64(int(key[1]) & 0xFFFFFFFF)
    for _ in range(10):
        hi0, lo0 = _mulhilo(c0, PHILOX_M0)
        hi1, lo1 = _mulhilo(c2, PHILOX_M1)
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0), lo1, (hi0 ^ c3 ^ k1), lo0
        k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
        k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def words_to_uniform(words):
    """Map 32-bit words to (w >> 8) * 2**-24 in float64 (exact)."""
    return (np.asarray(words, dtype=np.uint64) >> np.uint64(8)).astype(np.float64) * 2.0 ** -24


def verify_uniforms(seed, step, row_id, n_pos):
    """(u_acc, u_smp), each of length n_pos, for slots 0..n_pos-1 of one row."""
    pos = np.arange(n_pos, dtype=np.uint64)
    ctr = np.zeros((n_pos, 4), dtype=np.uint64)
    ctr[:, 0] = pos
    ctr[:, 1] = np.uint64(int(row_id) & 0xFFFFFFFF)
    ctr[:, 2] = np.uint64(int(step) & 0xFFFFFFFF)
    ctr[:, 3] = np.uint64((int(step) >> 32) & 0xFFFFFFFF)
    key = (int(seed) & 0xFFFFFFFF, (int(seed) >> 32) & 0xFFFFFFFF)
    w = philox4x32_10(ctr, key)
    return words_to_uniform(w[:, 0]), words_to_uniform(w[:, 1])
