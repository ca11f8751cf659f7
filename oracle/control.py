"""Speculation control between rounds (oracle; test infrastructure).

Dynamic gamma (blog.lonae.com/posts/2026-draft-model-kv-jDwzYp, bimodal-
acceptance paragraph): each request's acceptance rate over its last 16 steps
sets its next speculation length, 8 above 60%, 4 from 30% to 60%, 2 below
30%; with the temperature coupling of the same paragraph, a request whose
temperature is above 0.8 drafts a single token.

Readings: a step is one tested draft position, accepted (1) or rejected (0);
a round that accepted n of its gamma drafts adds n ones, then a zero when it
stopped on a rejection (positions after the first rejection are not
tested).  The rate is taken over the last min(16, steps seen) outcomes; a
request with no outcome yet drafts 4.  A round flagged by the verify call
(num_accepted < 0) adds nothing.

History word: bits 0..15 hold the outcomes (bit 0 the newest), bits 16..20
how many of them are valid (0..16).
"""

import numpy as np

WINDOW = 16


def push(word, n, g):
    hist, count = word & 0xFFFF, (word >> 16) & 0x1F
    if n < 0:
        return word
    outcomes = [1] * n + ([0] if n < g else [])
    for o in outcomes:
        hist = ((hist << 1) | o) & 0xFFFF
        count = min(count + 1, WINDOW)
    return hist | (count << 16)


def gamma_of(word, temp=None, couple_temperature=False):
    # the temperature is a float32 input: the threshold test is taken in float32
    if couple_temperature and temp is not None and np.float32(temp) > np.float32(0.8):
        return 1
    hist, count = word & 0xFFFF, (word >> 16) & 0x1F
    if count == 0:
        return 4
    ones = bin(hist & ((1 << count) - 1)).count("1")
    # rate = ones / count, compared in integers: > 0.6, >= 0.3
    if 5 * ones > 3 * count:
        return 8
    if 10 * ones >= 3 * count:
        return 4
    return 2


def gamma_update(history, num_accepted, gamma_used, temp_target=None, couple_temperature=False):
    """Returns (new history words [B], next gammas [B], next draft offsets [B+1])."""
    B = len(history)
    hist = np.array([push(int(history[b]), int(num_accepted[b]), int(gamma_used[b]))
                     for b in range(B)], dtype=np.int64)
    g = np.array([gamma_of(int(hist[b]), None if temp_target is None else float(temp_target[b]),
                           couple_temperature) for b in range(B)], dtype=np.int64)
    off = np.zeros(B + 1, dtype=np.int64)
    off[1:] = np.cumsum(g)
    return hist, g, off
