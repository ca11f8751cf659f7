"""Causal- or tree-masked verify attention, float64 (oracle; test infrastructure).

The target scores all draft positions in one forward pass; the causal mask
makes every position see exactly what it would see in step-by-step decoding
(kwkr §2.1).  For a token tree the mask is the tree's ancestor relation
(cf-1 §5.4 mentions the batch-verification mask matrix; the lonae
tree-attention paragraphs describe the per-tree-shape causal mask).

For batch row b with prefix length L = prefix_len[b] and N new tokens whose
keys/values sit at cache slots [L, L + N):

    O[b, h, i] = sum_j softmax_j(Q[b,h,i] . K[b,h,j] * scale + M_ij) V[b,h,j]

over j in [0, L) (the committed prefix, visible to every query) and
j = L + t for every new token t that is an ancestor of i or i itself
(M_ij = 0; every other key has M_ij = -inf).  With no parent array the new
tokens form a chain and the mask is causal.  LSE = log sum_j exp(score_ij).

Readings: scale is 1/sqrt(d); inputs are taken after any positional
encoding; every head has its own K/V (no grouping).
"""

import numpy as np


def ancestor_mask(parents, N):
    """[N, N] bool: mask[i, t] is True when t is i or an ancestor of i.

    parents=None gives a chain (t <= i).
    """
    if parents is None:
        return np.tril(np.ones((N, N), dtype=bool))
    m = np.zeros((N, N), dtype=bool)
    for i in range(N):
        j = i
        while j >= 0:
            m[i, j] = True
            j = int(parents[j]) if j > 0 else -1
    return m


def attention_head(q, k, v, L, mask, scale):
    """One (b, h): q [N, d], k/v [>= L+N, d] float64, mask [N, N] -> (O [N, d], LSE [N])."""
    N = q.shape[0]
    keys = k[:L + N]
    vals = v[:L + N]
    s = (q @ keys.T) * scale
    s[:, L:L + N] = np.where(mask, s[:, L:L + N], -np.inf)
    smax = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - smax)
    denom = np.sum(e, axis=1, keepdims=True)
    o = (e / denom) @ vals
    lse = (smax + np.log(denom))[:, 0]
    return o, lse


def verify_attention(q, k, v, prefix_len, parents=None, scale=None):
    """q: [B, H, N, d]; k, v: [B, H, S_max, d] (float64); parents: [B, N] or None.

    Returns O [B, H, N, d] and LSE [B, H, N] in float64.
    """
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        mask = ancestor_mask(None if parents is None else parents[b], N)
        L = int(prefix_len[b])
        for h in range(H):
            out[b, h], lse[b, h] = attention_head(q[b, h], k[b, h], v[b, h], L, mask, scale)
    return out, lse
