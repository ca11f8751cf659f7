"""Pins of the verify-attention oracle.

* against torch.nn.functional.scaled_dot_product_attention (float32 on the
  CPU, explicit boolean mask built from the tree);
* a single query with no new-token mask is plain softmax(q K^T / sqrt(d)) V;
* a chain-shaped tree gives exactly the causal mask;
* jointly permuting the prefix keys and values leaves the output unchanged.
"""

import numpy as np
import torch

from oracle.attention import ancestor_mask, attention_head, verify_attention


def rand_case(rng, B=2, H=3, N=7, d=16, L=(10, 4), S=24):
    q = rng.normal(size=(B, H, N, d))
    k = rng.normal(size=(B, H, S, d))
    v = rng.normal(size=(B, H, S, d))
    return q, k, v, np.array(L)


def sdpa_reference(q, k, v, prefix_len, parents):
    B, H, N, d = q.shape
    out = np.zeros_like(q)
    for b in range(B):
        L = int(prefix_len[b])
        allowed = np.zeros((N, L + N), dtype=bool)
        allowed[:, :L] = True
        allowed[:, L:] = ancestor_mask(None if parents is None else parents[b], N)
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q[b], dtype=torch.float32),
            torch.tensor(k[b, :, :L + N], dtype=torch.float32),
            torch.tensor(v[b, :, :L + N], dtype=torch.float32),
            attn_mask=torch.tensor(allowed))
        out[b] = o.numpy()
    return out


def test_matches_torch_sdpa_tree_mask():
    rng = np.random.default_rng(0)
    q, k, v, L = rand_case(rng)
    parents = np.array([[-1, 0, 0, 1, 1, 2, 3], [-1, 0, 1, 2, 0, 4, 4]])
    o, _ = verify_attention(q, k, v, L, parents)
    assert np.max(np.abs(o - sdpa_reference(q, k, v, L, parents))) < 1e-5


def test_matches_torch_sdpa_causal():
    rng = np.random.default_rng(1)
    q, k, v, L = rand_case(rng, L=(0, 17))
    o, _ = verify_attention(q, k, v, L, None)
    assert np.max(np.abs(o - sdpa_reference(q, k, v, L, None))) < 1e-5


def test_single_query_is_plain_softmax_attention():
    rng = np.random.default_rng(2)
    d, L = 32, 50
    q = rng.normal(size=(1, d))
    k = rng.normal(size=(L + 1, d))
    v = rng.normal(size=(L + 1, d))
    o, lse = attention_head(q, k, v, L, np.ones((1, 1), dtype=bool), 1 / np.sqrt(d))
    s = (k @ q[0]) / np.sqrt(d)
    w = np.exp(s - s.max())
    assert np.allclose(o[0], (w / w.sum()) @ v, atol=1e-13)
    assert abs(lse[0] - (s.max() + np.log(w.sum()))) < 1e-12


def test_chain_tree_equals_causal():
    rng = np.random.default_rng(3)
    q, k, v, L = rand_case(rng)
    chain = np.tile(np.arange(-1, 6), (2, 1))
    o1, l1 = verify_attention(q, k, v, L, chain)
    o2, l2 = verify_attention(q, k, v, L, None)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_prefix_permutation_invariance():
    rng = np.random.default_rng(4)
    q, k, v, L = rand_case(rng, L=(12, 12))
    parents = np.array([[-1, 0, 0, 1, 2, 2, 5]] * 2)
    o1, _ = verify_attention(q, k, v, L, parents)
    perm = rng.permutation(12)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, :12] = k[:, :, perm]
    v2[:, :, :12] = v[:, :, perm]
    o2, _ = verify_attention(q, k2, v2, L, parents)
    assert np.max(np.abs(o1 - o2)) < 1e-12


def test_ancestor_mask_counts():
    parents = [-1, 0, 0, 1, 1, 2, 2]
    m = ancestor_mask(parents, 7)
    assert m.sum(axis=1).tolist() == [1, 2, 2, 3, 3, 3, 3]
    assert np.array_equal(ancestor_mask(None, 4), np.tril(np.ones((4, 4), dtype=bool)))
