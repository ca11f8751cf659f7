"""Pins of the KV-cache commit oracle.

The cache invariant the pages ask for (cf-1 §3.3: keep the accepted
positions, drop everything after the accept point, test all-accept and
all-reject first) is checked against a model of what an autoregressive
decoder would have cached: the entry at slot s is a fixed function of the
token at s and of s itself.  The tree forward pass computes each node's
entry at its own position (prefix length + depth) and stores it at slot
L + node; after the commit every slot below the new length must hold the
entry of the token the decoder sees there.
"""

import numpy as np

import oracle
from oracle import tree as TR
from oracle.kv import commit_row_plan, kv_commit
import synth

LAYERS, H, D = 2, 3, 8


def entry(token, pos, layer, head, which):
    """Deterministic stand-in for a K or V vector of `token` at position `pos`."""
    rng = np.random.default_rng([int(token), int(pos), layer, head, which])
    return rng.standard_normal(D)


def fill_round(B, S_max, L, seq_prefix, parents, tokens, depth):
    """Caches holding the prefix and the round's nodes as the forward pass wrote them."""
    k = np.full((LAYERS, B, H, S_max, D), np.nan)
    v = np.full((LAYERS, B, H, S_max, D), np.nan)
    for b in range(B):
        for s in range(L[b]):
            for l in range(LAYERS):
                for h in range(H):
                    k[l, b, h, s] = entry(seq_prefix[b][s], s, l, h, 0)
                    v[l, b, h, s] = entry(seq_prefix[b][s], s, l, h, 1)
        for node in range(len(parents[b])):
            pos = L[b] + depth[b][node]
            for l in range(LAYERS):
                for h in range(H):
                    k[l, b, h, L[b] + node] = entry(tokens[b][node], pos, l, h, 0)
                    v[l, b, h, L[b] + node] = entry(tokens[b][node], pos, l, h, 1)
    return k, v


def depths(parents):
    d = [0] * len(parents)
    for i in range(1, len(parents)):
        d[i] = d[parents[i]] + 1
    return d


def test_commit_matches_autoregressive_cache_after_tree_verify():
    d = synth.peaked_tree(seed=60, B=12, N=21, V=64)
    B, N = d["B"], d["N"]
    rng = np.random.default_rng(61)
    L = rng.integers(0, 6, size=B)
    S_max = int(L.max()) + N + 3
    prefix = [list(rng.integers(0, 64, size=int(L[b]))) for b in range(B)]
    toks = d["tokens"].copy()
    toks[:, 0] = rng.integers(0, 64, size=B)    # the root: the last committed token
    par = [list(d["parents"][b]) for b in range(B)]
    dep = [depths(p) for p in par]
    k, v = fill_round(B, S_max, L, prefix, par, toks, dep)
    n_acc, path, out, p_at, st, res = oracle.verify_tree_topk(
        d["target"], d["dtype"], d["parents"], toks, None, d["temp_target"], seed=3, step=1)
    assert max(n_acc) >= 2
    k2, v2, new_len = kv_commit(k, v, L, n_acc, path, N)
    for b in range(B):
        n = int(n_acc[b])
        assert new_len[b] == L[b] + 1 + n
        seq = list(prefix[b]) + [toks[b, 0]] + [toks[b, path[b][i]] for i in range(n)]
        assert len(seq) == new_len[b]
        for s, t in enumerate(seq):
            for l in range(LAYERS):
                for h in range(H):
                    assert np.array_equal(k2[l, b, h, s], entry(t, s, l, h, 0))
                    assert np.array_equal(v2[l, b, h, s], entry(t, s, l, h, 1))


def test_all_accept_and_all_reject_chains():
    """A linear round (a chain): nothing moves; the length counts the accepted drafts."""
    B, N, S_max = 3, 6, 20
    rng = np.random.default_rng(62)
    k = rng.standard_normal((1, B, 2, S_max, 4))
    v = rng.standard_normal((1, B, 2, S_max, 4))
    L = np.array([0, 7, 14])
    for n_acc in ([5, 5, 5], [0, 0, 0], [5, 0, 3]):
        k2, v2, nl = kv_commit(k, v, L, np.array(n_acc), None, N)
        assert list(nl) == [L[b] + 1 + n_acc[b] for b in range(B)]
        assert np.array_equal(k2, k) and np.array_equal(v2, v)


def test_error_and_invalid_rows():
    N, S = 5, 12
    assert commit_row_plan(4, -1, [1, 2], N, S) == (4, [])          # flagged by the verify step
    assert commit_row_plan(8, 2, [1, 2], N, S) == (-1, [])          # L + N > S_max
    assert commit_row_plan(2, 2, [2, 2], N, S) == (-1, [])          # not increasing
    assert commit_row_plan(2, 2, [1, 5], N, S) == (-1, [])          # node id out of range
    assert commit_row_plan(2, 5, [1, 2, 3, 4, 5], N, S) == (-1, [])  # depth > N - 1
    assert commit_row_plan(2, 2, [2, 4], N, S) == (5, [(4, 3), (6, 4)])


def test_moves_read_the_entries_as_they_were():
    """path [2, 3]: slot L+3 is both a source and a destination."""
    k = np.arange(10, dtype=np.float64).reshape(1, 1, 1, 10, 1)
    k2, _, nl = kv_commit(k, k, [1], [2], [[2, 3]], 5)
    assert nl[0] == 4
    assert list(k2[0, 0, 0, :4, 0]) == [0, 1, 3, 4]
