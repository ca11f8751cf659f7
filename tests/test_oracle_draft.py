"""Pins of the drafting oracle: top-k against NumPy's stable sort and SciPy's
log-softmax, and tree pruning against the definition of the kept set (the
n_max - 1 candidates of largest cumulative draft probability, closed under
ancestors) and breadth-first order, plus a hand-made case with ties."""

import numpy as np
import scipy.special

from oracle import draft as D
import synth


def test_topk_matches_stable_sort_and_log_softmax():
    rng = np.random.default_rng(90)
    for trial in range(30):
        V = int(rng.integers(5, 300))
        x = synth.bf16_values(synth.bf16_bits(rng.normal(0, 2, size=V).astype(np.float32)))
        x = x.astype(np.float64)
        x[rng.integers(0, V, size=V // 4)] = x[0]          # plenty of ties
        k = int(rng.integers(1, min(V, 16) + 1))
        T = [1.0, 0.7, 1.3][trial % 3]
        tok, lp = D.topk_candidates(x, k, T)
        ref = np.lexsort((np.arange(V), -x))[:k]
        assert np.array_equal(tok, ref)
        ls = scipy.special.log_softmax(x / T)
        assert np.allclose(lp, ls[ref], rtol=0, atol=1e-12)
    tok, lp = D.topk_candidates(np.array([1.0, 3.0, 3.0, 2.0]), 3, 0.0)
    assert list(tok) == [1, 2, 3] and lp[0] == 0.0 and np.all(np.isneginf(lp[1:]))


def full_forest(rng, V, width, depth):
    """Every node's top-`width` children, levels in order (parents before children)."""
    parent, token, logq = [], [], []
    frontier = [-1]
    for _ in range(depth):
        nxt = []
        for p in frontier:
            y = rng.normal(0, 2, size=V)
            tok, lp = D.topk_candidates(y, width, 1.0)
            for t, l in zip(tok, lp):
                parent.append(p)
                token.append(int(t))
                logq.append(l)
                nxt.append(len(parent) - 1)
        frontier = nxt
    return np.array(parent), np.array(token), np.array(logq)


def test_prune_keeps_the_top_cumulative_set_breadth_first():
    rng = np.random.default_rng(91)
    for n_max in (1, 8, 40, 64, 400):
        parent, token, logq = full_forest(rng, 50, 4, 4)
        par, tok, cum, npass = D.prune_tree(parent, token, logq, n_max)
        C = len(parent)
        n = len(par)
        assert n == min(n_max, C + 1)
        # cumulative log q of every candidate
        cum_all = np.zeros(C)
        for i in range(C):
            cum_all[i] = logq[i] + (cum_all[parent[i]] if parent[i] >= 0 else 0.0)
        kept = np.sort(cum[1:])[::-1]
        if n > 1:
            assert np.allclose(kept, np.sort(cum_all)[::-1][:n - 1], atol=0)
        # breadth-first: parents before children, depth non-decreasing, parents ordered
        d = np.zeros(n, dtype=int)
        for i in range(1, n):
            assert 0 <= par[i] < i
            d[i] = d[par[i]] + 1
        assert np.all(np.diff(d) >= 0)
        assert all(cum[i] <= cum[par[i]] for i in range(1, n))     # log q <= 0 along a path
        for i in range(2, n):
            if d[i] == d[i - 1]:
                assert par[i] >= par[i - 1]
        assert npass == int(np.sum(np.exp(cum[1:]) >= 0.1))


def test_prune_ties_and_impossible_candidates():
    # root children a (log 0), b (log 0), c (-inf); a's children tie with b's
    parent = np.array([-1, -1, -1, 0, 0, 1])
    token = np.array([10, 11, 12, 20, 21, 30])
    logq = np.array([0.0, 0.0, -np.inf, -1.0, -1.0, -1.0])
    par, tok, cum, _ = D.prune_tree(parent, token, logq, 5)
    # kept: a, b (depth 1), then the depth-2 ties in parent order, a's first: 20, 21
    assert list(tok) == [-1, 10, 11, 20, 21]
    assert list(par) == [-1, 0, 0, 1, 1]
    par, tok, cum, _ = D.prune_tree(parent, token, logq, 10)
    assert 12 not in tok                      # zero probability: never kept
    assert list(tok) == [-1, 10, 11, 20, 21, 30]


def test_topk_signed_zeros_are_one_value():
    # -0 and +0 compare equal as logits, so the lower id ranks first and
    # both carry the same log-probability
    tok, lp = D.topk_candidates(np.array([-1.0, -0.0, 0.0, -2.0]), 3, 1.0)
    assert tok.tolist() == [1, 2, 0]
    assert lp[0] == lp[1]
    assert abs(lp[0] - (0.0 - np.log(2.0 + np.exp(-1.0) + np.exp(-2.0)))) < 1e-15
