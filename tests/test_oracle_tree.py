"""Pins of the tree-verify oracle.

* TOPK: exact enumeration of the walk at V=5, depth 2, width 2 and 3: the
  first emitted token follows the root's target softmax, and the whole
  round is consistent with autoregressive sampling from the target (the
  pages require the tree path to preserve the target law the way the
  linear verify does: kwkr §5.3, lonae tree-attention paragraph);
* SAMPLED_WOR: children drawn from q without replacement, exact enumeration
  over the draws and the walk: same two properties;
* a chain-shaped tree equals the linear verify with a greedy draft
  (temp_draft = 0, drafts = draft argmax), output for output;
* greedy trees accept exactly the child equal to the target argmax.
"""

import itertools

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import linear as L
from oracle import tree as TR
from exact_law import ALMOST_ONE, ar_consistency_error, law_distance, segments
from test_oracle_linear import ContextTable, lib_softmax


def build_topk_tree(tab, width, depth, Td=1.0):
    ctxs, parents, tokens = [()], [-1], [0]
    frontier = [0]
    for _ in range(depth):
        nxt = []
        for n in frontier:
            q = lib_softmax(tab.draft(ctxs[n]), Td)
            order = sorted(range(tab.V), key=lambda v: (-q[v], v))[:width]
            for v in order:
                ctxs.append(ctxs[n] + (v,))
                parents.append(n)
                tokens.append(v)
                nxt.append(len(ctxs) - 1)
        frontier = nxt
    x = np.array([tab.target(c) for c in ctxs])
    return ctxs, parents, tokens, x


def walk_law(run, parents, tokens, N):
    """Exact law of the sequence one tree round emits; run(u_acc, u_smp) -> TreeRowResult."""
    law = {}

    def explore(node, depth, prob, fixed, path_tokens):
        kids = [c for c in range(1, N) if parents[c] == node]
        rej = 1.0
        fixed = dict(fixed)
        for c in kids:
            def accepted(u, c=c, fixed=fixed):
                ua = [ALMOST_ONE] * N
                for k, v in fixed.items():
                    ua[k] = v
                ua[c] = u
                r = run(ua, [0.5] * N)
                return r.num_accepted > depth and r.path_nodes[depth] == c
            A = segments(accepted).get(True, 0.0)
            if A > 0.0:
                explore(c, depth + 1, prob * rej * A, {**fixed, c: 0.0},
                        path_tokens + (tokens[c],))
            rej *= 1.0 - A
            fixed[c] = ALMOST_ONE
            if rej == 0.0:
                break
        if rej > 0.0:
            def emitted(us, fixed=fixed):
                ua = [ALMOST_ONE] * N
                for k, v in fixed.items():
                    ua[k] = v
                usm = [0.5] * N
                usm[node] = us
                return int(run(ua, usm).out_tokens[depth])
            for v, pv in segments(emitted).items():
                s = path_tokens + (v,)
                law[s] = law.get(s, 0.0) + prob * rej * pv

    explore(0, 0, 1.0, {}, ())
    return law


def ar_of(tab, Tt):
    def ar(seq, ctx):
        pr, c = 1.0, tuple(ctx)
        for t in seq:
            pr *= lib_softmax(tab.target(c), Tt)[t]
            c = c + (t,)
        return pr
    return ar


@pytest.mark.parametrize("V,width,depth,seed,Tt", [(5, 2, 2, 21, 1.0), (5, 3, 2, 22, 0.8),
                                                    (4, 2, 3, 23, 1.2)])
def test_topk_walk_law_is_autoregressive(V, width, depth, seed, Tt):
    tab = ContextTable(V, seed, pert=1.0)
    ctxs, parents, tokens, x = build_topk_tree(tab, width, depth)
    N = len(ctxs)

    def run(ua, us):
        return TR.verify_tree_topk_row(x, parents, tokens, N, Tt, ua, us)

    law = walk_law(run, parents, tokens, N)
    assert abs(sum(law.values()) - 1.0) < 1e-10
    first = {}
    for s, pr in law.items():
        first[s[0]] = first.get(s[0], 0.0) + pr
    assert law_distance(first, lib_softmax(x[0], Tt)) < 1e-10
    assert ar_consistency_error(law, ar_of(tab, Tt), depth + 1) < 1e-10


def test_topk_negative_control_unmasked_residual(monkeypatch):
    """Drawing from p without removing the rejected children must break the law."""
    tab = ContextTable(5, 21, pert=1.0)
    ctxs, parents, tokens, x = build_topk_tree(tab, 2, 1)
    N = len(ctxs)
    orig = TR.verify_tree_topk_row

    def unmasked(x, parents, tokens, n, Tt, ua, us):
        r = orig(x, parents, tokens, n, Tt, ua, us)
        if r.stop_kind == "reject":   # replace the draw with an unmasked one from p
            k, _ = L.inverse_cdf(L.softmax_t(x[r.stop_node], Tt), us[r.stop_node])
            r.out_tokens[r.num_accepted] = k
        return r

    law = walk_law(lambda ua, us: unmasked(x, parents, tokens, N, 1.0, ua, us),
                   parents, tokens, N)
    first = {}
    for s, pr in law.items():
        first[s[0]] = first.get(s[0], 0.0) + pr
    assert law_distance(first, lib_softmax(x[0], 1.0)) > 1e-3


def wor_draws(q, k):
    """All ordered k-draws without replacement from q with their probabilities."""
    out = []
    for perm in itertools.permutations(range(len(q)), k):
        pr, left = 1.0, 1.0
        for v in perm:
            if left <= 0:
                pr = 0.0
                break
            pr *= q[v] / left
            left -= q[v]
        if pr > 0:
            out.append((perm, pr))
    return out


@pytest.mark.parametrize("V,k,seed,Tt,Td", [(4, 2, 31, 1.0, 1.0), (4, 3, 32, 0.9, 1.1),
                                            (5, 2, 33, 1.0, 0.7)])
def test_sampled_wor_law_is_autoregressive(V, k, seed, Tt, Td):
    tab = ContextTable(V, seed, pert=1.0)
    q_root = lib_softmax(tab.draft(()), Td)
    total = {}
    for draw, pr in wor_draws(q_root, k):
        ctxs = [()] + [(v,) for v in draw]
        parents = [-1] + [0] * k
        tokens = [0] + list(draw)
        x = np.array([tab.target(c) for c in ctxs])
        y = np.array([tab.draft(c) for c in ctxs])
        N = len(ctxs)

        def run(ua, us):
            return TR.verify_tree_sampled_wor_row(x, y, parents, tokens, N, Tt, Td, ua, us)

        for s, ps in walk_law(run, parents, tokens, N).items():
            total[s] = total.get(s, 0.0) + pr * ps
    assert abs(sum(total.values()) - 1.0) < 1e-10
    first = {}
    for s, p in total.items():
        first[s[0]] = first.get(s[0], 0.0) + p
    assert law_distance(first, lib_softmax(tab.target(()), Tt)) < 1e-10
    assert ar_consistency_error(total, ar_of(tab, Tt), 2) < 1e-10


def test_topk_rule_with_draft_q_is_lossy():
    """Using the draft q (not a point mass) with deterministic top-k children is lossy,
    which is why TOPK mode takes q = delta (plain enumeration, planted on the CPU)."""
    tab = ContextTable(5, 21, pert=1.0)
    ctxs, parents, tokens, x = build_topk_tree(tab, 2, 1)
    y = np.array([tab.draft(c) for c in ctxs])
    N = len(ctxs)

    def run(ua, us):
        return TR.verify_tree_sampled_wor_row(x, y, parents, tokens, N, 1.0, 1.0, ua, us)

    law = walk_law(run, parents, tokens, N)
    first = {}
    for s, pr in law.items():
        first[s[0]] = first.get(s[0], 0.0) + pr
    assert law_distance(first, lib_softmax(x[0], 1.0)) > 1e-2


def chain_inputs(rng, gamma, V):
    x = rng.normal(0, 1.5, size=(gamma + 1, V))
    y = rng.normal(0, 1.5, size=(gamma, V))
    d = np.argmax(y, axis=1)
    # make acceptance likely so deep chains occur
    for i in range(gamma):
        x[i, d[i]] = x[i].max() + rng.uniform(0, 6)
    return x, y, d


def test_chain_tree_equals_linear_with_greedy_draft():
    rng = np.random.default_rng(40)
    gamma, V = 6, 64
    depths = []
    for trial in range(60):
        x, y, d = chain_inputs(rng, gamma, V)
        parents = [-1] + list(range(gamma))
        tokens = [0] + list(d)
        Tt = [1.0, 0.7, 1.3][trial % 3]
        u_acc, u_smp = oracle.verify_uniforms(trial, 2, 5, gamma + 1)
        lin = L.verify_linear_row(x, y, d, Tt, 0.0, u_acc, u_smp)
        tr = TR.verify_tree_topk_row(x, parents, tokens, gamma + 1, Tt, u_acc, u_smp)
        assert lin.num_accepted == tr.num_accepted
        assert np.array_equal(lin.out_tokens, tr.out_tokens)
        assert list(tr.path_nodes[:tr.num_accepted]) == list(range(1, tr.num_accepted + 1))
        depths.append(tr.num_accepted)
    assert len(set(depths)) >= 4


def test_sampled_wor_chain_equals_linear_with_draft_q():
    """A chain has one child per node, so q_j = q and p_j = p at every test:
    SAMPLED_WOR reduces to the linear verify with the draft's own q."""
    rng = np.random.default_rng(44)
    gamma, V = 5, 48
    depths = []
    for trial in range(80):
        x = rng.normal(0, 1.5, size=(gamma + 1, V))
        y = x[:gamma] + rng.normal(0, 0.4, size=(gamma, V))
        Tt, Td = [(1.0, 1.0), (0.8, 1.2), (1.3, 0.6), (0.0, 1.0)][trial % 4]
        d = np.array([rng.choice(V, p=lib_softmax(y[i], Td)) for i in range(gamma)])
        yt = np.vstack([y, rng.normal(0, 1.5, size=(1, V))])   # the leaf's draft row is unused
        parents = [-1] + list(range(gamma))
        tokens = [0] + list(d)
        u_acc, u_smp = oracle.verify_uniforms(trial, 3, 7, gamma + 1)
        lin = L.verify_linear_row(x, y, d, Tt, Td, u_acc, u_smp)
        tr = TR.verify_tree_sampled_wor_row(x, yt, parents, tokens, gamma + 1, Tt, Td,
                                            u_acc, u_smp)
        assert lin.num_accepted == tr.num_accepted
        if not tr.flagged_sample:
            assert np.array_equal(lin.out_tokens, tr.out_tokens)
        assert list(tr.path_nodes[:tr.num_accepted]) == list(range(1, tr.num_accepted + 1))
        for i in range(gamma):
            assert tr.p_at_node[i + 1] == lin.p_at_draft[i]
        depths.append(tr.num_accepted)
    assert len(set(depths)) >= 4


def test_sampled_wor_error_and_warning_rows():
    V = 6
    x = np.zeros((4, V))
    y = np.zeros((4, V))
    u = [0.5] * 4
    par, tok = [-1, 0, 0, 1], [0, 1, 2, 3]
    run = TR.verify_tree_sampled_wor_row
    assert run(x, y, par, tok, 4, 1.0, -1.0, u, u).status == L.ROW_BAD_TEMP
    assert run(x, y, [-1, 0, 3, 1], tok, 4, 1.0, 1.0, u, u).status == L.ROW_BAD_SHAPE
    assert run(x, y, par, [0, 1, 2, V], 4, 1.0, 1.0, u, u).status == L.ROW_BAD_TOKEN
    xb = x.copy()
    xb[3] = -np.inf          # the walk (accepting 1, then 3) stops at leaf 3: its bonus draw reads it
    assert run(xb, y, par, tok, 4, 1.0, 1.0, u, u).status == L.ROW_NONFINITE
    yb = y.copy()
    yb[1] = -np.inf          # node 1 has a child, so its draft row is read
    assert run(x, yb, par, tok, 4, 1.0, 1.0, u, u).status == L.ROW_NONFINITE
    yb = y.copy()
    yb[2] = -np.inf          # leaves' draft rows are never read
    assert run(x, yb, par, tok, 4, 1.0, 1.0, u, u).status == L.ROW_OK
    yq = y.copy()
    yq[0, 1] = -np.inf       # child token 1 impossible under the root's draft
    r = run(x, yq, par, tok, 4, 1.0, 1.0, [0.5, 0.999, 0.999, 0.999], u)
    assert r.status & L.ROW_WARN_QZERO and r.num_accepted >= 1 and r.path_nodes[0] == 1


def test_leaf_target_rows_read_only_by_a_bonus_draw():
    """A leaf's target row is read only when the walk stops at that leaf (its
    bonus draw): a row without a finite maximum elsewhere among the leaves is
    never read, in both candidate modes; an inner node's row always is."""
    V = 6
    x = np.zeros((4, V))
    y = np.zeros((4, V))
    par, tok = [-1, 0, 0, 1], [0, 1, 2, 3]
    us = [0.5] * 4
    to_3 = [0.5, 0.01, 0.99, 0.01]     # accept 1 (ratio 1/6), then 3: stop at leaf 3
    to_2 = [0.5, 0.99, 0.01, 0.99]     # reject 1, accept 2 (ratio 1/5): stop at leaf 2
    bad2 = x.copy()
    bad2[2] = -np.inf
    bad2n = x.copy()
    bad2n[2, 4] = np.nan
    for row in (bad2, bad2n):
        r = TR.verify_tree_topk_row(row, par, tok, 4, 1.0, to_3, us)
        assert r.status == L.ROW_OK and r.num_accepted == 2 and r.stop_node == 3
        r = TR.verify_tree_topk_row(row, par, tok, 4, 1.0, to_2, us)
        assert r.status == L.ROW_NONFINITE and r.num_accepted == -1
        assert np.all(r.out_tokens == -1) and np.all(r.path_nodes == -1)
    # SAMPLED_WOR with uniform p and q: every ratio is 1
    wor_3 = [0.5, 0.5, 0.99, 0.5]      # accept 1, then 3
    r = TR.verify_tree_sampled_wor_row(bad2, y, par, tok, 4, 1.0, 1.0, wor_3, us)
    assert r.status == L.ROW_OK and r.stop_node == 3
    r = TR.verify_tree_sampled_wor_row(bad2, y, [-1, 0, 0, 0], tok, 4, 1.0, 1.0,
                                       [0.5, 1.5, 0.5, 0.5], us)
    assert r.status == L.ROW_NONFINITE        # node 1 rejected, node 2 accepted: leaf 2
    # an inner node's target row is read whatever the walk does
    bad1 = x.copy()
    bad1[1] = -np.inf
    assert TR.verify_tree_topk_row(bad1, par, tok, 4, 1.0, to_2, us).status == L.ROW_NONFINITE
    assert TR.verify_tree_sampled_wor_row(bad1, y, par, tok, 4, 1.0, 1.0, wor_3,
                                          us).status == L.ROW_NONFINITE
    # a tree of the root alone: the root is the leaf the walk stops at
    r = TR.verify_tree_topk_row(bad2[2:3].repeat(4, 0), par, tok, 1, 1.0, to_3, us)
    assert r.status == L.ROW_NONFINITE


def test_greedy_tree_accepts_target_argmax_child():
    rng = np.random.default_rng(41)
    V = 16
    tab = ContextTable(V, 42)
    ctxs, parents, tokens, x = build_topk_tree(tab, 3, 2)
    N = len(ctxs)
    for trial in range(20):
        xx = x + rng.normal(0, 0.01, size=x.shape)
        u_acc, u_smp = oracle.verify_uniforms(trial, 0, 0, N)
        r = TR.verify_tree_topk_row(xx, parents, tokens, N, 0.0, u_acc, u_smp)
        node, depth = 0, 0
        while True:
            a = int(np.argmax(xx[node]))
            kids = [c for c in range(1, N) if parents[c] == node]
            hit = [c for c in kids if tokens[c] == a]
            if not hit:
                assert r.out_tokens[depth] == a and r.num_accepted == depth
                break
            assert r.path_nodes[depth] == hit[0]
            node, depth = hit[0], depth + 1


def test_tree_error_rows():
    x = np.zeros((3, 4))
    u = [0.5] * 3
    assert TR.verify_tree_topk_row(x, [-1, 0, 2], [0, 1, 2], 3, 1.0, u, u).status == L.ROW_BAD_SHAPE
    assert TR.verify_tree_topk_row(x, [-1, 0, 0], [0, 1, 9], 3, 1.0, u, u).status == L.ROW_BAD_TOKEN
    r = TR.verify_tree_topk_row(x, [-1, 0, 0], [0, 1, 2], 2, 1.0, u, u)
    assert r.status == 0 and r.num_accepted in (0, 1)


def test_tree_batch_p_at_node():
    rng = np.random.default_rng(43)
    B, N, V = 3, 7, 20
    tgt = rng.normal(0, 2, size=(B, N, V)).astype(np.float32)
    parents = np.tile(np.array([-1, 0, 0, 1, 1, 2, 2]), (B, 1))
    toks = rng.integers(0, V, size=(B, N))
    T = np.array([1.0, 0.5, 0.0], dtype=np.float32)
    n_acc, path, out, p_at, st, res = oracle.verify_tree_topk(tgt, 0, parents, toks, None, T)
    for b in range(B):
        for n in range(1, N):
            p = lib_softmax(tgt[b, parents[b, n]].astype(np.float64), float(T[b]))
            assert abs(p_at[b, n] - p[toks[b, n]]) <= 1e-12 * max(1.0, p[toks[b, n]])
        assert st[b] == 0 and 0 <= n_acc[b] <= 2
