"""Drafting helpers on the device side of a round (oracle; test infrastructure).

The tree-attention paragraphs of blog.lonae.com/posts/2026-draft-model-kv-
jDwzYp build the round's tree from the draft: every draft position branches
into the draft's top-k candidates (or temperature samples), the tree is
gamma levels deep, and in production it is pruned rather than fully
expanded (the page keeps nodes by cumulative draft probability, up to a node
budget).

* topk_candidates: the k tokens of largest logit in a draft row (ties to the
  lower token id), with their log-probabilities log softmax(x / T) (T = 0: a
  one-hot draft, log 1 for the argmax and -inf for the rest).
* prune_tree: from a forest of drafted candidates (each with its parent,
  token and log q under the parent's draft row, parents listed before their
  children), keep the n_max - 1 candidates of largest cumulative log q
  (the sum along the path from the root) whose parent is kept, preferring on
  ties the shallower candidate, then the earlier parent, then the lower
  sibling rank; renumber the kept nodes breadth first (depth, then the new
  index of the parent, then sibling rank) behind the root, node 0.  Also
  counts kept nodes whose cumulative probability reaches tau.
"""

import numpy as np


def topk_candidates(x, k, temp):
    """x: [V] float64 logits; returns (tokens [k] int64, logprob [k] float64)."""
    x = np.asarray(x, dtype=np.float64)
    V = len(x)
    order = sorted(range(V), key=lambda v: (-x[v], v))[:k]
    if temp == 0.0:
        lp = np.array([0.0 if i == 0 else -np.inf for i in range(len(order))])
    else:
        z = x / temp
        m = np.max(z)
        lse = m + np.log(np.sum(np.exp(z - m)))
        lp = np.array([z[v] - lse for v in order])
    return np.array(order, dtype=np.int64), lp


def prune_tree(parent, token, logq, n_max, tau=0.1):
    """parent[i] in [-1, i) (-1: child of the root), token[i], logq[i]: one candidate forest.

    Returns (parents [n], tokens [n], cum_logprob [n], n_pass_tau) of the kept tree
    in breadth-first order, node 0 being the root (token -1, cum 0).
    """
    C = len(parent)
    depth = np.zeros(C, dtype=np.int64)
    cum = np.zeros(C)
    rank = np.zeros(C, dtype=np.int64)
    seen = {}
    for i in range(C):
        p = int(parent[i])
        depth[i] = 1 if p < 0 else depth[p] + 1
        cum[i] = logq[i] + (0.0 if p < 0 else cum[p])
        rank[i] = seen.get(p, 0)
        seen[p] = rank[i] + 1
    order = sorted(range(C), key=lambda i: (-cum[i], depth[i], int(parent[i]), rank[i]))
    kept = []
    keep = np.zeros(C, dtype=bool)
    for i in order:
        if len(kept) >= n_max - 1:
            break
        p = int(parent[i])
        if cum[i] == -np.inf:
            continue
        if p < 0 or keep[p]:
            keep[i] = True
            kept.append(i)
    # breadth-first renumbering
    new = {-1: 0}
    out = [-1]
    for d in range(1, int(depth.max(initial=0)) + 1):
        level = [i for i in kept if depth[i] == d]
        level.sort(key=lambda i: (new[int(parent[i])], rank[i]))
        for i in level:
            new[i] = len(out)
            out.append(i)
    n = len(out)
    parents = np.array([-1] + [new[int(parent[i])] for i in out[1:]], dtype=np.int64)
    tokens = np.array([-1] + [int(token[i]) for i in out[1:]], dtype=np.int64)
    cl = np.array([0.0] + [cum[i] for i in out[1:]])
    n_pass = int(np.sum(np.exp(cl[1:]) >= tau))
    return parents, tokens, cl, n_pass
