"""Trees at the limits the tree verify accepts (64 nodes: a root and 63 draft
nodes), over V=32000 bf16 rows, for the GPU parity tests.

* chains of 64 nodes whose target rows favour the next node's token by a
  margin of 13 to 24 logits, so walks accepted to depth 63 (Philox slot 63)
  sit beside walks that stop part-way;
* stars of 63 children of the root, so a walk tests up to 63 siblings in a
  row (the 63-sibling prefix sums of TOPK, the 63 residual passes of
  SAMPLED_WOR) before it draws from what is left.

TOPK children are given tokens (a point-mass draft); SAMPLED_WOR children are
Gumbel-top-k draws without replacement from the node's bf16 draft row.
"""

import numpy as np

import synth

V = 32000
N = 64


def _bf16(a):
    return synth.bf16_bits(np.asarray(a, dtype=np.float32))


def _vals(bits):
    return synth.bf16_values(bits).astype(np.float64)


def _gumbel_topk(rng, logits, T, k):
    z = logits / T + rng.gumbel(size=logits.shape)
    return np.argsort(-z, kind="stable")[:k]


def _tree(kind, B, target, draft, parents, tokens, T, seed):
    d = dict(kind=kind, dtype=synth.BF16, B=B, N=N, V=V, target=target, parents=parents,
             tokens=tokens, n_nodes=None, temp_target=np.full(B, T, np.float32), seed=seed,
             step=3)
    if kind == "tree_wor":
        d["draft"] = draft
        d["temp_draft"] = np.full(B, T, np.float32)
    return d


def topk_chain(seed=41, B=16):
    rng = np.random.default_rng(seed)
    parents = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    tokens = rng.integers(0, V, size=(B, N)).astype(np.int32)
    tokens[:, 0] = 0
    x = rng.normal(0, 1, size=(B, N, V)).astype(np.float32)
    margin = np.array([24.0, 24.0, 15.0, 13.0])[np.arange(B) % 4]
    for b in range(B):
        for n in range(N - 1):
            x[b, n, tokens[b, n + 1]] = margin[b] + rng.normal(0, 0.2)
    return _tree("tree", B, _bf16(x), None, parents, tokens, 1.0, seed)


def topk_star(seed=42, B=32):
    rng = np.random.default_rng(seed)
    parents = np.zeros((B, N), dtype=np.int32)
    parents[:, 0] = -1
    tokens = np.zeros((B, N), dtype=np.int32)
    x = rng.normal(0, 1, size=(B, N, V)).astype(np.float32)
    for b in range(B):
        kids = rng.choice(V, size=N - 1, replace=False)
        tokens[b, 1:] = kids
        # 63 children of about 0.5-1% each: most walks reject every sibling
        x[b, 0, kids] = rng.normal(6.5, 0.4, size=N - 1)
    return _tree("tree", B, _bf16(x), None, parents, tokens, 1.0, seed)


def wor_chain(seed=43, B=16):
    rng = np.random.default_rng(seed)
    parents = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    yb = _bf16(rng.normal(0, 2, size=(B, N, V)))
    y = _vals(yb)
    tokens = np.zeros((B, N), dtype=np.int32)
    x = y + rng.normal(0, 0.7, size=(B, N, V))
    boost = np.array([30.0, 30.0, 8.0, 0.0])[np.arange(B) % 4]
    for b in range(B):
        for n in range(N - 1):
            c = int(_gumbel_topk(rng, y[b, n], 1.0, 1)[0])
            tokens[b, n + 1] = c
            x[b, n, c] = y[b, n, c] + boost[b]
    return _tree("tree_wor", B, _bf16(x), yb, parents, tokens, 1.0, seed)


def wor_star(seed=44, B=32):
    rng = np.random.default_rng(seed)
    parents = np.zeros((B, N), dtype=np.int32)
    parents[:, 0] = -1
    yb = _bf16(rng.normal(0, 3, size=(B, N, V)))
    y = _vals(yb)
    x = y + rng.normal(0, 4.0, size=(B, N, V))
    tokens = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        tokens[b, 1:] = _gumbel_topk(rng, y[b, 0], 1.0, N - 1)
    return _tree("tree_wor", B, _bf16(x), yb, parents, tokens, 1.0, seed)
