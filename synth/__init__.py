"""Seeded synthetic inputs for the verify step (shared by tests, bench and smoke).

This module only builds inputs: logits, draft tokens, temperatures, ragged
offsets, token trees and attention tensors.  It holds none of the verify
arithmetic; the randoms the verify step itself draws come from Philox inside
the oracle and inside the HIP library, never from here.

Workloads (all synthetic; the pages publish no dataset, suite or weights for
this step):

* ``linear_v1000``  B=1, gamma=4, V=1000, fp32.  Draft logits N(0, 2^2),
  target = draft + N(0, 0.5^2), T = 1, draft tokens drawn from the draft
  softmax.
* ``mc_v8``         the same generator at V=8, one fixed (p, q) pair repeated
  over n trials with gamma=1 (the distribution check).
* ``linear_v32k``   B=32, gamma=5, V=32000, bf16.  Draft N(0, 3^2), target =
  draft + N(0, sigma_b^2) with sigma_b ~ U[0.2, 1.5], T = 0.8.
* ``linear_v128k``  B=128, gamma=8, V=128256, bf16, sigma_b ~ U[0.1, 2.0],
  T_b uniform over {0.6, 0.8, 1.0}, 13 rows (10%) greedy (T = 0, draft token
  = draft argmax).
* ``tree_v32k``     B=64 token trees of at most 64 nodes (root included) over
  V=32000 bf16: best-first top-4 expansion to depth 4 by cumulative draft
  probability; node rows draft N(0, 2^2), target = draft + N(0, 0.5^2), T=1.
* ``tree_wor_v32k`` B=64 trees of at most 64 nodes over V=32000 bf16 whose
  children are 4 draws without replacement from the node's draft softmax
  (Gumbel-top-4 of the bf16 draft row), best-first by cumulative draft
  probability to depth 4; draft N(0, 2^2), target = draft + N(0, 0.5^2),
  T=1 for both (the SAMPLED_WOR candidate mode).
* ``attn_tree``     Q, K, V ~ N(0, 1) bf16, B=64, H=32, N=64, d=128, prefix
  L=4096 (cache length 4160), masked by the ``tree_v32k`` trees.
* ``bimodal_v152k`` B=256, V=152064 bf16; half the rows sigma=3.0, half
  sigma=0.3 (shuffled); draft N(0, 3^2); T=1; gamma_b in {2, 4, 8} from a
  16-step synthetic acceptance history (>60% -> 8, 30-60% -> 4, <30% -> 2);
  ragged rows packed by offsets.

The row layout matches the library: target rows of batch row b start at
offsets[b] + b, draft rows at offsets[b].
"""

import heapq

import numpy as np
import scipy.special

F32 = 0
BF16 = 1

# Dynamic speculation length from the acceptance rate over the last 16 steps
# (lonae bimodal-acceptance paragraph): above 60% -> 8, 30-60% -> 4, below 30% -> 2.
HISTORY_STEPS = 16


def gamma_from_history(accepted_steps, window=HISTORY_STEPS):
    rate = accepted_steps / window
    if rate > 0.6:
        return 8
    if rate >= 0.3:
        return 4
    return 2


def bf16_bits(x):
    """Round float32/float64 values to bf16 (round to nearest even); returns uint16 bits."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        c = flat_u[s:s + step]
        lsb = (c >> np.uint32(16)) & np.uint32(1)
        r = c + (np.uint32(0x7FFF) + lsb)      # NaN patterns may wrap; fixed below
        flat_o[s:s + step] = (r >> np.uint32(16)).astype(np.uint16)
        nan = (c & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        if nan.any():
            flat_o[s:s + step][nan] = 0x7FC0
    return out


def bf16_values(bits):
    """uint16 bf16 bits -> float32 values (for building inputs from rounded logits)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _gumbel_tokens(rng, logits, temps):
    """One draw per row from softmax(logits / T) by the Gumbel-max trick; T=0 -> argmax."""
    n, V = logits.shape
    out = np.empty(n, dtype=np.int32)
    temps = np.asarray(temps, dtype=np.float64)
    for s in range(0, n, 64):
        blk = logits[s:s + 64].astype(np.float64)
        T = temps[s:s + 64, None]
        g = rng.gumbel(size=blk.shape)
        z = np.where(T > 0, blk / np.where(T > 0, T, 1.0) + g, blk)
        out[s:s + 64] = np.argmax(z, axis=1)
    return out


def _linear_batch(rng, gammas, V, draft_sd, sigma, temps_t, temps_d, dtype):
    """Ragged linear batch; sigma and temps are per batch row."""
    gammas = np.asarray(gammas, dtype=np.int64)
    B = len(gammas)
    off = np.zeros(B + 1, dtype=np.int32)
    off[1:] = np.cumsum(gammas)
    n_d = int(off[-1])
    tgt = np.empty((n_d + B, V), dtype=np.float32)
    dft = np.empty((n_d, V), dtype=np.float32)
    for b in range(B):
        g = int(gammas[b])
        y = rng.standard_normal((g + 1, V), dtype=np.float32) * np.float32(draft_sd)
        x = y + rng.standard_normal((g + 1, V), dtype=np.float32) * np.float32(sigma[b])
        dft[off[b]:off[b + 1]] = y[:g]
        tgt[off[b] + b:off[b + 1] + b + 1] = x
    if dtype == BF16:
        tgt_s, dft_s = bf16_bits(tgt), bf16_bits(dft)
        dft_vals = bf16_values(dft_s)
    else:
        tgt_s, dft_s = tgt, dft
        dft_vals = dft
    row_td = np.repeat(np.asarray(temps_d, dtype=np.float32), gammas)
    toks = _gumbel_tokens(rng, dft_vals, row_td) if n_d else np.zeros(0, dtype=np.int32)
    return dict(kind="linear", dtype=dtype, B=B, V=V, target=tgt_s, draft=dft_s,
                offsets=off, tokens=toks,
                temp_target=np.asarray(temps_t, dtype=np.float32),
                temp_draft=np.asarray(temps_d, dtype=np.float32),
                gammas=gammas.astype(np.int32), seed=0, step=0)


def linear_v1000(seed=1):
    rng = np.random.default_rng(seed)
    T = np.ones(1, dtype=np.float32)
    return _linear_batch(rng, [4], 1000, 2.0, [0.5], T, T, F32)


def mc_v8(n_trials, seed=1):
    """n_trials rows with gamma=1 and one fixed (target, draft) logit pair at V=8."""
    rng = np.random.default_rng(seed)
    V = 8
    y = rng.standard_normal((1, V)).astype(np.float32) * np.float32(2.0)
    x0 = y + rng.standard_normal((1, V)).astype(np.float32) * np.float32(0.5)
    x1 = rng.standard_normal((1, V)).astype(np.float32) * np.float32(2.0)
    tgt = np.tile(np.vstack([x0, x1]), (n_trials, 1))
    dft = np.tile(y, (n_trials, 1))
    g = rng.gumbel(size=(n_trials, V))
    toks = np.argmax(y.astype(np.float64) + g, axis=1).astype(np.int32)
    off = np.arange(n_trials + 1, dtype=np.int32)
    T = np.ones(n_trials, dtype=np.float32)
    return dict(kind="linear", dtype=F32, B=n_trials, V=V, target=tgt, draft=dft, offsets=off,
                tokens=toks, temp_target=T, temp_draft=T.copy(),
                gammas=np.ones(n_trials, dtype=np.int32), seed=0, step=0,
                x0=x0[0], y0=y[0])


def linear_v32k(seed=2, B=32):
    rng = np.random.default_rng(seed)
    sigma = rng.uniform(0.2, 1.5, size=B)
    T = np.full(B, 0.8, dtype=np.float32)
    return _linear_batch(rng, [5] * B, 32000, 3.0, sigma, T, T, BF16)


def linear_v128k(seed=3, B=128, V=128256):
    rng = np.random.default_rng(seed)
    sigma = rng.uniform(0.1, 2.0, size=B)
    T = rng.choice(np.array([0.6, 0.8, 1.0], dtype=np.float32), size=B)
    greedy = rng.permutation(B)[:int(round(0.1 * B))]
    T[greedy] = 0.0
    return _linear_batch(rng, [8] * B, V, 3.0, sigma, T, T.copy(), BF16)


def bimodal_v152k(seed=5, B=256, V=152064):
    rng = np.random.default_rng(seed)
    sigma = np.where(rng.permutation(B) < B // 2, 3.0, 0.3)
    rate = np.where(sigma > 1.0, 0.10, 0.65)
    hist = rng.random((B, HISTORY_STEPS)) < rate[:, None]
    gammas = np.array([gamma_from_history(int(h.sum())) for h in hist])
    T = np.ones(B, dtype=np.float32)
    d = _linear_batch(rng, gammas, V, 3.0, sigma, T, T.copy(), BF16)
    d["sigma"] = sigma
    d["history_accepts"] = hist.sum(axis=1)
    return d


def build_topk_tree(rng, V, n_max=64, width=4, depth=4, draft_sd=2.0):
    """Best-first top-`width` expansion to `depth` by cumulative draft probability.

    Returns (draft_rows [n, V] float32, parents [n], tokens [n], depth [n],
    cum_prob [n]) in BFS order (depth, parent, rank), siblings in descending
    draft probability (ties -> lower token id).
    """
    rows, logq, sel = [], [], []
    heap = []

    def expand(idx):
        y = rows[idx]
        lq = scipy.special.log_softmax(y.astype(np.float64))
        order = np.lexsort((np.arange(V), -lq))[:width]
        for rank, tok in enumerate(order):
            cum = sel[idx][3] + lq[tok]
            heapq.heappush(heap, (-cum, sel[idx][1] + 1, idx, rank, int(tok)))

    rows.append(rng.standard_normal(V).astype(np.float32) * np.float32(draft_sd))
    sel.append((-1, 0, 0, 0.0, 0))   # (parent, depth, rank, cum_logprob, token)
    if depth > 0:
        expand(0)
    while len(sel) < n_max and heap:
        negcum, dep, parent, rank, tok = heapq.heappop(heap)
        rows.append(rng.standard_normal(V).astype(np.float32) * np.float32(draft_sd))
        sel.append((parent, dep, rank, -negcum, tok))
        if dep < depth:
            expand(len(sel) - 1)
    # BFS renumbering: depth, then new parent index, then sibling rank
    n = len(sel)
    new = {0: 0}
    order = [0]
    for dep in range(1, depth + 1):
        level = [i for i in range(n) if sel[i][1] == dep]
        level.sort(key=lambda i: (new[sel[i][0]], sel[i][2]))
        for i in level:
            new[i] = len(order)
            order.append(i)
    parents = np.array([-1] + [new[sel[i][0]] for i in order[1:]], dtype=np.int32)
    tokens = np.array([0] + [sel[i][4] for i in order[1:]], dtype=np.int32)
    depths = np.array([sel[i][1] for i in order], dtype=np.int32)
    cum = np.exp(np.array([sel[i][3] for i in order]))
    return np.stack([rows[i] for i in order]), parents, tokens, depths, cum


def tree_v32k(seed=4, B=64, N=64, V=32000, pert=0.5, draft_sd=2.0, temp=1.0, dtype=BF16):
    rng = np.random.default_rng(seed)
    tgt = np.empty((B, N, V), dtype=np.float32)
    parents = np.full((B, N), -1, dtype=np.int32)
    tokens = np.zeros((B, N), dtype=np.int32)
    n_nodes = np.zeros(B, dtype=np.int32)
    depth_hist = np.zeros(5, dtype=np.int64)
    passing = 0
    for b in range(B):
        y, par, tok, dep, cum = build_topk_tree(rng, V, N, draft_sd=draft_sd)
        n = len(par)
        x = y + rng.standard_normal(y.shape, dtype=np.float32) * np.float32(pert)
        tgt[b, :n] = x
        if n < N:
            tgt[b, n:] = rng.standard_normal((N - n, V), dtype=np.float32)
        parents[b, :n] = par
        tokens[b, :n] = tok
        n_nodes[b] = n
        depth_hist += np.bincount(dep, minlength=5)[:5]
        passing += int(np.sum(cum[1:] >= 0.1))
    tgt_s = bf16_bits(tgt) if dtype == BF16 else tgt
    T = np.full(B, temp, dtype=np.float32)
    return dict(kind="tree", dtype=dtype, B=B, N=N, V=V, target=tgt_s, parents=parents,
                tokens=tokens, n_nodes=n_nodes, temp_target=T, seed=0, step=0,
                depth_hist=depth_hist, nodes_passing_0p1=passing)


def build_wor_tree(rng, V, n_max=64, width=4, depth=4, draft_sd=2.0, temp=1.0, dtype=BF16):
    """Best-first expansion to `depth` of trees whose children are `width` draws
    without replacement from the node's draft softmax (temperature `temp`),
    ranked by cumulative draft probability along the path.

    Draws use the draft row as the verifier reads it (rounded to bf16 when
    dtype is BF16): the Gumbel-top-k of logits / temp, in draw order.
    Returns (draft_rows [n, V] float32 before rounding, parents [n],
    tokens [n], depth [n]) in BFS order (depth, parent, draw rank).
    """
    rows, sel = [], []
    heap = []

    def expand(idx):
        y = rows[idx]
        yv = bf16_values(bf16_bits(y)) if dtype == BF16 else y
        z = yv.astype(np.float64) / temp + rng.gumbel(size=V)
        order = np.lexsort((np.arange(V), -z))[:width]
        lq = scipy.special.log_softmax(yv.astype(np.float64) / temp)
        for rank, tok in enumerate(order):
            cum = sel[idx][3] + lq[tok]
            heapq.heappush(heap, (-cum, sel[idx][1] + 1, idx, rank, int(tok)))

    rows.append(rng.standard_normal(V).astype(np.float32) * np.float32(draft_sd))
    sel.append((-1, 0, 0, 0.0, 0))   # (parent, depth, rank, cum_logprob, token)
    if depth > 0:
        expand(0)
    while len(sel) < n_max and heap:
        negcum, dep, parent, rank, tok = heapq.heappop(heap)
        rows.append(rng.standard_normal(V).astype(np.float32) * np.float32(draft_sd))
        sel.append((parent, dep, rank, -negcum, tok))
        if dep < depth:
            expand(len(sel) - 1)
    n = len(sel)
    new = {0: 0}
    order = [0]
    for dep in range(1, depth + 1):
        level = [i for i in range(n) if sel[i][1] == dep]
        level.sort(key=lambda i: (new[sel[i][0]], sel[i][2]))
        for i in level:
            new[i] = len(order)
            order.append(i)
    parents = np.array([-1] + [new[sel[i][0]] for i in order[1:]], dtype=np.int32)
    tokens = np.array([0] + [sel[i][4] for i in order[1:]], dtype=np.int32)
    depths = np.array([sel[i][1] for i in order], dtype=np.int32)
    return np.stack([rows[i] for i in order]), parents, tokens, depths


def tree_wor(seed=7, B=64, N=64, V=32000, pert=0.5, draft_sd=2.0, temp=1.0, dtype=BF16,
             width=4, depth=4):
    """SAMPLED_WOR trees: children drawn from the draft without replacement."""
    rng = np.random.default_rng(seed)
    tgt = np.empty((B, N, V), dtype=np.float32)
    dft = np.empty((B, N, V), dtype=np.float32)
    parents = np.full((B, N), -1, dtype=np.int32)
    tokens = np.zeros((B, N), dtype=np.int32)
    n_nodes = np.zeros(B, dtype=np.int32)
    n_inner = 0
    for b in range(B):
        y, par, tok, dep = build_wor_tree(rng, V, N, width=width, depth=depth,
                                          draft_sd=draft_sd, temp=temp, dtype=dtype)
        n = len(par)
        x = y + rng.standard_normal(y.shape, dtype=np.float32) * np.float32(pert)
        tgt[b, :n] = x
        dft[b, :n] = y
        if n < N:
            tgt[b, n:] = rng.standard_normal((N - n, V), dtype=np.float32)
            dft[b, n:] = rng.standard_normal((N - n, V), dtype=np.float32)
        parents[b, :n] = par
        tokens[b, :n] = tok
        n_nodes[b] = n
        n_inner += len(set(par[1:].tolist()))
    if dtype == BF16:
        tgt_s, dft_s = bf16_bits(tgt), bf16_bits(dft)
    else:
        tgt_s, dft_s = tgt, dft
    T = np.full(B, temp, dtype=np.float32)
    return dict(kind="tree_wor", dtype=dtype, B=B, N=N, V=V, target=tgt_s, draft=dft_s,
                parents=parents, tokens=tokens, n_nodes=n_nodes, temp_target=T,
                temp_draft=T.copy(), seed=0, step=0, n_inner=n_inner)


def tree_wor_v32k(seed=7, B=64, N=64, V=32000):
    return tree_wor(seed=seed, B=B, N=N, V=V)


def peaked_tree(seed=6, B=32, N=21, V=64, draft_sd=6.0, pert=0.5, temp=1.0, dtype=F32):
    """Small trees whose target agrees with a peaked draft, so walks reach depth >= 2."""
    return tree_v32k(seed=seed, B=B, N=N, V=V, pert=pert, draft_sd=draft_sd, temp=temp,
                     dtype=dtype)


def attn_slice(seed, b, h, rows, d):
    rng = np.random.default_rng([seed, b, h])
    return bf16_bits(rng.standard_normal((rows, d), dtype=np.float32))


def attn_tensors(seed=4, B=64, H=32, N=64, d=128, L=4096, S_max=None):
    """Q [B,H,N,d] and K, V [B,H,S_max,d] as bf16 bits, each (b, h) slice seeded on its own."""
    S = L + N if S_max is None else S_max
    q = np.empty((B, H, N, d), dtype=np.uint16)
    k = np.empty((B, H, S, d), dtype=np.uint16)
    v = np.empty((B, H, S, d), dtype=np.uint16)
    for b in range(B):
        for h in range(H):
            q[b, h] = attn_slice(seed * 3 + 0, b, h, N, d)
            k[b, h] = attn_slice(seed * 3 + 1, b, h, S, d)
            v[b, h] = attn_slice(seed * 3 + 2, b, h, S, d)
    return q, k, v, np.full(B, L, dtype=np.int32)


def inner_nodes(d):
    """Nodes with children, summed over a tree batch's trees."""
    par = np.asarray(d["parents"])
    B, N = par.shape
    nn = np.full(B, N) if d.get("n_nodes") is None else np.asarray(d["n_nodes"])
    return int(sum(len({int(p) for p in par[b, 1:int(nn[b])] if p >= 0}) for b in range(B)))


def logits_bytes(d):
    """Bytes of the logit rows one verify call must read, each once: every row
    of a linear batch; in a tree, the target rows (and, with sampled children,
    the draft rows) of the nodes with children.  A leaf's row, read only when
    the walk stops at it, is not counted."""
    esize = 2 if d["dtype"] == BF16 else 4
    if d["kind"] == "linear":
        rows = d["target"].shape[0] + d["draft"].shape[0]
    elif d["kind"] == "tree_wor":
        rows = 2 * inner_nodes(d)
    else:
        rows = inner_nodes(d)
    return rows * d["V"] * esize


WORKLOADS = {
    "linear_v1000": linear_v1000,
    "linear_v32k": linear_v32k,
    "linear_v128k": linear_v128k,
    "tree_v32k": tree_v32k,
    "tree_wor_v32k": tree_wor_v32k,
    "bimodal_v152k": bimodal_v152k,
}
