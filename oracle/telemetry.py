"""Round telemetry of the verify step (oracle; test infrastructure).

The lonae page names the health signals of a speculative deployment: the
acceptance rate with its per-request histogram (two peaks, near 8-15% and
55-70%, must stay distinguishable), the Speculative Efficiency
acceptance_rate * avg_accepted_tokens / draft_steps (aggregated over a
window; below 1.0 the speculation loses), and, for trees, Tree Width
Effective, the paths actually hit over the paths the tree offered (ideal
>= 0.4).

Counters over the rows of the calls in a window (error rows only counted):

* rounds, error_rows;
* drafted: draft steps of the round, gamma_b for a linear row and the depth
  of the deepest node for a tree (the draft model runs once per level);
* accepted: accepted draft tokens;
* full_accepts: rounds that accepted every step (linear n = gamma_b; tree:
  the walk reached a leaf);
* acc_rate_hist[k], k < 20: rows with accepted / drafted in [k/20, (k+1)/20)
  (the value 1 in the last bin; rows with drafted = 0 not binned);
* accepted_hist[n], n < 65: rows that accepted n tokens (n is also where the
  first rejection sat, when n < drafted);
* tree_paths: root-to-leaf paths of the tree rounds (their leaves);
* tree_paths_hit: of those, the paths through the first accepted node;
* sibling_rank_hist[r], r < 64: accepted tree nodes that were the (r+1)-th
  child of their parent in test order.

Readings (the page gives names and thresholds only): avg_accepted_tokens is
accepted / rounds and draft_steps is drafted / rounds, so the efficiency is
(accepted / drafted)^2 over the window and cannot exceed 1; a path is hit
when the round accepted its first node below the root.
"""

import numpy as np

ACC_BINS = 20
POS_BINS = 65
RANK_BINS = 64

FIELDS = ["rounds", "error_rows", "drafted", "accepted", "full_accepts", "tree_paths",
          "tree_paths_hit"]


def empty():
    t = {k: 0 for k in FIELDS}
    t["acc_rate_hist"] = np.zeros(ACC_BINS, dtype=np.int64)
    t["accepted_hist"] = np.zeros(POS_BINS, dtype=np.int64)
    t["sibling_rank_hist"] = np.zeros(RANK_BINS, dtype=np.int64)
    return t


def _rate_bin(n, g):
    """Bin of n / g: the k with k/20 <= n/g < (k+1)/20, exact in integers."""
    return min(ACC_BINS - 1, (ACC_BINS * n) // g)


def _row(t, n, g):
    t["rounds"] += 1
    t["drafted"] += g
    t["accepted"] += n
    t["full_accepts"] += int(n == g)
    if g > 0:
        t["acc_rate_hist"][_rate_bin(n, g)] += 1
    t["accepted_hist"][min(n, POS_BINS - 1)] += 1


def add_linear(t, num_accepted, draft_offsets):
    for b in range(len(num_accepted)):
        n = int(num_accepted[b])
        if n < 0:
            t["error_rows"] += 1
            continue
        _row(t, n, int(draft_offsets[b + 1]) - int(draft_offsets[b]))
    return t


def add_tree(t, num_accepted, path_nodes, parents, n_nodes):
    B, N = np.asarray(parents).shape
    for b in range(B):
        n = int(num_accepted[b])
        if n < 0:
            t["error_rows"] += 1
            continue
        nn = N if n_nodes is None else int(n_nodes[b])
        par = [int(p) for p in parents[b][:nn]]
        depth = [0] * nn
        for i in range(1, nn):
            depth[i] = depth[par[i]] + 1
        kids = [[c for c in range(1, nn) if par[c] == i] for i in range(nn)]
        leaves = [i for i in range(nn) if not kids[i]]
        g = max(depth)
        t["rounds"] += 1
        t["drafted"] += g
        t["accepted"] += n
        last = int(path_nodes[b][n - 1]) if n > 0 else 0
        t["full_accepts"] += int(not kids[last])
        if g > 0:
            t["acc_rate_hist"][_rate_bin(n, g)] += 1
        t["accepted_hist"][min(n, POS_BINS - 1)] += 1
        t["tree_paths"] += len(leaves)
        if n > 0:
            first = int(path_nodes[b][0])

            def under(x):
                while x > 0 and depth[x] > 1:
                    x = par[x]
                return x == first
            t["tree_paths_hit"] += sum(1 for l in leaves if under(l))
        for i in range(n):
            c = int(path_nodes[b][i])
            rank = kids[par[c]].index(c)
            t["sibling_rank_hist"][min(rank, RANK_BINS - 1)] += 1
    return t


def summary(t):
    """The derived signals of a window (None where undefined)."""
    rounds, drafted, accepted = t["rounds"], t["drafted"], t["accepted"]
    out = dict(acceptance_rate=accepted / drafted if drafted else None,
               avg_accepted_tokens=accepted / rounds if rounds else None,
               draft_steps=drafted / rounds if rounds else None,
               tree_width_effective=(t["tree_paths_hit"] / t["tree_paths"]
                                     if t["tree_paths"] else None))
    if drafted and rounds:
        out["speculative_efficiency"] = (out["acceptance_rate"] * out["avg_accepted_tokens"]
                                         / out["draft_steps"])
    else:
        out["speculative_efficiency"] = None
    h = t["acc_rate_hist"]
    tot = int(h.sum())
    for q in (50, 95, 99):
        if tot:
            k = int(np.searchsorted(np.cumsum(h), q / 100.0 * tot))
            out["acc_rate_p%d_bin" % q] = min(k, ACC_BINS - 1)
        else:
            out["acc_rate_p%d_bin" % q] = None
    return out
