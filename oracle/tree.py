"""Tree verify step, float64 (oracle; test infrastructure).

The pages describe tree verification only in outline: the draft proposes
several branches at once, organised as a tree; the target scores the whole
tree in one forward pass and one path is kept (kwkr §5.3; cf-1 §5.4; the
lonae tree-attention paragraph, which builds the tree from the draft's top-k
or from temperature sampling at each depth).  The acceptance rule for a node
with several candidate children is not written out.  The reading used here
is the single-path rule of the linear verify (kwkr §2.3/§4.1, lonae
formal-definition paragraph) applied recursively over siblings:

TOPK mode (children are the draft's deterministic top-k): the proposal that
produced child c_j is a point mass at its token, so the acceptance ratio
p/q becomes p^(j)(c_j), where p^(j) is p with the tokens of the already
rejected siblings c_1..c_{j-1} removed and renormalised, and the residual
max(0, p^(j) - delta) is p^(j) with c_j removed.  Siblings are tested in
node-index order.  On acceptance the walk descends into the child; when
every child is rejected the emitted token is drawn from p with all tested
children removed; at a leaf the bonus token is drawn from p.

SAMPLED_WOR mode (children drawn from q without replacement): q_j is q with
c_1..c_{j-1} removed and renormalised; c_j is accepted when
u < min(1, p_j(c_j) / q_j(c_j)); on rejection p_{j+1} = norm(max(0, p_j - q_j));
after the last rejection the draw is from p_{k+1}.

Row n of the target logits is the target distribution for the token that
follows node n.  Node 0 is the root (the last committed token).  Node n's
randoms are Philox position n: u_acc(n) decides node n's own acceptance,
u_smp(n) is used for a draw made at node n.

Rows read (the pages do not say what a row without a finite maximum means;
the reading is that of the linear verify, applied to the rows the walk
reads): the target row of every node that has children (its children are
tested against it), in SAMPLED_WOR also that node's draft row, and, when the
walk stops at a leaf, that leaf's target row (its bonus draw).  A row among
them whose maximum logit is not finite makes the batch row an error row; the
other rows are never read.
"""

from dataclasses import dataclass

import numpy as np

from .decode import decode_logits
from .linear import (FLAG_EPS, ROW_BAD_SHAPE, ROW_BAD_TEMP, ROW_BAD_TOKEN, ROW_NONFINITE,
                     ROW_OK, ROW_WARN_QZERO, ROW_WARN_RZERO, inverse_cdf, softmax_t)
from .philox import verify_uniforms

TREE_TOPK = 0
TREE_SAMPLED_WOR = 1


@dataclass
class TreeRowResult:
    num_accepted: int            # depth of the accepted path (accepted nodes)
    path_nodes: np.ndarray       # [N-1] node ids of the accepted path, -1 padded
    out_tokens: np.ndarray       # [N] accepted tokens then the drawn token, -1 padded
    p_at_node: np.ndarray        # [N] p_parent(n)(token_n); 0 for the root and unused nodes
    status: int = ROW_OK
    flagged_accept: object = None   # depth at which the first fragile decision was taken
    flagged_sample: bool = False
    stop_node: int = -1
    stop_kind: str = ""


def _check_tree(parents, node_tokens, n_nodes, V):
    if not (1 <= n_nodes <= len(parents)):
        return ROW_BAD_SHAPE
    for i in range(1, n_nodes):
        if not (0 <= parents[i] < i):
            return ROW_BAD_SHAPE
        if not (0 <= node_tokens[i] < V):
            return ROW_BAD_TOKEN
    return ROW_OK


def _children(parents, n_nodes, node):
    return [c for c in range(1, n_nodes) if parents[c] == node]


def _empty(N):
    return (np.full(N - 1, -1, dtype=np.int64), np.full(N, -1, dtype=np.int64),
            np.zeros(N))


def verify_tree_topk_row(x, parents, node_tokens, n_nodes, temp_t, u_acc, u_smp):
    """x: [N, V] float64 target logits; parents, node_tokens: [N]; u_acc, u_smp: [N]."""
    x = np.asarray(x, dtype=np.float64)
    N, V = x.shape
    parents = [int(v) for v in parents]
    node_tokens = [int(v) for v in node_tokens]
    path, out, p_at = _empty(N)
    st = _check_tree(parents, node_tokens, n_nodes, V)
    if st == ROW_OK and (not np.isfinite(temp_t) or temp_t < 0):
        st = ROW_BAD_TEMP
    inner = sorted({parents[c] for c in range(1, n_nodes)}) if st == ROW_OK else []
    if st == ROW_OK and not all(np.isfinite(np.max(x[n])) for n in inner):
        st = ROW_NONFINITE
    if st != ROW_OK:
        return TreeRowResult(-1, path, out, p_at, st, None, False, -1, "error")

    p_rows = {n: softmax_t(x[n], temp_t) for n in inner}
    for c in range(1, n_nodes):
        p_at[c] = p_rows[parents[c]][node_tokens[c]]

    status = ROW_OK
    flagged = None
    node, depth = 0, 0
    while True:
        kids = _children(parents, n_nodes, node)
        if not kids:
            # a leaf: its target row is read by the bonus draw
            if not np.isfinite(np.max(x[node])):
                path, out, p_at = _empty(N)
                return TreeRowResult(-1, path, out, p_at, ROW_NONFINITE, None, False, -1,
                                     "error")
            p_rows[node] = softmax_t(x[node], temp_t)
        p = p_rows[node]
        removed = []
        removed_mass = 0.0
        accepted = None
        for c in kids:
            tok = node_tokens[c]
            denom = 1.0 - removed_mass
            if tok in removed or not denom > 0.0:
                ratio = 0.0
            else:
                ratio = p[tok] / denom
            if flagged is None and abs(u_acc[c] - ratio) < FLAG_EPS:
                flagged = depth
            if u_acc[c] < ratio:
                accepted = c
                break
            if tok not in removed:
                removed.append(tok)
                removed_mass += p[tok]
        if accepted is None:
            w = p.copy()
            if removed:
                w[removed] = 0.0
            if not np.sum(w) > 0.0:
                status |= ROW_WARN_RZERO
                w = p
            k, margin = inverse_cdf(w, u_smp[node])
            kind = "greedy" if temp_t == 0.0 else ("reject" if kids else "bonus")
            out[depth] = k
            flagged_sample = temp_t != 0.0 and margin < FLAG_EPS
            return TreeRowResult(depth, path, out, p_at, status, flagged, flagged_sample,
                                 node, kind)
        path[depth] = accepted
        out[depth] = node_tokens[accepted]
        depth += 1
        node = accepted


def verify_tree_sampled_wor_row(x, y, parents, node_tokens, n_nodes, temp_t, temp_d,
                                u_acc, u_smp):
    """SAMPLED_WOR mode; y: [N, V] draft logits (row n = draft distribution after node n)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    N, V = x.shape
    parents = [int(v) for v in parents]
    node_tokens = [int(v) for v in node_tokens]
    path, out, p_at = _empty(N)
    st = _check_tree(parents, node_tokens, n_nodes, V)
    if st == ROW_OK and (not (np.isfinite(temp_t) and np.isfinite(temp_d))
                         or temp_t < 0 or temp_d < 0):
        st = ROW_BAD_TEMP
    if st == ROW_OK:
        # every distribution the walk's tests read must exist: the target and
        # draft rows of each node that has children
        inner = sorted({parents[c] for c in range(1, n_nodes)})
        if not all(np.isfinite(np.max(x[n])) and np.isfinite(np.max(y[n])) for n in inner):
            st = ROW_NONFINITE
    if st != ROW_OK:
        return TreeRowResult(-1, path, out, p_at, st, None, False, -1, "error")

    for c in range(1, n_nodes):
        p_at[c] = softmax_t(x[parents[c]], temp_t)[node_tokens[c]]
    status = ROW_OK
    flagged = None
    node, depth = 0, 0
    while True:
        kids = _children(parents, n_nodes, node)
        if not kids and not np.isfinite(np.max(x[node])):
            # a leaf: its target row is read by the bonus draw
            path, out, p_at = _empty(N)
            return TreeRowResult(-1, path, out, p_at, ROW_NONFINITE, None, False, -1, "error")
        p = softmax_t(x[node], temp_t)
        q = softmax_t(y[node], temp_d) if kids else None
        pj, qj = p.copy(), (q.copy() if kids else None)
        accepted = None
        for c in kids:
            tok = node_tokens[c]
            if qj[tok] > 0:
                ratio = pj[tok] / qj[tok]
            else:
                # a sampled child the draft could not have drawn (as in the
                # linear verify: the ratio is +inf, or 0 when p is 0 too)
                status |= ROW_WARN_QZERO
                ratio = np.inf if pj[tok] > 0 else 0.0
            if flagged is None and abs(u_acc[c] - ratio) < FLAG_EPS:
                flagged = depth
            if u_acc[c] < ratio:
                accepted = c
                break
            res = np.maximum(pj - qj, 0.0)
            if np.sum(res) > 0.0:
                pj = res / np.sum(res)
            else:
                status |= ROW_WARN_RZERO
            qj = qj.copy()
            qj[tok] = 0.0
            if np.sum(qj) > 0.0:
                qj = qj / np.sum(qj)
        if accepted is None:
            k, margin = inverse_cdf(pj, u_smp[node])
            out[depth] = k
            kind = "reject" if kids else "bonus"
            return TreeRowResult(depth, path, out, p_at, status, flagged,
                                 margin < FLAG_EPS, node, kind)
        path[depth] = accepted
        out[depth] = node_tokens[accepted]
        depth += 1
        node = accepted


def verify_tree_topk(target_logits, dtype, parents, node_tokens, n_nodes, temp_target,
                     seed=0, step=0, row_ids=None):
    """Batch TOPK verify.  target_logits: [B, N, V] as stored; parents, node_tokens: [B, N].

    Returns (num_accepted [B], path_nodes [B, N-1], out_tokens [B, N],
    p_at_node [B, N], row_status [B], per-row TreeRowResult list).
    """
    parents = np.asarray(parents)
    node_tokens = np.asarray(node_tokens)
    B, N = parents.shape
    num_acc = np.full(B, -1, dtype=np.int64)
    path_nodes = np.full((B, N - 1), -1, dtype=np.int64)
    out_tokens = np.full((B, N), -1, dtype=np.int64)
    p_at = np.zeros((B, N))
    status = np.zeros(B, dtype=np.int64)
    results = []
    for b in range(B):
        nn = N if n_nodes is None else int(n_nodes[b])
        x = decode_logits(target_logits[b], dtype)
        rid = b if row_ids is None else int(row_ids[b])
        u_acc, u_smp = verify_uniforms(seed, step, rid, N)
        r = verify_tree_topk_row(x, parents[b], node_tokens[b], nn, float(temp_target[b]),
                                 u_acc, u_smp)
        results.append(r)
        num_acc[b] = r.num_accepted
        path_nodes[b] = r.path_nodes
        out_tokens[b] = r.out_tokens
        p_at[b] = r.p_at_node
        status[b] = r.status
    return num_acc, path_nodes, out_tokens, p_at, status, results


def verify_tree_sampled_wor(target_logits, draft_logits, dtype, parents, node_tokens, n_nodes,
                            temp_target, temp_draft, seed=0, step=0, row_ids=None):
    """Batch SAMPLED_WOR verify.  target_logits, draft_logits: [B, N, V] as stored.

    Returns the same tuple as :func:`verify_tree_topk`.
    """
    parents = np.asarray(parents)
    node_tokens = np.asarray(node_tokens)
    B, N = parents.shape
    num_acc = np.full(B, -1, dtype=np.int64)
    path_nodes = np.full((B, N - 1), -1, dtype=np.int64)
    out_tokens = np.full((B, N), -1, dtype=np.int64)
    p_at = np.zeros((B, N))
    status = np.zeros(B, dtype=np.int64)
    results = []
    for b in range(B):
        nn = N if n_nodes is None else int(n_nodes[b])
        x = decode_logits(target_logits[b], dtype)
        y = decode_logits(draft_logits[b], dtype)
        rid = b if row_ids is None else int(row_ids[b])
        u_acc, u_smp = verify_uniforms(seed, step, rid, N)
        r = verify_tree_sampled_wor_row(x, y, parents[b], node_tokens[b], nn,
                                        float(temp_target[b]), float(temp_draft[b]),
                                        u_acc, u_smp)
        results.append(r)
        num_acc[b] = r.num_accepted
        path_nodes[b] = r.path_nodes
        out_tokens[b] = r.out_tokens
        p_at[b] = r.p_at_node
        status[b] = r.status
    return num_acc, path_nodes, out_tokens, p_at, status, results
