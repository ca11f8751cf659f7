"""KV-cache commit after a verify step (oracle; test infrastructure).

The target's forward pass over a round writes the keys/values of the round's
N new tokens (node 0 = the last committed token, then the draft tokens or
tree nodes in node order) at cache slots [L, L + N) behind the committed
prefix of length L.  Once the verify step has accepted a path, the cache
must hold, behind the prefix, exactly the tokens an autoregressive decoder
would have seen: the root, then the accepted tokens in order, so the entries
of rejected tokens are dropped and the accepted ones moved down (cf-1 §3.3:
reuse the cached prefix, keep the accepted positions, discard every entry
after the accept point; kwkr §5.1: a pre-allocated cache spliced by offsets
rather than copied whole).

For batch row b with L = prefix_len[b] and n = num_accepted[b]:

* n < 0 (the verify step flagged the row): nothing changes and the new
  length is L;
* the path is invalid (L < 0, L + N > S_max, n > N - 1, or the accepted node
  ids are not strictly increasing within [1, N)): nothing changes and the
  new length is -1;
* otherwise the entry of the i-th accepted node path[i] (slot L + path[i])
  is written to slot L + 1 + i for i < n, for every layer and head, and the
  new length is L + 1 + n.  A linear verify is a chain: path[i] = i + 1, and
  no entry moves.

Entries at slots >= the new length are left unspecified.
"""

import numpy as np


def commit_row_plan(L, n, path, N, S_max):
    """(new_len, [(src_slot, dst_slot), ...]) for one batch row."""
    if n < 0:
        return L, []
    if L < 0 or L + N > S_max or n > N - 1:
        return -1, []
    nodes = [i + 1 for i in range(n)] if path is None else [int(path[i]) for i in range(n)]
    prev = 0
    for p in nodes:
        if not (prev < p < N):
            return -1, []
        prev = p
    return L + 1 + n, [(L + p, L + 1 + i) for i, p in enumerate(nodes)]


def kv_commit(k_cache, v_cache, prefix_len, num_accepted, path_nodes, N):
    """k_cache, v_cache: [layers, B, H, S_max, d] arrays (any dtype; copied).

    Returns (new K, new V, new_len [B]).  Moves are applied as one step:
    every destination receives the entry its source held before the call.
    """
    k = np.array(k_cache, copy=True)
    v = np.array(v_cache, copy=True)
    _, B, _, S_max, _ = k.shape
    new_len = np.zeros(B, dtype=np.int64)
    for b in range(B):
        path = None if path_nodes is None else path_nodes[b]
        nl, moves = commit_row_plan(int(prefix_len[b]), int(num_accepted[b]), path, N, S_max)
        new_len[b] = nl
        for src, dst in moves:
            k[:, b, :, dst, :] = k_cache[:, b, :, src, :]
            v[:, b, :, dst, :] = v_cache[:, b, :, src, :]
    return k, v, new_len
