"""GPU parity of spec_verify_tree in SAMPLED_WOR mode against the oracle.

Children are draws without replacement from each node's draft softmax.  The
cases cover the full-size workload (B=64 trees of 64 nodes over V=32000
bf16), small peaked trees whose walks go deep and reject several siblings in
a row, multi-chunk and ragged vocabularies (one to ten groups of chunk
loads per pass), rows whose length in bytes is not a multiple of 16, greedy
target or draft rows, repeated sibling tokens, partial trees and error rows.
"""

import numpy as np
import pytest

import draw_bound as DB
import synth
from gpu_util import compare_tree, run_linear, run_oracle_tree, run_tree, say, tree_draw_weights
from oracle.philox import verify_uniforms

pytestmark = pytest.mark.gpu


def check(d, label):
    say("[wor] %s: B=%d N=%d V=%d" % (label, d["B"], d["N"], d["V"]))
    gpu = run_tree(d)
    ref = run_oracle_tree(d)
    s = compare_tree(gpu, ref, d)
    depth = np.bincount(np.maximum(gpu["num_accepted"], 0), minlength=5)
    rej = sum(_rejections(r, d, b) for b, r in enumerate(ref[5]))
    say("[wor] %s: ok %s depth histogram %s, rejected siblings %d" % (
        label, s, depth.tolist(), rej))
    return gpu, ref


def _rejections(r, d, b):
    """Siblings the oracle's walk rejected (each is one extra vocabulary pass)."""
    if r.num_accepted < 0:
        return 0
    par = d["parents"][b]
    nn = d["N"] if d.get("n_nodes") is None else int(d["n_nodes"][b])
    path = [0] + [int(v) for v in r.path_nodes[:r.num_accepted]]
    n = 0
    for i, node in enumerate(path):
        kids = [c for c in range(1, nn) if par[c] == node]
        if i + 1 < len(path):
            n += kids.index(path[i + 1])
        else:
            n += len(kids)
    return n


def test_tree_wor_v32k_full():
    d = synth.tree_wor_v32k()
    check(d, "tree_wor v32k bf16")


def test_wor_skewed_batch():
    """SAMPLED_WOR trees of 64 nodes over V=32000 with two of sixteen replaced
    by chains: the chains' units beyond their own waves run on the shared
    waves of the vocabulary pass."""
    d = synth.tree_wor(seed=41, B=16, N=64, V=32000, draft_sd=3.0, pert=0.5)
    d["parents"] = d["parents"].copy()
    for b in (3, 11):
        d["parents"][b] = np.arange(-1, d["N"] - 1, dtype=d["parents"].dtype)
    check(d, "V=32000 bf16, two chains")


def test_peaked_wor_trees_reject_and_go_deep():
    d = synth.tree_wor(seed=11, B=48, N=21, V=64, draft_sd=6.0, pert=1.0, dtype=synth.F32)
    gpu, ref = check(d, "peaked V=64 fp32")
    assert np.mean(gpu["num_accepted"] >= 2) > 0.3
    assert sum(_rejections(r, d, b) for b, r in enumerate(ref[5])) >= 40


def test_wor_multichunk_ragged_bf16():
    # V = 20000: 3 chunks (groups of 2 and 1), ragged last chunk
    d = synth.tree_wor(seed=12, B=16, N=40, V=20000, draft_sd=4.0, pert=1.0)
    check(d, "V=20000 bf16")


def test_wor_large_vocab_bf16():
    # V = 152064: 19 chunks (10 groups), last chunk 4608 wide
    d = synth.tree_wor(seed=13, B=4, N=16, V=152064, draft_sd=3.0, pert=1.0, width=3, depth=3)
    check(d, "V=152064 bf16")


def test_wor_unaligned_rows():
    # 1001 bf16 logits per row: rows are not 16-byte multiples (element loads)
    d = synth.tree_wor(seed=14, B=16, N=21, V=1001, draft_sd=5.0, pert=1.0)
    check(d, "V=1001 bf16 unaligned")
    d = synth.tree_wor(seed=15, B=8, N=21, V=8195, draft_sd=5.0, pert=1.0, dtype=synth.F32)
    check(d, "V=8195 fp32 unaligned")


def test_wor_greedy_and_mixed_temperatures():
    d = synth.tree_wor(seed=16, B=24, N=21, V=64, draft_sd=6.0, pert=1.0, dtype=synth.F32)
    tt, td = d["temp_target"].copy(), d["temp_draft"].copy()
    tt[0::4] = 0.0                  # greedy target
    td[1::4] = 0.0                  # greedy draft
    tt[2::4], td[2::4] = 0.0, 0.0   # both
    tt[3::4], td[3::4] = 0.7, 1.3   # different temperatures
    d["temp_target"], d["temp_draft"] = tt, td
    check(d, "greedy and mixed temperatures")


def test_wor_two_chunks_mixed_temperatures():
    # V = 12000: two chunks with the target term kept in LDS across a node's
    # passes, one-hot (greedy) terms included
    d = synth.tree_wor(seed=19, B=24, N=21, V=12000, draft_sd=5.0, pert=1.0)
    tt, td = d["temp_target"].copy(), d["temp_draft"].copy()
    tt[0::4] = 0.0
    td[1::4] = 0.0
    tt[3::4], td[3::4] = 0.7, 1.3
    d["temp_target"], d["temp_draft"] = tt, td
    check(d, "V=12000 bf16, mixed temperatures")


def test_wor_repeated_sibling_tokens():
    # duplicate children (a sampler with replacement): the zero-q path and warning
    d = synth.tree_wor(seed=17, B=24, N=21, V=64, draft_sd=6.0, pert=1.0, dtype=synth.F32)
    tok = d["tokens"].copy()
    par = d["parents"]
    for b in range(0, 24, 2):
        kids = [c for c in range(1, d["N"]) if par[b, c] == 0]
        if len(kids) >= 3:
            tok[b, kids[2]] = tok[b, kids[0]]
    d["tokens"] = tok
    gpu, ref = check(d, "repeated sibling tokens")


def test_wor_partial_trees_and_error_rows():
    d = synth.tree_wor(seed=18, B=14, N=21, V=64, draft_sd=6.0, pert=1.0, dtype=synth.F32)
    d["n_nodes"] = d["n_nodes"].copy()
    d["n_nodes"][:4] = [1, 5, 9, 20]
    d["parents"] = d["parents"].copy()
    d["tokens"] = d["tokens"].copy()
    d["target"] = d["target"].copy()
    d["draft"] = d["draft"].copy()
    d["parents"][5, 3] = 7            # parent after child: bad shape
    d["tokens"][6, 2] = d["V"]        # token out of range
    d["n_nodes"][7] = 0               # bad node count
    d["temp_draft"] = d["temp_draft"].copy()
    d["temp_draft"][8] = np.nan       # bad draft temperature
    d["target"][9, 4] = -np.inf       # an inner node's target row without a finite maximum
    d["draft"][10, 0] = -np.inf       # the root's draft row: non-finite
    leaf = int(max(c for c in range(1, 21) if c not in set(d["parents"][11, 1:].tolist())))
    d["draft"][11, leaf] = -np.inf    # a leaf's draft row is never read: fine
    # A leaf's target row is read only by a walk that stops there (the walk up
    # to it reads inner rows only): an error at the leaf the walk stops at,
    # nothing at a leaf no walk reaches.
    ref0 = run_oracle_tree(d)
    assert ref0[5][12].stop_kind == "bonus"
    d["target"][12, ref0[5][12].stop_node, 3] = np.nan
    unread = [n for n in range(1, 21) if n not in set(d["parents"][13, 1:].tolist())
              and n != ref0[5][13].stop_node]
    d["target"][13, unread[0]] = -np.inf
    gpu, ref = check(d, "partial trees and error rows")
    assert list(gpu["num_accepted"][[5, 6, 7, 8, 9, 10, 12]]) == [-1] * 7
    assert gpu["num_accepted"][11] >= 0 and gpu["row_status"][11] & 0xFF == 0
    assert gpu["num_accepted"][13] >= 0 and gpu["row_status"][13] & 0xFF == 0


@pytest.mark.parametrize("B", [600, 1100])
def test_wor_many_trees(B):
    """SAMPLED_WOR over more trees than the vocabulary pass compacts (512) and
    caches in LDS (1024): ragged node counts, an inner node's non-finite
    draft row (an error) and a non-finite target row at the leaf a walk stops
    at (an error)."""
    d = synth.tree_wor(seed=30 + B, B=B, N=16, V=64, draft_sd=6.0, pert=1.0, dtype=synth.F32)
    d["n_nodes"] = d["n_nodes"].copy()
    d["n_nodes"][::9] = np.minimum(d["n_nodes"][::9], 4)
    d["target"] = d["target"].copy()
    d["draft"] = d["draft"].copy()
    d["draft"][11, int(d["parents"][11, 3])] = -np.inf
    ref0 = run_oracle_tree(d)
    b_stop = next(b for b in range(20, B) if ref0[5][b].stop_kind == "bonus")
    d["target"][b_stop, ref0[5][b_stop].stop_node, 2] = np.nan
    gpu, ref = check(d, "%d SAMPLED_WOR trees" % B)
    assert gpu["num_accepted"][11] == -1 and gpu["num_accepted"][b_stop] == -1


def test_wor_chain_equals_linear():
    """One child per node: SAMPLED_WOR is the linear verify with the draft's q."""
    rng = np.random.default_rng(19)
    B, g, V = 16, 6, 3000
    y = rng.normal(0, 2, size=(B, g + 1, V)).astype(np.float32)
    x = y + rng.normal(0, 0.6, size=(B, g + 1, V)).astype(np.float32)
    xb, yb = synth.bf16_bits(x), synth.bf16_bits(y)
    yv = synth.bf16_values(yb).astype(np.float64)
    T = np.linspace(0.6, 1.4, B).astype(np.float32)
    dtok = np.zeros((B, g), np.int32)
    for b in range(B):
        for i in range(g):
            z = yv[b, i] / T[b] + rng.gumbel(size=V)
            dtok[b, i] = int(np.argmax(z))
    lin = dict(kind="linear", dtype=1, B=B, V=V, target=xb.reshape(B * (g + 1), V),
               draft=yb[:, :g].reshape(B * g, V), offsets=np.arange(B + 1, dtype=np.int32) * g,
               tokens=dtok.reshape(-1), temp_target=T, temp_draft=T.copy(), seed=4, step=2)
    tree = dict(kind="tree_wor", dtype=1, B=B, N=g + 1, V=V, target=xb, draft=yb,
                parents=np.tile(np.arange(-1, g, dtype=np.int32), (B, 1)),
                tokens=np.concatenate([np.zeros((B, 1), np.int32), dtok], 1),
                n_nodes=None, temp_target=T, temp_draft=T.copy(), seed=4, step=2)
    gl = run_linear(lin)
    gt = run_tree(tree)
    assert np.array_equal(gl["num_accepted"], gt["num_accepted"])
    same = np.array_equal(gl["out_tokens"].reshape(B, g + 1), gt["out_tokens"])
    say("[wor] chain == linear: depths %s, tokens identical: %s" % (
        gt["num_accepted"].tolist(), same))
    # both draws are admissible under the float32 bound of the same stop weights
    ref = run_oracle_tree(tree)
    compare_tree(gt, ref, tree)
    tally = DB.DrawTally()
    for b in range(B):
        n = gt["num_accepted"][b]
        assert np.array_equal(gl["out_tokens"].reshape(B, g + 1)[b][:n], gt["out_tokens"][b][:n])
        r = ref[5][b]
        if r.flagged_accept is None:
            w, e, masked = tree_draw_weights(tree, b, r)
            u = verify_uniforms(tree["seed"], tree["step"], b, g + 1)[1][r.stop_node]
            tally.add(int(gl["out_tokens"].reshape(B, g + 1)[b][n]), w, e, u, masked)
    say("[wor] chain == linear: linear draws against the tree's bound %s" % tally.summary())
