"""GPU parity of spec_verify_tree (TOPK) against the oracle."""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import compare_tree, run_linear, run_oracle_tree, run_tree, say

pytestmark = pytest.mark.gpu


def run_oracle(d):
    return run_oracle_tree(d)


def check(d, label):
    say("[tree] %s: B=%d N=%d V=%d" % (label, d["B"], d["N"], d["V"]))
    gpu = run_tree(d)
    ref = run_oracle(d)
    s = compare_tree(gpu, ref, d)
    depth = np.bincount(np.maximum(gpu["num_accepted"], 0), minlength=5)
    say("[tree] %s: ok %s depth histogram %s" % (label, s, depth.tolist()))
    return gpu, ref


def test_tree_v32k_full():
    d = synth.tree_v32k()
    say("[tree] nodes passing cumulative 0.1: %d; depth histogram %s" % (
        d["nodes_passing_0p1"], d["depth_hist"].tolist()))
    check(d, "tree v32k bf16")


def test_tree_v32k_skewed_batch():
    """The full-size batch with every eighth tree replaced by a 64-node chain
    (63 rows with children against about 19): the chains' units beyond their
    own waves run on the shared waves of the vocabulary pass."""
    d = synth.tree_v32k()
    d["parents"] = d["parents"].copy()
    for b in range(0, d["B"], 8):
        d["parents"][b] = np.arange(-1, d["N"] - 1, dtype=d["parents"].dtype)
    check(d, "tree v32k bf16, chains in every eighth row")


def test_peaked_trees_reach_depth():
    d = synth.peaked_tree()
    gpu, _ = check(d, "peaked V=64 fp32")
    assert np.mean(gpu["num_accepted"] >= 2) > 0.5


def test_peaked_trees_bf16_multichunk():
    d = synth.tree_v32k(seed=21, B=16, N=40, V=20000, draft_sd=6.0, pert=0.5)
    check(d, "peaked V=20000 bf16")


def test_largest_vocabulary_trees():
    # V = 524288 (64 chunks): the stop draw picks one chunk of 64
    d = synth.tree_v32k(seed=24, B=2, N=8, V=524288, draft_sd=3.0, pert=0.5)
    check(d, "V=524288 bf16")


def test_greedy_and_mixed_temperature_trees():
    d = synth.peaked_tree(seed=22, B=24)
    d["temp_target"] = np.where(np.arange(24) % 3 == 0, 0.0, d["temp_target"]).astype(np.float32)
    check(d, "greedy trees")


def test_partial_trees_and_error_rows():
    d = synth.peaked_tree(seed=23, B=12, N=21)
    d["n_nodes"] = d["n_nodes"].copy()
    d["n_nodes"][:4] = [1, 5, 9, 20]
    d["parents"] = d["parents"].copy()
    d["tokens"] = d["tokens"].copy()
    d["parents"][5, 3] = 7          # parent after child: bad shape
    d["tokens"][6, 2] = d["V"]      # token out of range
    d["n_nodes"][7] = 0             # bad node count
    d["temp_target"] = d["temp_target"].copy()
    d["temp_target"][8] = np.nan    # bad temperature
    d["target"] = d["target"].copy()
    d["target"][9, int(d["parents"][9, 5])] = -np.inf   # an inner node's row: read, an error
    # A leaf's row is read only by a walk that stops there; the walk up to a
    # leaf reads inner rows only, so a non-finite row at the leaf a walk
    # stops at leaves the walk as it was and makes the row an error, while one
    # at a leaf no walk reaches changes nothing.
    ref0 = run_oracle_tree(d)
    b_stop = next(b for b in (10, 11) if ref0[5][b].stop_kind == "bonus")
    d["target"][b_stop, ref0[5][b_stop].stop_node, 7] = np.nan
    b_other = 21 - b_stop
    unread = [n for n in range(1, d["N"]) if n not in set(d["parents"][b_other, 1:].tolist())
              and n != ref0[5][b_other].stop_node]
    d["target"][b_other, unread[0]] = -np.inf
    gpu, ref = check(d, "partial trees and error rows")
    assert list(gpu["num_accepted"][[5, 6, 7, 8, 9, b_stop]]) == [-1] * 6
    assert gpu["row_status"][b_stop] == ref[4][b_stop] != 0
    assert gpu["num_accepted"][b_other] >= 0 and gpu["row_status"][b_other] & 0xFF == 0


@pytest.mark.parametrize("B", [600, 1100])
def test_many_trees(B):
    """More trees than the vocabulary pass compacts (512: leaf rows are then
    skipped as they come) and than it caches in LDS (1024), with ragged node
    counts, an inner node's non-finite row (an error) and a non-finite row at
    the leaf a walk stops at (an error) or at a leaf no walk reaches."""
    d = synth.peaked_tree(seed=25 + B, B=B, N=16)
    d["n_nodes"] = d["n_nodes"].copy()
    d["n_nodes"][::7] = np.minimum(d["n_nodes"][::7], 3)
    d["n_nodes"][5] = 1
    d["target"] = d["target"].copy()
    d["target"][10, int(d["parents"][10, 2])] = -np.inf
    ref0 = run_oracle_tree(d)
    stops = [b for b in range(20, B) if ref0[5][b].stop_kind == "bonus"][:2]
    d["target"][stops[0], ref0[5][stops[0]].stop_node, 1] = np.nan
    others = [b for b in range(20, B) if ref0[5][b].stop_kind == "reject" and b not in stops]
    b_other = others[0]
    unread = [n for n in range(1, int(d["n_nodes"][b_other]))
              if n not in set(d["parents"][b_other, 1:int(d["n_nodes"][b_other])].tolist())]
    d["target"][b_other, unread[0]] = -np.inf
    gpu, ref = check(d, "%d trees" % B)
    assert gpu["num_accepted"][10] == -1 and gpu["num_accepted"][stops[0]] == -1
    assert gpu["num_accepted"][b_other] >= 0


def test_chain_tree_equals_linear_greedy_draft():
    rng = np.random.default_rng(31)
    B, g, V = 16, 6, 3000
    y = rng.normal(0, 3, size=(B, g, V)).astype(np.float32)
    x = rng.normal(0, 3, size=(B, g + 1, V)).astype(np.float32)
    dtok = np.argmax(synth.bf16_values(synth.bf16_bits(y)), axis=2)
    for b in range(B):
        for i in range(g):
            x[b, i, dtok[b, i]] = x[b, i].max() + rng.uniform(0, 5)
    xb, yb = synth.bf16_bits(x), synth.bf16_bits(y)
    T = np.linspace(0.5, 1.5, B).astype(np.float32)
    lin = dict(kind="linear", dtype=1, B=B, V=V, target=xb.reshape(B * (g + 1), V),
               draft=yb.reshape(B * g, V), offsets=np.arange(B + 1, dtype=np.int32) * g,
               tokens=dtok.reshape(-1).astype(np.int32), temp_target=T,
               temp_draft=np.zeros(B, np.float32), seed=4, step=2)
    tree = dict(kind="tree", dtype=1, B=B, N=g + 1, V=V, target=xb,
                parents=np.tile(np.arange(-1, g, dtype=np.int32), (B, 1)),
                tokens=np.concatenate([np.zeros((B, 1), np.int32), dtok.astype(np.int32)], 1),
                n_nodes=None, temp_target=T, seed=4, step=2)
    gl = run_linear(lin)
    gt = run_tree(tree)
    assert np.array_equal(gl["num_accepted"], gt["num_accepted"])
    assert np.array_equal(gl["out_tokens"].reshape(B, g + 1), gt["out_tokens"])
    say("[tree] chain == linear, depths %s" % gt["num_accepted"].tolist())
