"""HIP-graph replay of verify calls equals eager execution, replay after replay.

The benchmark replays captured verify calls, so a captured call must give the
same bits as an eager one on every replay, with unrelated eager work (sharing
the workspace) and synchronisations between replays.
"""

import numpy as np
import pytest

import synth
from gpu_util import i32, f32, logits_to_dev, say, torch_mod

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    torch = torch_mod()
    import rejection_sampling_verify_04_amd as sv
    d = synth.linear_v32k(B=8)
    t = synth.peaked_tree(seed=9, B=8, N=21, V=20000, dtype=synth.BF16)
    lin_args = (logits_to_dev(d["target"], 1), logits_to_dev(d["draft"], 1), i32(d["offsets"]),
                i32(d["tokens"]), f32(d["temp_target"]), f32(d["temp_draft"]))
    tree_args = (logits_to_dev(t["target"], 1), i32(t["parents"]), i32(t["tokens"]),
                 f32(t["temp_target"]))
    tree_nn = i32(t["n_nodes"])
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
    eager_lin = sv.verify_linear(*lin_args, seed=3, step=11, workspace=ws)
    eager_lin = {k: v.clone() for k, v in eager_lin.items()}
    eager_tree = sv.verify_tree(*tree_args, n_nodes=tree_nn, seed=3, step=11, workspace=ws)
    eager_tree = {k: v.clone() for k, v in eager_tree.items()}
    torch.cuda.synchronize()

    lin_out = {k: torch.empty_like(v) for k, v in eager_lin.items()}
    tree_out = {k: torch.empty_like(v) for k, v in eager_tree.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sv.verify_linear(*lin_args, seed=3, step=11, workspace=ws, outputs=lin_out)
        sv.verify_tree(*tree_args, n_nodes=tree_nn, seed=3, step=11, workspace=ws,
                       outputs=tree_out)
    other = synth.linear_v32k(seed=5, B=8)
    other_args = (logits_to_dev(other["target"], 1), logits_to_dev(other["draft"], 1),
                  i32(other["offsets"]), i32(other["tokens"]), f32(other["temp_target"]),
                  f32(other["temp_draft"]))
    for rep in range(4):
        for v in list(lin_out.values()) + list(tree_out.values()):
            v.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in eager_lin:
            assert torch.equal(lin_out[k], eager_lin[k]), (rep, "linear", k)
        for k in eager_tree:
            assert torch.equal(tree_out[k], eager_tree[k]), (rep, "tree", k)
        sv.verify_linear(*other_args, seed=rep, workspace=ws)   # eager work in between
        torch.cuda.synchronize()
    say("[graph] 4 replays equal to eager")
