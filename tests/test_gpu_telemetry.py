"""GPU parity of the telemetry counters and summary against the oracle.

Both sides count the same verify outputs (the library's own), so every
counter must match exactly and the summary to float64 rounding.  Windows
span several calls; trees include partial trees, error rows, TOPK and
SAMPLED_WOR walks; the full-size case is the bimodal workload
(B=256, V=152064 bf16), whose two acceptance peaks the histogram keeps apart.
"""

import numpy as np
import pytest

from oracle import telemetry as TM
import synth
from gpu_util import i32, run_linear, run_tree, say, torch_mod

pytestmark = pytest.mark.gpu


def compare(acc, t, label):
    import rejection_sampling_verify_04_amd as sv
    got = sv.telemetry_fields(acc)
    for k in TM.FIELDS:
        assert got[k] == t[k], (label, k, got[k], t[k])
    for name, _ in sv.TELEMETRY_BINS:
        assert np.array_equal(np.array(got[name]), t[name]), (label, name)
    s_gpu = sv.telemetry_summary(acc).cpu().numpy()
    s_ref = TM.summary(t)
    for i, name in enumerate(sv.SUMMARY_FIELDS):
        ref = s_ref[name]
        if ref is None:
            assert np.isnan(s_gpu[i]) or (name.endswith("_bin") and s_gpu[i] == -1), (label, name)
        elif name.endswith("_bin"):
            assert s_gpu[i] == ref, (label, name, s_gpu[i], ref)
        else:
            assert abs(s_gpu[i] - ref) <= 1e-12 * max(1.0, abs(ref)), (label, name, s_gpu[i], ref)
    say("[telemetry] %s: ok %s" % (label, {k: (round(v, 4) if v is not None else None)
                                            for k, v in s_ref.items()}))


def test_linear_window_over_calls():
    import rejection_sampling_verify_04_amd as sv
    acc = sv.telemetry_block()
    t = TM.empty()
    for seed in range(3):
        d = synth.bimodal_v152k(seed=5 + seed, B=96, V=4000)
        g = run_linear(d, seed=seed, step=seed)
        n = g["num_accepted"]
        if seed == 2:
            n = n.copy()
            n[::7] = -1                     # error rows
        sv.telemetry_linear(i32(n), i32(d["offsets"]), acc)
        TM.add_linear(t, n, d["offsets"])
    compare(acc, t, "linear window of 3 calls")


def test_tree_windows_topk_and_wor():
    import rejection_sampling_verify_04_amd as sv
    acc = sv.telemetry_block()
    t = TM.empty()
    cases = [synth.peaked_tree(seed=81, B=24, N=21),
             synth.tree_wor(seed=82, B=24, N=21, V=64, draft_sd=6.0, pert=1.0, dtype=synth.F32)]
    d = synth.peaked_tree(seed=83, B=12, N=21)
    d["n_nodes"] = d["n_nodes"].copy()
    d["n_nodes"][:4] = [1, 5, 9, 20]
    cases.append(d)
    for d in cases:
        g = run_tree(d)
        n, path = g["num_accepted"], g["path_nodes"]
        sv.telemetry_tree(i32(n), i32(path), i32(d["parents"]), acc,
                          n_nodes=None if d.get("n_nodes") is None else i32(d["n_nodes"]))
        TM.add_tree(t, n, path, d["parents"], d.get("n_nodes"))
    assert t["tree_paths_hit"] > 0 and t["sibling_rank_hist"][1:].sum() > 0
    compare(acc, t, "tree window (TOPK, SAMPLED_WOR, partial trees)")


def test_bimodal_full_size():
    import rejection_sampling_verify_04_amd as sv
    d = synth.bimodal_v152k()
    g = run_linear(d)
    acc = sv.telemetry_block()
    sv.telemetry_linear(i32(g["num_accepted"]), i32(d["offsets"]), acc)
    t = TM.add_linear(TM.empty(), g["num_accepted"], d["offsets"])
    compare(acc, t, "bimodal_v152k")
    h = np.array(sv.telemetry_fields(acc)["acc_rate_hist"])
    say("[telemetry] bimodal acceptance histogram (5%% bins): %s" % h.tolist())
    assert h[:6].sum() > h[6:10].sum() and h[10:].sum() > h[6:10].sum()


def test_tree_full_width_ragged_batch():
    """64-node trees (every lane of a wave a node), a batch that leaves the last
    block of four trees part-filled, error rows mixed in, then the full-size
    tree workload (B=64, N=64, V=32000 bf16) in the same window."""
    import rejection_sampling_verify_04_amd as sv
    acc = sv.telemetry_block()
    t = TM.empty()
    d = synth.tree_v32k(seed=91, B=37, V=2000)
    g = run_tree(d)
    n = g["num_accepted"].copy()
    n[::5] = -1
    sv.telemetry_tree(i32(n), i32(g["path_nodes"]), i32(d["parents"]), acc)
    TM.add_tree(t, n, g["path_nodes"], d["parents"], None)
    d = synth.tree_v32k()
    g = run_tree(d)
    sv.telemetry_tree(i32(g["num_accepted"]), i32(g["path_nodes"]), i32(d["parents"]), acc)
    TM.add_tree(t, g["num_accepted"], g["path_nodes"], d["parents"], None)
    assert t["error_rows"] == 8 and t["rounds"] == 64 + 29
    compare(acc, t, "64-node trees, B=37 with error rows, then B=64")


def test_tree_degenerate_shapes():
    """Root-only trees (N=1: no path, every tree a full accept of zero tokens),
    two-node trees, and a batch of one tree, in one window."""
    import rejection_sampling_verify_04_amd as sv
    torch = torch_mod()
    acc = sv.telemetry_block()
    t = TM.empty()
    # N = 1: the path array is empty
    par1 = np.full((5, 1), -1, dtype=np.int32)
    n1 = np.zeros(5, dtype=np.int32)
    sv.telemetry_tree(i32(n1), torch.zeros((5, 0), dtype=torch.int32, device="cuda"), i32(par1), acc)
    TM.add_tree(t, n1, np.zeros((5, 0), dtype=np.int32), par1, None)
    # N = 2: a root and one child, accepted or not, one error row
    par2 = np.array([[-1, 0]] * 6, dtype=np.int32)
    n2 = np.array([0, 1, 1, 0, -1, 1], dtype=np.int32)
    path2 = np.array([[1 if k > 0 else -1] for k in n2], dtype=np.int32)
    sv.telemetry_tree(i32(n2), i32(path2), i32(par2), acc)
    TM.add_tree(t, n2, path2, par2, None)
    # one tree of 64 nodes, a chain accepted to depth 3
    par3 = np.array([[-1] + list(range(63))], dtype=np.int32)
    n3 = np.array([3], dtype=np.int32)
    path3 = np.full((1, 63), -1, dtype=np.int32)
    path3[0, :3] = [1, 2, 3]
    sv.telemetry_tree(i32(n3), i32(path3), i32(par3), acc)
    TM.add_tree(t, n3, path3, par3, None)
    assert t["rounds"] == 11 and t["error_rows"] == 1 and t["tree_paths_hit"] == 4
    compare(acc, t, "root-only, two-node and single-chain trees")
