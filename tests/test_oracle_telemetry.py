"""Pins of the telemetry oracle: hand-counted rounds, a hand-drawn tree, the
efficiency's closed form under its reading, and the two acceptance peaks of a
bimodal workload (the lonae page: a per-request histogram must keep the
low and the high peak apart)."""

import numpy as np

import oracle
from oracle import telemetry as TM
import synth


def test_linear_counts_by_hand():
    n = np.array([5, 0, 3, -1, 2, 0])
    off = np.array([0, 5, 10, 15, 19, 21, 21])       # gammas 5, 5, 5, 4, 2, 0
    t = TM.add_linear(TM.empty(), n, off)
    assert t["rounds"] == 5 and t["error_rows"] == 1
    assert t["drafted"] == 5 + 5 + 5 + 2 + 0 and t["accepted"] == 5 + 0 + 3 + 2 + 0
    assert t["full_accepts"] == 3                    # 5/5, 2/2 and 0/0
    want = np.zeros(20, dtype=np.int64)
    want[19] += 2                                    # rates 1.0 (5/5, 2/2)
    want[0] += 1                                     # 0/5
    want[12] += 1                                    # 3/5 = 0.6 -> [0.60, 0.65)
    assert np.array_equal(t["acc_rate_hist"], want)  # the gamma = 0 row is not binned
    assert list(t["accepted_hist"][:6]) == [2, 0, 1, 1, 0, 1]


def test_tree_counts_by_hand():
    #        0
    #      /   \
    #     1     2
    #    / \     \
    #   3   4     5
    par = np.array([[-1, 0, 0, 1, 1, 2], [-1, 0, 0, 1, 1, 2], [-1, 0, 0, 1, 1, 2]])
    path = np.array([[1, 4, -1, -1, -1], [2, -1, -1, -1, -1], [-1, -1, -1, -1, -1]])
    n = np.array([2, 1, 0])
    t = TM.add_tree(TM.empty(), n, path, par, None)
    assert t["rounds"] == 3 and t["drafted"] == 6 and t["accepted"] == 3
    assert t["full_accepts"] == 1                    # node 4 is a leaf; node 2 is not
    assert t["tree_paths"] == 9                      # three leaves per round
    assert t["tree_paths_hit"] == 2 + 1 + 0          # leaves under node 1, under node 2, none
    assert list(t["sibling_rank_hist"][:3]) == [1, 2, 0]   # 1: 1st; 4: 2nd; 2: 2nd
    assert list(t["acc_rate_hist"][[0, 10, 19]]) == [1, 1, 1]
    s = TM.summary(t)
    assert abs(s["tree_width_effective"] - 3 / 9) < 1e-15


def test_efficiency_reading_is_the_squared_window_rate():
    rng = np.random.default_rng(80)
    g = rng.integers(1, 9, size=200)
    off = np.concatenate([[0], np.cumsum(g)])
    n = np.array([rng.integers(0, gi + 1) for gi in g])
    s = TM.summary(TM.add_linear(TM.empty(), n, off))
    r = n.sum() / g.sum()
    assert abs(s["speculative_efficiency"] - r * r) < 1e-12
    assert s["speculative_efficiency"] <= 1.0


def test_bimodal_workload_shows_two_acceptance_peaks():
    d = synth.bimodal_v152k(seed=5, B=96, V=512)
    n, *_ = oracle.verify_linear(d["target"], d["draft"], d["dtype"], d["offsets"], d["tokens"],
                                 d["temp_target"], d["temp_draft"])
    t = TM.add_linear(TM.empty(), n, d["offsets"])
    h = t["acc_rate_hist"]
    low, mid, high = h[:6].sum(), h[6:10].sum(), h[10:].sum()
    assert low >= 0.25 * t["rounds"] and high >= 0.25 * t["rounds"]
    assert mid < min(low, high)
    g = d["offsets"][1:] - d["offsets"][:-1]
    rate = n / g
    assert rate[d["sigma"] < 1].mean() > 3 * rate[d["sigma"] > 1].mean()
