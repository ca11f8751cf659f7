"""Figures printed on the pages (tests/golden/pages_figures.json) and the input generators."""

import json
import os

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import linear as L
import synth
from exact_law import segments

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))


def closed_form(alpha, gamma):
    return (1 - alpha ** (gamma + 1)) / (1 - alpha)


def exact_alpha(p, q):
    """Per-position acceptance of the oracle, by exact enumeration over d ~ q and u."""
    x = np.log(np.maximum(p, 0)).reshape(1, -1)
    y = np.log(np.maximum(q, 0)).reshape(1, -1)
    xx = np.vstack([x, x])
    a = 0.0
    for d in range(len(q)):
        if q[d] > 0:
            acc = segments(lambda u: L.verify_linear_row(xx, y, [d], 1.0, 1.0, [0.5, u],
                                                         [0.5, 0.5]).num_accepted == 1)
            a += q[d] * acc.get(True, 0.0)
    return a


def test_linear_example_about_two_tokens():
    g = GOLDEN["linear_example"]
    # p, q with sum min(p, q) = 0.5
    a = exact_alpha(np.array([0.5, 0.5, 0.0]), np.array([0.0, 0.5, 0.5]))
    assert abs(a - g["alpha"]) < 1e-12
    val = sum(a ** k for k in range(g["gamma"] + 1))
    assert abs(val - closed_form(g["alpha"], g["gamma"])) < 1e-10
    assert round(val) == g["printed_tokens"]          # 1.9375, printed as about 2


def test_speedup_example_formula_vs_print():
    g = GOLDEN["speedup_example"]
    tokens = closed_form(g["alpha"], g["gamma"])
    with_c = tokens / (1 + g["gamma"] * g["c"])
    # the printed "about 3.0" is closer to the c-free value; the formula gives 2.674
    assert abs(with_c - 2.674) < 1e-3 and abs(tokens - 2.941) < 1e-3
    assert abs(tokens - g["printed_speedup"]) < 0.1


def test_full_tree_node_count():
    g = GOLDEN["tree_node_count"]
    rng = np.random.default_rng(0)
    _, par, tok, dep, _ = synth.build_topk_tree(rng, 40, n_max=10 ** 6, width=g["width"],
                                                depth=g["gamma"])
    assert len(par) == g["printed_total"]
    assert np.bincount(dep).tolist() == g["printed_levels"]
    assert np.all(par[1:] < np.arange(1, len(par)))


def test_dynamic_gamma_thresholds():
    g = GOLDEN["dynamic_gamma"]
    w = g["window"]
    got = [synth.gamma_from_history(k, w) for k in range(w + 1)]
    for k, gm in enumerate(got):
        rate = k / w
        want = g["above_60"] if rate > 0.6 else (g["from_30_to_60"] if rate >= 0.3 else g["below_30"])
        assert gm == want


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.00390625, 1.005859375, 1.0078125, -3.3, 65504.0, 1e-40], dtype=np.float32)
    bits = synth.bf16_bits(vals)
    back = synth.bf16_values(bits).astype(np.float64)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0
    assert back[1] == 1.0
    for v, b, bb in zip(vals.astype(np.float64), bits, back):
        up = synth.bf16_values(np.array([b + 1], dtype=np.uint16))[0]
        dn = synth.bf16_values(np.array([b - 1], dtype=np.uint16))[0]
        assert abs(bb - v) <= abs(up - v) and abs(bb - v) <= abs(dn - v)


def test_generators_are_deterministic_and_shaped():
    a = synth.linear_v32k(B=4)
    b = synth.linear_v32k(B=4)
    assert np.array_equal(a["target"], b["target"]) and np.array_equal(a["tokens"], b["tokens"])
    assert a["target"].shape == (4 * 6, 32000) and a["draft"].shape == (4 * 5, 32000)
    assert a["target"].dtype == np.uint16
    c = synth.linear_v1000()
    assert c["target"].shape == (5, 1000) and c["target"].dtype == np.float32


def test_small_tree_generator_structure():
    d = synth.tree_v32k(B=3, N=16, V=500)
    for b in range(3):
        n = d["n_nodes"][b]
        par = d["parents"][b, :n]
        assert par[0] == -1 and np.all(par[1:] < np.arange(1, n)) and np.all(par[1:] >= 0)
        # siblings in descending draft probability: ranks increase with index
        for node in range(n):
            kids = np.where(par == node)[0]
            assert np.all(np.diff(kids) > 0)


def test_bimodal_generator_gammas():
    d = synth.bimodal_v152k(B=64, V=256)
    assert set(np.unique(d["gammas"])) <= {2, 4, 8}
    lo = d["gammas"][d["sigma"] > 1.0]
    hi = d["gammas"][d["sigma"] < 1.0]
    assert np.mean(lo == 2) > 0.8 and np.mean(hi >= 4) > 0.8
    assert d["offsets"][-1] == d["gammas"].sum()
