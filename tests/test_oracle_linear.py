"""Pins of the linear-verify oracle against what the pages and the mathematics fix.

* exact law of the emitted token at V=8 equals the target softmax
  (lonae formal-definition paragraph: the corrected output law is the target
  law), with the "resample from the target" variant as a negative control;
* the joint law of a whole round is consistent with autoregressive sampling
  from the target (kwkr §4.1: the joint law of any finite sequence is the
  target's);
* the expected number of emitted tokens per round under a constant
  per-position acceptance alpha is (1 - alpha^(gamma+1)) / (1 - alpha)
  (cf-1 §2.3), exactly and by Philox Monte Carlo;
* all-accept / all-reject edge cases (cf-1 §3.3 asks for these first);
* T -> 0 reduces to exact match (kwkr §4.3).

The target law used for comparison comes from scipy.special.softmax (a
library routine), never from the oracle itself.
"""

import itertools

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
from oracle import linear as L
from exact_law import ALMOST_ONE, ar_consistency_error, law_distance, segments

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def lib_softmax(x, T):
    x = np.asarray(x, dtype=np.float64)
    if T == 0:
        p = np.zeros_like(x)
        p[np.argmax(x)] = 1.0
        return p
    return scipy.special.softmax(x / T)


def config1_rows(V, seed):
    """Draft N(0, 2^2); target = draft + N(0, 0.5^2) (the V=1000 workload's generator)."""
    rng = np.random.default_rng(seed)
    y = rng.normal(0.0, 2.0, size=V)
    x = y + rng.normal(0.0, 0.5, size=V)
    x1 = rng.normal(0.0, 2.0, size=V)
    return x, x1, y


def single_position_law(x0, x1, y0, Tt, Td):
    """Exact law of the first emitted token of a gamma=1 round (d ~ q enumerated)."""
    V = len(x0)
    q = lib_softmax(y0, Td)
    law = {}
    for d in range(V):
        if q[d] == 0:
            continue

        def run(ua, us):
            return L.verify_linear_row([x0, x1], [y0], [d], Tt, Td, [0.5, ua], [us, 0.5])

        A = segments(lambda u: run(u, 0.5).num_accepted == 1).get(True, 0.0)
        law[d] = law.get(d, 0.0) + q[d] * A
        if A < 1.0:
            emit = segments(lambda us: int(run(ALMOST_ONE, us).out_tokens[0]))
            for v, w in emit.items():
                law[v] = law.get(v, 0.0) + q[d] * (1.0 - A) * w
    return law


@pytest.mark.parametrize("seed,Tt,Td", [(0, 1.0, 1.0), (1, 1.0, 1.0), (2, 0.7, 1.3),
                                        (3, 1.5, 0.6), (4, 1.0, 1.0)])
def test_exact_law_v8_equals_target(seed, Tt, Td):
    x0, x1, y0 = config1_rows(8, seed)
    law = single_position_law(x0, x1, y0, Tt, Td)
    assert abs(sum(law.values()) - 1.0) < 1e-11
    assert law_distance(law, lib_softmax(x0, Tt)) < 1e-11


def test_negative_control_resample_from_target_is_lossy(monkeypatch):
    """Planting the 'resample from the target p' variant must break the law."""
    x0, x1, y0 = config1_rows(8, 0)
    monkeypatch.setattr(L, "residual_weights", lambda p, q: p.copy())
    law = single_position_law(x0, x1, y0, 1.0, 1.0)
    assert law_distance(law, lib_softmax(x0, 1.0)) > 1e-3


def test_negative_control_residual_sign_flip_is_lossy(monkeypatch):
    """Planting max(0, q - p) (a wrong sign) must break the law."""
    x0, x1, y0 = config1_rows(8, 1)
    monkeypatch.setattr(L, "residual_weights", lambda p, q: np.maximum(q - p, 0.0))
    law = single_position_law(x0, x1, y0, 1.0, 1.0)
    assert law_distance(law, lib_softmax(x0, 1.0)) > 1e-3


def test_negative_control_dropped_temperature_is_lossy(monkeypatch):
    """Planting a softmax that ignores the temperature must break the law at T != 1."""
    x0, x1, y0 = config1_rows(8, 2)
    orig = L.softmax_t
    monkeypatch.setattr(L, "softmax_t", lambda v, T: orig(v, 1.0) if T != 0 else orig(v, T))
    law = single_position_law(x0, x1, y0, 0.7, 1.3)
    assert law_distance(law, lib_softmax(x0, 0.7)) > 1e-3


class ContextTable:
    """A toy 'model': logits are a fixed random function of the context."""

    def __init__(self, V, seed, scale_t=1.5, scale_d=1.5, pert=0.7):
        self.V, self.seed = V, seed
        self.scale_t, self.scale_d, self.pert = scale_t, scale_d, pert
        self.cache = {}

    def _rows(self, ctx):
        if ctx not in self.cache:
            h = hash((self.seed,) + tuple(ctx)) & 0xFFFFFFFF
            rng = np.random.default_rng(h)
            d = rng.normal(0, self.scale_d, self.V)
            t = d + rng.normal(0, self.pert, self.V)
            self.cache[ctx] = (t, d)
        return self.cache[ctx]

    def target(self, ctx):
        return self._rows(tuple(ctx))[0]

    def draft(self, ctx):
        return self._rows(tuple(ctx))[1]


def linear_round_law(tab, gamma, Tt, Td):
    """Exact law of the token sequence one linear verify round emits."""
    V = tab.V
    law = {}
    for drafts in itertools.product(range(V), repeat=gamma):
        w = 1.0
        for i, d in enumerate(drafts):
            w *= lib_softmax(tab.draft(drafts[:i]), Td)[d]
        if w == 0.0:
            continue
        x = [tab.target(drafts[:i]) for i in range(gamma + 1)]
        y = [tab.draft(drafts[:i]) for i in range(gamma)]

        def run(ua, us):
            return L.verify_linear_row(x, y, drafts, Tt, Td, ua, us)

        reach = 1.0
        for k in range(gamma + 1):
            if reach == 0.0:
                break
            if k < gamma:
                head = [0.5] + [0.0] * k
                tail = [ALMOST_ONE] * (gamma - k - 1)
                A = segments(lambda u: run(head + [u] + tail, [0.5] * (gamma + 1))
                             .num_accepted > k).get(True, 0.0)
                p_stop = reach * (1.0 - A)
                ua_stop = head + [ALMOST_ONE] + tail
            else:
                A = 0.0
                p_stop = reach
                ua_stop = [0.5] + [0.0] * gamma
            if p_stop > 0.0:
                def emit(us, k=k, ua_stop=ua_stop):
                    u_smp = [0.5] * (gamma + 1)
                    u_smp[k] = us
                    return int(run(ua_stop, u_smp).out_tokens[k])
                for v, pv in segments(emit).items():
                    s = tuple(drafts[:k]) + (v,)
                    law[s] = law.get(s, 0.0) + w * p_stop * pv
            reach *= A
    return law


@pytest.mark.parametrize("V,gamma,seed,Tt,Td", [(4, 2, 11, 1.0, 1.0), (3, 3, 12, 0.8, 1.2),
                                               (4, 2, 13, 1.2, 0.7)])
def test_round_law_is_autoregressive(V, gamma, seed, Tt, Td):
    tab = ContextTable(V, seed)
    law = linear_round_law(tab, gamma, Tt, Td)
    assert abs(sum(law.values()) - 1.0) < 1e-10

    def ar(seq, ctx):
        pr, c = 1.0, tuple(ctx)
        for t in seq:
            pr *= lib_softmax(tab.target(c), Tt)[t]
            c = c + (t,)
        return pr

    assert ar_consistency_error(law, ar, gamma + 1) < 1e-10


def constant_alpha_rows(gamma):
    # p = (0.5, 0.2, 0.3), q = (0.5, 0.5, 0): sum_v min(p, q) = 0.7 at every position
    x = np.log(np.array([0.5, 0.2, 0.3]))
    y = np.log(np.array([0.5, 0.5, 0.0]))
    return np.tile(x, (gamma + 1, 1)), np.tile(y, (gamma, 1))


def test_constant_alpha_exact_expected_tokens():
    """Per-position acceptance = sum min(p, q) = 0.7 exactly, so the expected tokens
    per round is sum_k alpha^k = (1 - alpha^(gamma+1)) / (1 - alpha) (cf-1 §2.3)."""
    gamma = 5
    x, y = constant_alpha_rows(gamma)
    q = np.array([0.5, 0.5, 0.0])
    alpha = 0.0
    for d in (0, 1):
        A = segments(lambda u: L.verify_linear_row(x[:2], y[:1], [d], 1.0, 1.0, [0.5, u],
                                                   [0.5, 0.5]).num_accepted == 1)
        alpha += q[d] * A.get(True, 0.0)
    assert abs(alpha - 0.7) < 1e-12
    # The rows are identical and the uniforms independent across slots, so
    # P(num_accepted >= k) = alpha^k and E[emitted] = sum_{k<=gamma} alpha^k.
    mean_emitted = sum(alpha ** k for k in range(gamma + 1))
    assert abs(mean_emitted - (1 - 0.7 ** 6) / (1 - 0.7)) < 1e-10
    assert abs(mean_emitted - 2.94117) < 1e-5


def test_constant_alpha_monte_carlo_closed_form():
    """Full batch path (Philox uniforms, ragged packing) vs the closed form."""
    gamma, B = 5, 4096
    rng = np.random.default_rng(7)
    x, y = constant_alpha_rows(gamma)
    tgt = np.tile(x, (B, 1)).astype(np.float32)
    dft = np.tile(y, (B, 1)).astype(np.float32)
    toks = rng.integers(0, 2, size=B * gamma)      # q = (0.5, 0.5, 0)
    off = np.arange(B + 1) * gamma
    T = np.ones(B, dtype=np.float32)
    n_acc, *_ = oracle.verify_linear(tgt, dft, 0, off, toks, T, T, seed=3, step=1)
    emitted = n_acc + 1
    closed = (1 - 0.7 ** (gamma + 1)) / (1 - 0.7)
    se = emitted.std() / np.sqrt(B)
    assert abs(emitted.mean() - closed) < 4 * se
    # truncated geometric law of num_accepted
    expect = np.array([0.7 ** k * 0.3 for k in range(gamma)] + [0.7 ** gamma]) * B
    obs = np.bincount(n_acc, minlength=gamma + 1)
    chi2 = ((obs - expect) ** 2 / expect).sum()
    assert scipy.stats.chi2.sf(chi2, gamma) > 1e-3


def test_all_accept_when_target_equals_draft():
    rng = np.random.default_rng(5)
    gamma, V = 6, 50
    y = rng.normal(0, 3, size=(gamma, V))
    x = np.vstack([y, rng.normal(0, 3, size=(1, V))])
    toks = [int(np.argmax(y[i] + rng.gumbel(size=V))) for i in range(gamma)]
    for seed in range(20):
        u_acc, u_smp = oracle.verify_uniforms(seed, 0, 0, gamma + 1)
        r = L.verify_linear_row(x, y, toks, 1.0, 1.0, u_acc, u_smp)
        assert r.num_accepted == gamma and r.stop_kind == "bonus"
        assert list(r.out_tokens[:gamma]) == toks
        assert np.all(r.ratio == 1.0)


def test_all_accept_bonus_law_is_target():
    rng = np.random.default_rng(6)
    V = 6
    y = rng.normal(0, 2, size=(1, V))
    xb = rng.normal(0, 2, size=V)
    x = np.vstack([y, xb])
    emit = segments(lambda us: int(L.verify_linear_row(x, y, [2], 1.0, 1.0, [0.5, 0.3],
                                                       [0.5, us]).out_tokens[1]))
    assert law_distance(emit, lib_softmax(xb, 1.0)) < 1e-12


def test_all_reject_when_target_excludes_drafts():
    rng = np.random.default_rng(8)
    gamma, V = 4, 40
    y = rng.normal(0, 2, size=(gamma, V))
    x = rng.normal(0, 2, size=(gamma + 1, V))
    toks = [int(np.argmax(y[i])) for i in range(gamma)]
    for i in range(gamma):
        x[i, toks[i]] = -np.inf
    for seed in range(20):
        u_acc, u_smp = oracle.verify_uniforms(seed, 0, 0, gamma + 1)
        r = L.verify_linear_row(x, y, toks, 1.0, 1.0, u_acc, u_smp)
        assert r.num_accepted == 0 and r.stop_kind == "reject"
        k = r.out_tokens[0]
        assert k != toks[0]
        assert lib_softmax(x[0], 1.0)[k] > lib_softmax(y[0], 1.0)[k]   # residual > 0
        assert np.all(r.out_tokens[1:] == -1)
    # the emitted law is the normalised residual at position 0
    p, q = lib_softmax(x[0], 1.0), lib_softmax(y[0], 1.0)
    res = np.maximum(p - q, 0)
    emit = segments(lambda us: int(L.verify_linear_row(x, y, toks, 1.0, 1.0,
                                                       [0.5] * (gamma + 1),
                                                       [us] + [0.5] * gamma).out_tokens[0]))
    assert law_distance(emit, res / res.sum()) < 1e-12


def distinct_gap_rows(rng, n, V):
    """Rows of bf16-exact logits, all distinct and 0.0625 apart (gap >= one bf16 step near 8-16)."""
    rows = []
    for _ in range(n):
        rows.append((rng.permutation(V) - V / 2) * 0.0625)
    return np.array(rows)


def test_greedy_is_exact_match():
    rng = np.random.default_rng(9)
    gamma, V = 7, 64
    for trial in range(40):
        x = rng.normal(0, 2, size=(gamma + 1, V))
        y = rng.normal(0, 2, size=(gamma, V))
        am = np.argmax(x, axis=1)
        toks = [int(am[i]) if rng.random() < 0.7 else int(rng.integers(V)) for i in range(gamma)]
        u_acc, u_smp = oracle.verify_uniforms(trial, 0, 0, gamma + 1)
        r = L.verify_linear_row(x, y, toks, 0.0, 0.8, u_acc, u_smp)
        k = next((i for i in range(gamma) if toks[i] != am[i]), gamma)
        assert r.num_accepted == k
        assert list(r.out_tokens[:k]) == toks[:k]
        assert r.out_tokens[k] == am[k]


def test_argmax_ties_take_lowest_index():
    x = np.array([[1.0, 3.0, 3.0, 2.0]])
    r = L.verify_linear_row(x, np.zeros((0, 4)), [], 0.0, 0.0, [0.5], [0.5])
    assert r.out_tokens[0] == 1


def test_small_temperature_matches_greedy_on_gapped_rows():
    rng = np.random.default_rng(10)
    gamma, V = 5, 64
    same = 0
    for trial in range(30):
        x = distinct_gap_rows(rng, gamma + 1, V)
        y = distinct_gap_rows(rng, gamma, V)
        ya = np.argmax(y, axis=1)
        toks = [int(np.argmax(x[i])) if rng.random() < 0.6 else int(ya[i]) for i in range(gamma)]
        u_acc, u_smp = oracle.verify_uniforms(trial, 0, 0, gamma + 1)
        g = L.verify_linear_row(x, y, toks, 0.0, 0.0, u_acc, u_smp)
        s = L.verify_linear_row(x, y, toks, 1e-3, 1e-3, u_acc, u_smp)
        assert g.num_accepted == s.num_accepted
        assert np.array_equal(g.out_tokens, s.out_tokens)
        same += 1
    assert same == 30


def test_inverse_cdf_boundaries_and_zero_mass():
    w = np.array([0.0, 0.25, 0.0, 0.5, 0.25])
    assert L.inverse_cdf(w, 0.0)[0] == 1
    assert L.inverse_cdf(w, 0.25)[0] == 3          # C(1) = 0.25 is not > 0.25
    assert L.inverse_cdf(w, 0.75 - 1e-12)[0] == 3
    assert L.inverse_cdf(w, 0.75)[0] == 4
    law = segments(lambda u: L.inverse_cdf(w, u)[0])
    assert law_distance(law, w) < 1e-12


def test_error_rows():
    x = np.zeros((3, 5))
    y = np.zeros((2, 5))
    u = [0.5] * 3
    assert L.verify_linear_row(x, y, [0, 5], 1.0, 1.0, u, u).status == L.ROW_BAD_TOKEN
    assert L.verify_linear_row(x, y, [0, 1], -1.0, 1.0, u, u).status == L.ROW_BAD_TEMP
    x2 = x.copy()
    x2[1] = -np.inf
    r = L.verify_linear_row(x2, y, [0, 1], 1.0, 1.0, u, u)
    assert r.status == L.ROW_NONFINITE and r.num_accepted == -1
    assert np.all(r.out_tokens == -1)


def test_q_zero_warning_accepts():
    x = np.log(np.array([[0.5, 0.5, 1e-300], [0.3, 0.3, 0.4]]))
    y = np.log(np.array([[1.0, 1e-300, 0.0]]))
    y[0, 2] = -np.inf
    r = L.verify_linear_row(x, y, [2], 1.0, 1.0, [0.5, 0.9], [0.5, 0.5])
    assert r.status & L.ROW_WARN_QZERO
    assert r.num_accepted == 1


def test_ragged_batch_uses_row_ids_not_packing():
    rng = np.random.default_rng(12)
    V = 30
    gammas = [3, 0, 5, 1]
    off = np.concatenate([[0], np.cumsum(gammas)])
    B = len(gammas)
    tgt = rng.normal(0, 2, size=(int(off[-1]) + B, V)).astype(np.float32)
    dft = rng.normal(0, 2, size=(int(off[-1]), V)).astype(np.float32)
    toks = rng.integers(0, V, size=int(off[-1]))
    T = np.ones(B, dtype=np.float32)
    ids = np.array([40, 41, 42, 43], dtype=np.uint32)
    full = oracle.verify_linear(tgt, dft, 0, off, toks, T, T, seed=5, step=9, row_ids=ids)
    # row 2 alone, with the same row id, gives the same outputs
    b = 2
    o0, o1 = int(off[b]), int(off[b + 1])
    t0 = o0 + b
    solo = oracle.verify_linear(tgt[t0:t0 + gammas[b] + 1], dft[o0:o1], 0,
                                np.array([0, gammas[b]]), toks[o0:o1], T[:1], T[:1],
                                seed=5, step=9, row_ids=ids[b:b + 1])
    assert full[0][b] == solo[0][0]
    assert np.array_equal(full[1][t0:t0 + gammas[b] + 1], solo[1])
    assert full[0][1] == 0 and full[1][off[1] + 1] >= 0


def test_negative_control_round_law(monkeypatch):
    """The joint-law check must reject the lossy 'resample from p' variant too."""
    monkeypatch.setattr(L, "residual_weights", lambda p, q: p.copy())
    tab = ContextTable(4, 11)
    law = linear_round_law(tab, 2, 1.0, 1.0)

    def ar(seq, ctx):
        pr, c = 1.0, tuple(ctx)
        for t in seq:
            pr *= lib_softmax(tab.target(c), 1.0)[t]
            c = c + (t,)
        return pr

    assert ar_consistency_error(law, ar, 3) > 1e-3
