"""CPU checks of the float32 draw bound (tests/draw_bound.py) the GPU parity
tests hold every emitted token to.

* The oracle's own token is always admissible, and a decidable draw has only
  that token.
* A float32 computation of the stop weights written here (2^(x k^ - c) with
  k^ = float32(log2(e)/T), a float32 exponent and 2^x, the float64 row sum, a
  float32 1/s and product, the float32 residual) draws an admissible token on
  every row.
* Weights perturbed at random anywhere inside the per-token bound draw
  admissible tokens; perturbations twenty times larger do not (the check has
  teeth).
"""

import numpy as np

import draw_bound as DB
import synth
from oracle import linear as OL


def f32_probs(x, T):
    """Softmax weights formed as the vocabulary pass and the finish pass form them."""
    x32 = x.astype(np.float32)
    kh = np.float32(DB.LOG2E / float(np.float32(T)))
    c = np.ceil(np.float32(np.max(x32) * kh))
    t = (x32.astype(np.float64) * float(kh) - float(c)).astype(np.float32)   # one rounding (fma)
    e = np.exp2(t)                                                           # float32 2^x
    s = float(np.sum(e.astype(np.float64)))
    inv = np.float32(1.0 / s)
    return (e * inv).astype(np.float32)


def f32_draw(w32, u):
    c = np.cumsum(w32.astype(np.float64))
    k = int(np.searchsorted(c, u * c[-1], side="right"))
    return min(k, len(c) - 1)


def rows(seed, n, V):
    rng = np.random.default_rng(seed)
    for i in range(n):
        y = synth.bf16_values(synth.bf16_bits(rng.normal(0, 3, size=V).astype(np.float32)))
        sig = rng.choice([0.05, 0.3, 1.0])
        x = synth.bf16_values(synth.bf16_bits((y + rng.normal(0, sig, size=V)).astype(np.float32)))
        T = float(rng.choice(np.array([0.6, 0.8, 1.0, 1.3], dtype=np.float32)))
        yield x.astype(np.float64), y.astype(np.float64), T, rng.uniform()


def test_oracle_token_is_admissible_and_bound_is_small():
    for x, y, T, u in rows(1, 40, 5000):
        for w, e in (DB.prob_bound(x, T), DB.residual_bound(x, y, T, T)):
            ok, k, margin, window = DB.admissible(w, e, u)
            assert ok[k]
            assert window < 5e-6
            if margin > 2 * window:
                assert ok.sum() == 1


def test_float32_weights_draw_admissible_tokens():
    differ = 0
    for x, y, T, u in rows(2, 120, 20000):
        p32, q32 = f32_probs(x, T), f32_probs(y, T)
        for w32, (w, e) in ((p32, DB.prob_bound(x, T)),
                            (np.maximum(p32 - q32, np.float32(0)), DB.residual_bound(x, y, T, T))):
            k32 = f32_draw(w32, u)
            ok, k, _, _ = DB.admissible(w, e, u)
            assert ok[k32], (k32, k)
            # the float32 weights themselves lie inside the per-token bound
            assert np.all(np.abs(w32.astype(np.float64) - w) <= e)
            differ += int(k32 != k)
    assert differ <= 3


def test_perturbations_inside_the_bound_stay_admissible():
    rng = np.random.default_rng(3)
    bad_small = bad_large = 0
    for x, y, T, u in rows(4, 60, 3000):
        w, e = DB.residual_bound(x, y, T, T)
        ok, k, _, _ = DB.admissible(w, e, u)
        # move u * R onto a boundary region so that perturbations matter
        c = np.cumsum(w)
        j = int(np.nonzero(w > 0)[0][len(np.nonzero(w > 0)[0]) // 2])
        u = float(c[j] / c[-1])
        ok, k, _, _ = DB.admissible(w, e, u)
        for _ in range(20):
            wp = np.maximum(w + e * rng.uniform(-1, 1, size=len(w)), 0.0)
            bad_small += int(not ok[OL.inverse_cdf(wp, u)[0]])
            wl = np.maximum(w + 20 * e * rng.uniform(-1, 1, size=len(w)), 0.0)
            bad_large += int(not ok[OL.inverse_cdf(wl, u)[0]])
    assert bad_small == 0
    assert bad_large > 0


def test_masked_tokens_are_never_admissible():
    x, y, T, u = next(rows(5, 1, 4000))
    w, e = DB.prob_bound(x, T)
    masked = np.zeros(len(w), dtype=bool)
    top = np.argsort(-w)[:4]
    masked[top] = True
    w = np.where(masked, 0.0, w)
    for uu in np.linspace(0.0, 0.999, 50):
        ok, k, _, _ = DB.admissible(w, e, uu, masked)
        assert ok[k] and not ok[top].any()


def test_wor_bound_matches_the_oracle_recursion():
    """The lambda form's weights equal the oracle's recursive residual (up to scale)."""
    rng = np.random.default_rng(6)
    V = 300
    for trial in range(20):
        y = rng.normal(0, 2, size=V)
        x = y + rng.normal(0, 0.8, size=V)
        toks = list(rng.choice(V, size=rng.integers(1, 12), replace=False))
        w, e = DB.wor_bound(x, y, 1.0, 1.0, toks)
        # the recursive residual after every child (token toks[j]) is rejected
        p = OL.softmax_t(x, 1.0)
        q = OL.softmax_t(y, 1.0)
        pj, qj = p.copy(), q.copy()
        for t in toks:
            res = np.maximum(pj - qj, 0.0)
            if res.sum() > 0:
                pj = res / res.sum()
            qj = qj.copy()
            qj[t] = 0.0
            qj = qj / qj.sum()
        assert np.allclose(w / w.sum(), pj, rtol=1e-9, atol=1e-15)
        assert np.all(e >= 0) and np.all(np.isfinite(e))
