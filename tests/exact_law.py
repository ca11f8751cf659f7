"""Exact laws of the oracle's outputs by bisection over its uniforms.

Every random choice the oracle makes is a monotone, piecewise-constant
function of one uniform with the others held fixed: an acceptance is
"u < ratio" and an inverse-CDF draw is non-decreasing in u.  For such a
function, equal values at the two ends of an interval mean it is constant
on that interval, so bisection finds every jump to ~1e-13 with a few dozen
calls per jump, and the measure of each value is exact to that precision.
No formula of the method is retyped here: only the oracle is called.
"""

import numpy as np

ALMOST_ONE = 1.0 - 2.0 ** -40


def segments(f, lo=0.0, hi=ALMOST_ONE, tol=1e-13):
    """Measure of each value of a monotone step function f on [lo, hi].

    Returns a dict value -> length, with the total length rescaled to 1 so
    that [lo, hi] stands for [0, 1).
    """
    out = {}
    fl, fh = f(lo), f(hi)

    def rec(a, fa, b, fb):
        if fa == fb:
            out[fa] = out.get(fa, 0.0) + (b - a)
            return
        if b - a < tol:
            # jump located to within tol; split the sliver evenly
            out[fa] = out.get(fa, 0.0) + (b - a) / 2
            out[fb] = out.get(fb, 0.0) + (b - a) / 2
            return
        m = 0.5 * (a + b)
        fm = f(m)
        rec(a, fa, m, fm)
        rec(m, fm, b, fb)

    rec(lo, fl, hi, fh)
    scale = 1.0 / (hi - lo)
    return {k: v * scale for k, v in out.items()}


def accept_measure(f_accepts):
    """Measure of {u : f_accepts(u)} for an acceptance test of the form u < ratio."""
    seg = segments(lambda u: bool(f_accepts(u)))
    return seg.get(True, 0.0)


def ar_consistency_error(round_law, ar_prob, max_len):
    """Largest violation of the autoregressive identity for one verify round.

    round_law: dict tuple(tokens) -> probability that one round emits exactly
    that sequence.  ar_prob(seq, ctx) is the target's autoregressive
    probability of seq after context ctx.  For every sequence s with
    |s| = m <= max_len, later rounds continue autoregressively, so

      P_AR(s) = sum_{j < m} R(s[:j]) * P_AR(s[j:] | s[:j]) + P(round starts with s)

    must hold.  Returns max |lhs - rhs| over all s that carry mass on either side.
    """
    seqs = set()
    for s in round_law:
        for m in range(1, len(s) + 1):
            seqs.add(s[:m])
    worst = 0.0
    vocab = sorted({t for s in round_law for t in s})
    # extend with every sequence of length <= max_len over the vocabulary
    frontier = [()]
    allseq = []
    for _ in range(max_len):
        frontier = [s + (v,) for s in frontier for v in vocab]
        allseq.extend(frontier)
    for s in allseq:
        m = len(s)
        rhs = 0.0
        for j in range(1, m):
            rj = round_law.get(s[:j], 0.0)
            if rj:
                rhs += rj * ar_prob(s[j:], s[:j])
        rhs += sum(pr for t, pr in round_law.items() if len(t) >= m and t[:m] == s)
        lhs = ar_prob(s, ())
        worst = max(worst, abs(lhs - rhs))
    return worst


def law_distance(law, p):
    """max_v |law(v) - p(v)| for a dict law over token ids and a probability vector p."""
    dev = 0.0
    for v in range(len(p)):
        dev = max(dev, abs(law.get(v, 0.0) - p[v]))
    extra = sum(w for k, w in law.items() if not (0 <= k < len(p)))
    return max(dev, extra)
