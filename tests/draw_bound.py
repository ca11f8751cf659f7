"""Error bound of a float32 draw against the exact (float64) oracle draw.

The verify draws its emitted token by inverse CDF: the smallest index k whose
cumulative mass C(k) of the stop weights w exceeds u * R, R the total (the
lonae formal-definition paragraph gives the residual max(0, p - q) as the
distribution after a rejection; the bonus comes from p).  The oracle forms w
in float64.  The kernels form each weight in float32 and sum in float64, so
their D(j) = C(j) - u R differs from the oracle's by a bounded amount; a
token is an admissible GPU result when, for weights anywhere inside that
bound, inverse CDF could return it.  Every draw is checked against this set;
the oracle's own k is always in it, and a draw is decidable when it is the
only member.

The bound (derivation in the design notes, R14):

* a probability p_v = softmax(x / T)_v is formed as 2^(x_v k^ - c) / s with
  k^ = float32(log2(e) / T), c an integer offset at or above max_v x_v k^ - 1
  and s the float64 sum of the same float32 exponentials;
* |p^_v - p_v| <= |p_v(k^) - p_v(k)| + p_v (tau_v + sigma + 2 u32), where the
  first term is the exact effect of the rounded k (computed here in float64),
  tau_v = ln2 u32 (1 + (max x - x_v) k^) + eps_exp bounds the relative error
  of one exponential (the rounding of the float32 exponent, then the hardware
  2^x), sigma = sum_v p_v tau_v + 5 u32 that of s (the pairwise float32 sum of
  32 exponentials per lane), and 2 u32 the float32 1/s and the product;
* a residual weight max(0, p - q) adds the bounds of p and q and the float32
  difference u32 |p - q|;
* SAMPLED_WOR weights max(0, a - L_v b) (the lambda form of the recursive
  residual) add |dL_v| b_v, with dL propagated through each rejection to
  first order as a linear combination of each pass's independent errors (the
  result is doubled for the second-order terms);
* D(j) then errs by at most (1 - u) A(j) + u (A_tot - A(j)) with A the prefix
  sums of the weight bounds, plus 5 u32 (C(j + 8) + u R) for the float32 sums
  of eight weights per thread (or 32 per lane in the vocabulary pass's chunk
  masses) and 1e-12 R for the float64 sums.

eps_exp = 2^-23 (one float32 ulp) is the hardware 2^x error this assumes; the
GPU test of `spec_verify_exp2` measures the actual error against it (0.70 ulp
at most on 2^24 random exponents of [-126, 1]).
"""

import math

import numpy as np

U32 = 2.0 ** -24               # unit roundoff of float32
EPS_EXP = 2.0 ** -23           # relative error allowed for the hardware 2^x (one ulp)
LOG2E = 1.4426950408889634074
LN2 = math.log(2.0)
TINY = 2.0 ** -120             # absolute floor: flushed subnormal exponentials
SLACK = 1.01                   # second-order terms of the first-order bounds
WOR_SLACK = 2.0                # second-order terms of the propagation through the rejections


def k_hat(T):
    """log2(e) / T rounded once to float32, T the float32 temperature."""
    return float(np.float32(LOG2E / float(np.float32(T))))


def prob_bound(x, T):
    """(p, e): the exact softmax(x / T) in float64 and a bound on |p_gpu - p| per token."""
    x = np.asarray(x, dtype=np.float64)
    V = len(x)
    if T == 0.0:
        p = np.zeros(V)
        p[int(np.argmax(x))] = 1.0
        return p, np.zeros(V)
    T = float(np.float32(T))
    xm = np.max(x)
    z = (x - xm) / T
    p = np.exp(z)
    p /= p.sum()
    kh = k_hat(T)
    ph = np.exp2((x - xm) * kh)
    ph /= ph.sum()
    # a -inf logit has an exactly zero exponential on both sides: no error
    fin = np.isfinite(x)
    tau = np.where(fin, LN2 * U32 * (1.0 + (xm - np.where(fin, x, xm)) * kh) + EPS_EXP, 0.0)
    sigma = float(np.sum(p * tau)) + 5.0 * U32
    e = np.abs(ph - p) + p * (tau + sigma + 2.0 * U32)
    return p, SLACK * e + TINY


def residual_bound(x, y, Tt, Td):
    """Weights max(0, p - q) of a rejection and their bounds."""
    p, ep = prob_bound(x, Tt)
    q, eq = prob_bound(y, Td)
    w = np.maximum(p - q, 0.0)
    return w, ep + eq + U32 * np.abs(p - q)


def wor_bound(x, y, Tt, Td, rejected):
    """Weights of the draw after SAMPLED_WOR rejections of `rejected` (in test
    order) at one node, in the lambda form max(0, a - L_v b), and their bounds.

    Each rejection sets mu = lambda + P / Q, P the total of the current
    weights and Q the draft mass left.  P depends on every lambda the current
    weights were formed with (dP / dL_v = -b_v where a_v > L_v b_v), so the
    error of mu is propagated to first order as a linear combination of the
    independent errors of each pass (the weights' own bounds in P, the error of
    Q, the rounding of mu); the bound of each lambda is then the sum of the
    combination's absolute coefficients times the sources' bounds.
    """
    a, ea = prob_bound(x, Tt)
    b, eb = prob_bound(y, Td)
    V = len(a)
    n_src = len(rejected) + 1
    lam_vals = [0.0]                       # lambda values in use; lambda_0 = 0 exactly
    lam_coef = [np.zeros(n_src)]           # their errors as combinations of the sources
    src = np.zeros(n_src)                  # bounds of the independent sources
    ref = np.zeros(V, dtype=np.int64)      # which lambda each token's L refers to
    cur = 0                                # lambda of the tokens still in q
    removed = np.zeros(V, dtype=bool)
    Q, dQ = 1.0, 0.0
    for j, t in enumerate(rejected):
        if removed[t]:
            continue        # a repeated token has zero draft mass left: not a rejection of mass
        L = np.asarray(lam_vals)[ref]
        wts = a - L * b
        pos = wts > 0.0
        P = float(np.sum(wts[pos]))
        mu = lam_vals[cur] + P / Q
        eg = ea + L * eb + U32 * (a + L * b)
        near = wts > -eg
        dP_ind = float(np.sum(eg[near])) + 5.0 * U32 * P
        src[j] = dP_ind / Q + P * dQ / (Q * Q) + 2.0 * U32 * mu
        coef = lam_coef[cur].copy()
        for i in np.unique(ref[pos]):
            coef -= (float(np.sum(b[pos & (ref == i)])) / Q) * lam_coef[i]
        coef[j] += 1.0
        # the new weights: mu for the tokens still in q and for t itself
        stay = ~removed
        Ln = np.where(stay, mu, L)
        G = float(np.sum(np.maximum(a - Ln * b, 0.0)))
        if G > 0.0:
            lam_vals.append(mu)
            lam_coef.append(coef)
            cur = len(lam_vals) - 1
            ref = np.where(stay, cur, ref)
        removed[t] = True
        Q -= b[t]
        dQ = max(dQ + eb[t], float(np.sum(eb[~removed]))) + 5.0 * U32 * Q
        if not Q > 0.0:
            break
    L = np.asarray(lam_vals)[ref]
    dlam = np.array([float(np.sum(np.abs(c) * src)) for c in lam_coef])
    w = np.maximum(a - L * b, 0.0)
    e = ea + L * eb + dlam[ref] * b + U32 * (a + L * b)
    return w, WOR_SLACK * e + TINY


def admissible(w, e, u, masked=None):
    """Boolean mask of the tokens a draw within the bound may return, the
    oracle's token, and the bound on D at that token's two edges."""
    w = np.asarray(w, dtype=np.float64)
    e = np.asarray(e, dtype=np.float64)
    V = len(w)
    C = np.cumsum(w)
    R = C[-1]
    t = u * R
    A = np.cumsum(e)
    At = A[-1]
    D = C - t
    ahead = C[np.minimum(np.arange(V) + 8, V - 1)]
    delta = (1.0 - u) * A + u * (At - A) + 5.0 * U32 * (ahead + t) + 1e-12 * R
    D_prev = np.concatenate([[-t], D[:-1]])
    delta_prev = np.concatenate([[u * At + 5.0 * U32 * t + 1e-12 * R], delta[:-1]])
    choosable = (w > 0.0) | (e > 0.0)
    if masked is not None:
        choosable &= ~masked
    ok = choosable & (D + delta > 0.0) & (D_prev - delta_prev <= 0.0)
    if D[-1] - delta[-1] <= 0.0 and choosable.any():
        ok[np.nonzero(choosable)[0][-1]] = True      # u R left uncrossed by rounding
    k = int(np.searchsorted(C, t, side="right"))
    k = min(k, V - 1)
    lo = C[k - 1] if k > 0 else 0.0
    margin = min(abs(t - lo), abs(C[k] - t))
    window = max(delta_prev[k], delta[k])
    return ok, k, float(margin), float(window)


class DrawTally:
    """Counts of a parity run's draws: how many were compared, matched the
    oracle exactly, differed inside the bound, were decidable (one admissible
    token), and, among those the former absolute 1e-6 window would have
    excused, how many matched exactly."""

    def __init__(self):
        self.compared = self.exact = self.within = self.decidable = 0
        self.old_excused = self.old_excused_exact = 0
        self.max_window = 0.0

    def add(self, k_gpu, w, e, u, masked=None, old_eps=1e-6):
        ok, k, margin, window = admissible(w, e, u, masked)
        assert 0 <= k_gpu < len(w) and ok[k_gpu], (
            "drawn token %d outside the float32 bound: oracle %d, margin %.3g, window %.3g, "
            "admissible %s" % (k_gpu, k, margin, window, np.nonzero(ok)[0][:8].tolist()))
        self.compared += 1
        self.exact += int(k_gpu == k)
        self.within += int(k_gpu != k)
        self.decidable += int(ok.sum() == 1)
        self.max_window = max(self.max_window, window)
        if margin < old_eps:
            self.old_excused += 1
            self.old_excused_exact += int(k_gpu == k)
        return k_gpu == k

    def summary(self):
        return dict(draws=self.compared, exact=self.exact, within_bound=self.within,
                    decidable=self.decidable, old_window_excused=self.old_excused,
                    old_window_excused_exact=self.old_excused_exact,
                    max_window=self.max_window)
