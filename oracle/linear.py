"""Linear (chain) verify step, float64 (oracle; test infrastructure).

What is computed, per batch row b with gamma = gamma_b draft tokens
d_0..d_{gamma-1} (target positions 0..gamma, draft positions 0..gamma-1):

1. Temperature softmax of every target row and every draft row over the
   vocabulary, p_i = softmax(x_i / T_t) and q_i = softmax(y_i / T_d)
   (kwkr §3.3 and §5.2 set draft and target temperatures separately).  A
   temperature of 0 is greedy decoding: a one-hot at the first maximum
   (kwkr §4.3 "first pitfall": rejection then reduces to exact match).
2. Acceptance of d_i with probability min(1, p_i(d_i) / q_i(d_i)): accept
   outright when p >= q, otherwise with probability p/q (kwkr §2.3, §4.1;
   cf-1 §2.2).  It is taken as "u < min(1, r_i)" with a counter-based
   uniform u = u_acc(i+1) (d_i sits in sequence slot i+1); since u < 1 this
   is "u < r_i".
3. Stop at the first rejection and drop every later draft token (kwkr §4.3
   "third pitfall"; the lonae formal-definition paragraph).
4. On a rejection at i, draw the replacement from the normalised residual
   max(0, p_i - q_i) (lonae formal-definition paragraph).  kwkr §2.3/§4.1 and
   cf-1 §2.1 say "resample from the target"; that variant does not preserve
   the target law (a plain enumeration shows it), so the residual is used.
5. When all gamma drafts are accepted, draw the bonus token from p_gamma, the
   target row after the last draft (the lonae paragraph counts gamma drafts
   plus one bonus position).

Draws are by inverse CDF in vocabulary order: the smallest index k whose
cumulative mass exceeds u * R, R the total mass of the unnormalised weights.

Edge readings (silent on the pages):
* q_i(d_i) = 0 with p_i(d_i) > 0 gives r = +inf (accept); both zero gives
  r = 0 (reject).  The row is marked with WARN_QZERO.
* A rejection whose residual mass is exactly zero (possible only through
  rounding) draws from p_i instead; the row is marked with WARN_RZERO.
* A token outside [0, V), a negative or non-finite temperature, or a row
  whose maximum logit is not finite makes the row an error row:
  num_accepted = -1 and every output token -1.
"""

from dataclasses import dataclass, field

import numpy as np

from .decode import decode_logits
from .philox import verify_uniforms

# Row status bits (errors make the row's outputs -1; warnings do not).
ROW_OK = 0
ROW_BAD_TOKEN = 1
ROW_BAD_SHAPE = 2
ROW_NONFINITE = 4
ROW_BAD_TEMP = 8
ROW_WARN_QZERO = 256
ROW_WARN_RZERO = 512
ROW_ERROR_MASK = 0xFF

# A decision whose float margin is below this is "flagged": a float32
# implementation may legitimately decide it the other way.
FLAG_EPS = 1e-6


def softmax_t(logits, temp):
    """softmax(logits / temp) in float64; temp == 0 gives a one-hot at the first maximum."""
    x = np.asarray(logits, dtype=np.float64)
    if temp == 0.0:
        p = np.zeros_like(x)
        p[int(np.argmax(x))] = 1.0
        return p
    z = x / temp
    z = z - np.max(z)
    e = np.exp(z)
    return e / np.sum(e)


def residual_weights(p, q):
    """Unnormalised residual max(0, p - q) (lonae formal-definition paragraph)."""
    return np.maximum(p - q, 0.0)


def inverse_cdf(weights, u):
    """Smallest index k with C(k) > u * R, C the cumulative sum in index order.

    Returns (k, margin): margin is the distance of u * R from the nearer of
    C(k-1) and C(k), in the same (probability) units as the weights.
    """
    c = np.cumsum(weights)
    total = c[-1]
    t = u * total
    k = int(np.searchsorted(c, t, side="right"))
    k = min(k, len(c) - 1)
    lo = c[k - 1] if k > 0 else 0.0
    margin = min(abs(t - lo), abs(c[k] - t))
    return k, float(margin)


@dataclass
class LinearRowResult:
    num_accepted: int
    out_tokens: np.ndarray          # [gamma + 1], -1 padded
    p_at_draft: np.ndarray          # [gamma]
    q_at_draft: np.ndarray          # [gamma]
    ratio: np.ndarray               # [gamma] r_i = p_i(d_i) / q_i(d_i)
    status: int = ROW_OK
    # Index of the first acceptance decision whose margin |u - r| < FLAG_EPS
    # among the decisions taken (None if none): outputs from there on are
    # not unique under float32.
    flagged_accept: object = None
    # True when the final draw's margin is below FLAG_EPS.
    flagged_sample: bool = False
    stop_kind: str = ""             # "reject", "bonus", "greedy" or "error"
    min_accept_margin: float = field(default=np.inf)


def verify_linear_row(x, y, tokens, temp_t, temp_d, u_acc, u_smp):
    """Verify one row.

    x: [gamma+1, V] target logits (float64); y: [gamma, V] draft logits;
    tokens: [gamma] draft token ids; u_acc, u_smp: [gamma+1] uniforms indexed
    by sequence slot: slot 0 is the last committed token and d_i sits in slot
    i+1, so the acceptance of d_i uses u_acc[i+1] and the draw made after
    slot k (at target position k) uses u_smp[k].  u_acc[0] is unused.
    """
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    tokens = np.asarray(tokens, dtype=np.int64)
    gamma = len(tokens)
    V = x.shape[1]
    out = np.full(gamma + 1, -1, dtype=np.int64)
    p_at = np.zeros(gamma)
    q_at = np.zeros(gamma)
    ratio = np.zeros(gamma)

    def error(status):
        return LinearRowResult(-1, out, p_at, q_at, ratio, status, None, False, "error")

    if not (np.isfinite(temp_t) and np.isfinite(temp_d)) or temp_t < 0 or temp_d < 0:
        return error(ROW_BAD_TEMP)
    if gamma and (tokens.min() < 0 or tokens.max() >= V):
        return error(ROW_BAD_TOKEN)
    if not np.all(np.isfinite(np.max(x, axis=1))) or (
            gamma and not np.all(np.isfinite(np.max(y, axis=1)))):
        return error(ROW_NONFINITE)

    status = ROW_OK
    p_rows = [softmax_t(x[i], temp_t) for i in range(gamma + 1)]
    q_rows = [softmax_t(y[i], temp_d) for i in range(gamma)]
    for i in range(gamma):
        p_at[i] = p_rows[i][tokens[i]]
        q_at[i] = q_rows[i][tokens[i]]
        if q_at[i] > 0:
            ratio[i] = p_at[i] / q_at[i]
        else:
            status |= ROW_WARN_QZERO
            ratio[i] = np.inf if p_at[i] > 0 else 0.0

    flagged = None
    min_margin = np.inf
    n_acc = gamma
    for i in range(gamma):
        margin = abs(u_acc[i + 1] - ratio[i])
        min_margin = min(min_margin, margin)
        if flagged is None and margin < FLAG_EPS:
            flagged = i
        if not (u_acc[i + 1] < ratio[i]):
            n_acc = i
            break

    out[:n_acc] = tokens[:n_acc]
    greedy = temp_t == 0.0
    if greedy:
        # p is one-hot: the residual max(0, p - q) and p itself both put all
        # their mass on argmax x_{n_acc}, so the draw is that argmax.
        w = p_rows[n_acc]
        kind = "greedy"
    elif n_acc < gamma:
        w = residual_weights(p_rows[n_acc], q_rows[n_acc])
        kind = "reject"
        if not np.sum(w) > 0:
            status |= ROW_WARN_RZERO
            w = p_rows[n_acc]
    else:
        w = p_rows[gamma]
        kind = "bonus"
    k, smp_margin = inverse_cdf(w, u_smp[n_acc])
    out[n_acc] = k
    flagged_sample = (not greedy) and smp_margin < FLAG_EPS
    return LinearRowResult(n_acc, out, p_at, q_at, ratio, status, flagged, flagged_sample,
                           kind, min_margin)


def verify_linear(target_logits, draft_logits, dtype, draft_offsets, draft_tokens,
                  temp_target, temp_draft, seed=0, step=0, row_ids=None):
    """Verify a ragged batch.

    target_logits: [sum(gamma_b + 1), V] as stored (bf16 bits or float32);
    draft_logits:  [sum(gamma_b), V]; draft_offsets: [B + 1]; the target rows
    of row b start at draft_offsets[b] + b.  Uniforms for row b come from
    Philox with row_id = row_ids[b] (or b) at slots 0..gamma_b.
    Returns (num_accepted [B], out_tokens [sum(gamma_b + 1)], p_at_draft,
    q_at_draft, row_status [B], per-row LinearRowResult list).
    """
    off = np.asarray(draft_offsets, dtype=np.int64)
    B = len(off) - 1
    toks = np.asarray(draft_tokens, dtype=np.int64)
    n_t = int(off[-1]) + B
    num_acc = np.full(B, -1, dtype=np.int64)
    out_tokens = np.full(n_t, -1, dtype=np.int64)
    p_at = np.zeros(int(off[-1]))
    q_at = np.zeros(int(off[-1]))
    status = np.zeros(B, dtype=np.int64)
    results = []
    for b in range(B):
        o0, o1 = int(off[b]), int(off[b + 1])
        if o1 < o0 or o1 - o0 > 64:
            status[b] = ROW_BAD_SHAPE
            results.append(None)
            continue
        g = o1 - o0
        t0 = o0 + b
        x = decode_logits(target_logits[t0:t0 + g + 1], dtype)
        y = decode_logits(draft_logits[o0:o1], dtype)
        rid = b if row_ids is None else int(row_ids[b])
        u_acc, u_smp = verify_uniforms(seed, step, rid, g + 1)
        r = verify_linear_row(x, y, toks[o0:o1], float(temp_target[b]), float(temp_draft[b]),
                              u_acc, u_smp)
        results.append(r)
        num_acc[b] = r.num_accepted
        out_tokens[t0:t0 + g + 1] = r.out_tokens
        p_at[o0:o1] = r.p_at_draft
        q_at[o0:o1] = r.q_at_draft
        status[b] = r.status
    return num_acc, out_tokens, p_at, q_at, status, results
