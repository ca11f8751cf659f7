"""GPU parity of spec_verify_linear against the oracle (element by element).

Covers the V=1000 fp32 workload, the V=32000 / V=128256 / V=152064 bf16
workloads at full size, several-chunk ragged tails, unaligned vocabularies,
greedy and mixed-greedy rows, all-accept / all-reject, error rows, row ids,
determinism, and the V=8 distribution check over 10^6 trials.
"""

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
import synth
from gpu_util import (compare_linear, run_linear, run_oracle_linear, say, torch_mod)

pytestmark = pytest.mark.gpu


def check(d, label, **kw):
    say("[linear] %s: B=%d V=%d dtype=%d sum_gamma=%d" % (label, d["B"], d["V"], d["dtype"],
                                                         int(d["offsets"][-1])))
    gpu = run_linear(d, **kw)
    ref = run_oracle_linear(d, **kw)
    s = compare_linear(gpu, ref, d, seed=kw.get("seed"), step=kw.get("step"),
                       row_ids=kw.get("row_ids"))
    say("[linear] %s: ok %s" % (label, s))
    return gpu, ref, s


def ragged(seed, gammas, V, dtype, temps=None, sigma=1.0, draft_sd=3.0):
    rng = np.random.default_rng(seed)
    B = len(gammas)
    T = np.full(B, 0.9, dtype=np.float32) if temps is None else np.asarray(temps, np.float32)
    return synth._linear_batch(rng, gammas, V, draft_sd, np.full(B, sigma), T, T.copy(), dtype)


def test_v1000_fp32():
    check(synth.linear_v1000(), "v1000 fp32")


def test_v32k_bf16_full():
    check(synth.linear_v32k(), "v32k bf16")


def test_ragged_multichunk_bf16():
    rng = np.random.default_rng(11)
    gammas = rng.integers(0, 9, size=24)
    check(ragged(11, gammas, 20000, synth.BF16, sigma=0.6), "ragged 20000 bf16")


def test_ragged_multichunk_fp32_unaligned():
    rng = np.random.default_rng(12)
    gammas = rng.integers(0, 7, size=12)
    check(ragged(12, gammas, 10007, synth.F32, sigma=0.4), "ragged 10007 fp32 (scalar path)")


def test_ragged_fp32_five_chunks():
    # V = 40000 fp32 (aligned, 5 chunks): the pipelined mass pass in fp32
    rng = np.random.default_rng(21)
    gammas = rng.integers(0, 7, size=10)
    check(ragged(21, gammas, 40000, synth.F32, sigma=0.5), "ragged 40000 fp32")


@pytest.mark.parametrize("B", [700, 1100])
def test_many_rows_five_chunks(B):
    """More batch rows than the mass pass stages decisions for in LDS (512)
    and, at 1100, than the vocabulary pass stages offsets for (1024): V =
    40000 bf16 (five chunks, the pipelined mass pass), ragged gamma of 0-3,
    with a token out of range and a bad temperature."""
    rng = np.random.default_rng(40 + B)
    gammas = rng.integers(0, 4, size=B)
    d = ragged(40 + B, gammas, 40000, synth.BF16, sigma=0.5)
    d["tokens"] = d["tokens"].copy()
    d["temp_target"] = d["temp_target"].copy()
    o = int(d["offsets"][B - 3])
    if d["offsets"][B - 2] > o:
        d["tokens"][o] = 40000                 # out of range: an error row
    d["temp_target"][B // 2] = np.nan            # bad temperature: an error row
    gpu, ref, s = check(d, "%d rows, V=40000 bf16" % B)
    assert gpu["num_accepted"][B // 2] == -1


def test_unaligned_bf16():
    check(ragged(13, [3, 5, 0, 2], 8191, synth.BF16, sigma=0.5), "8191 bf16 (scalar path)")


def test_greedy_and_mixed_temperatures():
    gammas = [6] * 8
    T_t = np.array([0, 0, 0.7, 1.0, 0.0, 1.3, 0.5, 0], dtype=np.float32)
    T_d = np.array([0, 0.8, 0.0, 1.0, 0.0, 0.0, 0.5, 0.6], dtype=np.float32)
    rng = np.random.default_rng(14)
    d = synth._linear_batch(rng, gammas, 9000, 3.0, np.full(8, 0.3), T_t, T_d, synth.BF16)
    # for greedy-draft rows, use the draft argmax as the draft token
    dv = synth.bf16_values(d["draft"])
    for b in range(8):
        if T_d[b] == 0:
            o0, o1 = d["offsets"][b], d["offsets"][b + 1]
            d["tokens"][o0:o1] = np.argmax(dv[o0:o1], axis=1)
    check(d, "greedy/mixed")


def test_all_accept_and_all_reject():
    rng = np.random.default_rng(15)
    d = ragged(15, [5] * 6, 12000, synth.BF16)
    tv = d["target"].copy()
    # rows 0-2: target rows equal draft rows (same temperature) -> all accepted
    for b in range(3):
        o0 = d["offsets"][b]
        tv[o0 + b:o0 + b + 5] = d["draft"][o0:o0 + 5]
    # rows 3-5: target logit at each draft token = -inf -> first draft rejected
    for b in range(3, 6):
        o0 = d["offsets"][b]
        for i in range(5):
            tv[o0 + b + i, d["tokens"][o0 + i]] = 0xFF80
    d["target"] = tv
    gpu, ref, _ = check(d, "all-accept/all-reject")
    assert list(gpu["num_accepted"]) == [5, 5, 5, 0, 0, 0]


def test_error_rows_do_not_stop_the_batch():
    d = ragged(16, [3, 4, 2, 5, 3], 5000, synth.BF16)
    d["tokens"] = d["tokens"].copy()
    d["tokens"][d["offsets"][1] + 2] = 5000           # row 1: token out of range
    d["temp_target"] = d["temp_target"].copy()
    d["temp_target"][2] = -1.0                        # row 2: bad temperature
    tv = d["target"].copy()
    o3 = d["offsets"][3] + 3
    tv[o3 + 1] = 0xFF80                               # row 3: an all -inf target row
    d["target"] = tv
    gpu, ref, _ = check(d, "error rows")
    assert list(gpu["num_accepted"][[1, 2, 3]]) == [-1, -1, -1]
    assert gpu["num_accepted"][0] >= 0 and gpu["num_accepted"][4] >= 0


def test_error_rows_multichunk():
    # V of three chunks: rows with nothing to draw are finished by their
    # first chunk's work item, the others by whichever chunk completes them
    d = ragged(18, [3, 4, 2, 5, 3, 6], 20000, synth.BF16)
    d["tokens"] = d["tokens"].copy()
    d["tokens"][d["offsets"][1] + 2] = -3             # row 1: token out of range
    d["temp_target"] = d["temp_target"].copy()
    d["temp_target"][2] = np.nan                      # row 2: bad temperature
    d["temp_target"][5] = 0.0                         # row 5: greedy (no draw)
    tv = d["target"].copy()
    o3 = d["offsets"][3] + 3
    tv[o3] = 0xFF80                                   # row 3: an all -inf target row
    d["target"] = tv
    gpu, ref, _ = check(d, "error rows, 3 chunks")
    assert list(gpu["num_accepted"][[1, 2, 3]]) == [-1, -1, -1]
    assert gpu["num_accepted"][0] >= 0 and gpu["num_accepted"][4] >= 0
    assert gpu["num_accepted"][5] >= 0


def test_longest_draft_runs():
    # gamma = 64 (the largest): 129 logit rows per decision, and Philox slot
    # 64 serves the 64th draft's test and the bonus draw after it
    for V, dt in ((1000, synth.F32), (20000, synth.BF16)):
        d = ragged(19, [64, 63, 40], V, dt, sigma=0.05)
        tv = d["target"].copy()
        o0 = d["offsets"][0]
        tv[o0:o0 + 64] = d["draft"][o0:o0 + 64]     # row 0: every draft accepted
        d["target"] = tv
        gpu, ref, _ = check(d, "gamma 64, V=%d" % V)
        assert gpu["num_accepted"][0] == 64


def test_largest_vocabulary():
    # V = 524288: the 64 chunks the finish passes support
    d = ragged(20, [2, 3], 524288, synth.BF16, sigma=0.3)
    check(d, "V=524288 bf16")


def test_row_ids_make_packing_irrelevant():
    d = ragged(17, [4, 4, 4, 4], 6000, synth.BF16)
    ids = np.array([7, 1000003, 5, 2 ** 31 + 9], dtype=np.uint32)
    gpu, ref, _ = check(d, "row ids", row_ids=ids, seed=99, step=12345678901)
    # the last row alone, with its id, gives the same outputs
    b = 3
    o0, o1 = d["offsets"][b], d["offsets"][b + 1]
    solo = dict(d, B=1, target=d["target"][o0 + b:o1 + b + 1], draft=d["draft"][o0:o1],
                offsets=np.array([0, o1 - o0], dtype=np.int32), tokens=d["tokens"][o0:o1],
                temp_target=d["temp_target"][b:b + 1], temp_draft=d["temp_draft"][b:b + 1])
    g2 = run_linear(solo, row_ids=ids[b:b + 1], seed=99, step=12345678901)
    assert g2["num_accepted"][0] == gpu["num_accepted"][b]
    assert np.array_equal(g2["out_tokens"], gpu["out_tokens"][o0 + b:o1 + b + 1])


def test_deterministic_repeat():
    d = synth.linear_v32k(B=8)
    a = run_linear(d)
    b = run_linear(d)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_v128k_full():
    d = synth.linear_v128k()
    gpu, ref, s = check(d, "v128k bf16 (greedy rows included)")
    assert s["max_rel_p"] < 1e-5


def test_bimodal_v152k_full():
    d = synth.bimodal_v152k()
    gpu, ref, s = check(d, "bimodal v152k ragged")
    n = gpu["num_accepted"]
    g = d["gammas"]
    say("[linear] bimodal accepted/drafted: low-sigma %.3f high-sigma %.3f" % (
        n[d["sigma"] < 1].sum() / g[d["sigma"] < 1].sum(), n[d["sigma"] > 1].sum() / g[d["sigma"] > 1].sum()))


def test_v8_distribution_million_trials():
    torch = torch_mod()
    n = 1_000_000
    d = synth.mc_v8(n)
    gpu = run_linear(d)
    first = gpu["out_tokens"][0::2]        # slot 1 of every trial: the first emitted token
    # token-for-token against the oracle on the first trials
    k = 20000
    sub = dict(d, B=k, target=d["target"][:2 * k], draft=d["draft"][:k], offsets=d["offsets"][:k + 1],
               tokens=d["tokens"][:k], temp_target=d["temp_target"][:k], temp_draft=d["temp_draft"][:k])
    ref = run_oracle_linear(sub)
    s = compare_linear({kk: (v[:k] if kk in ("num_accepted", "row_status", "p_at_draft", "q_at_draft")
                             else v[:2 * k]) for kk, v in gpu.items()}, ref, sub)
    say("[linear] v8 subset parity %s" % s)
    # law of the first emitted token against softmax(target row 0)
    p = scipy.special.softmax(d["x0"].astype(np.float64))
    counts = np.bincount(first, minlength=8)
    expect = p * n
    chi2 = float(((counts - expect) ** 2 / expect).sum())
    pval = scipy.stats.chi2.sf(chi2, 7)
    f = counts / n
    sigma = np.sqrt(p * (1 - p) / n)
    say("[linear] v8 chi2=%.2f p=%.3g max|f-p|/sigma=%.2f" % (chi2, pval, np.max(np.abs(f - p) / sigma)))
    assert pval > 1e-3
    assert np.all(np.abs(f - p) < 5 * sigma)
