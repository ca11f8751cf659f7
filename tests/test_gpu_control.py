"""GPU parity of the drafting and control helpers against the oracle.

* spec_verify_gamma_update: histories, next gammas and offsets bit-exact,
  batches wider than one work item, temperature coupling, and a short
  closed loop (draft with the controller's gammas, verify on the GPU,
  update on the GPU) checked round by round;
* spec_verify_draft_topk: tokens exact (ties to the lower id), log-
  probabilities within 1e-5, bf16 and fp32, k = 1..64, V up to 152064,
  greedy rows;
* spec_verify_tree_prune: kept trees exact on full 4-wide, 4-deep forests
  from the GPU's own top-k, budgets from 1 to beyond the forest, ragged
  candidate counts and malformed forests.
"""

import numpy as np
import pytest

import oracle
from oracle import control as OC, draft as OD
import synth
from gpu_util import f32, i32, logits_to_dev, run_linear, say, torch_mod

pytestmark = pytest.mark.gpu


def test_gamma_update_matches_oracle():
    import rejection_sampling_verify_04_amd as sv
    torch = torch_mod()
    rng = np.random.default_rng(100)
    B = 2500
    count = rng.integers(0, 17, size=B)
    hist = (rng.integers(0, 1 << 16, size=B) & ((1 << count) - 1)) | (count << 16)
    g = rng.choice([2, 4, 8], size=B)
    off = np.concatenate([[0], np.cumsum(g)]).astype(np.int32)
    n = np.array([rng.integers(-1, gi + 1) for gi in g], dtype=np.int32)
    temp = rng.choice([0.5, 0.8, 0.9, 1.2], size=B).astype(np.float32)
    for couple in (False, True):
        h_dev = torch.from_numpy(hist.astype(np.int32)).cuda()
        gn, on = sv.gamma_update(h_dev, i32(n), i32(off), temp_target=f32(temp),
                                 couple_temperature=couple)
        h_ref, g_ref, o_ref = OC.gamma_update(hist, n, g, temp, couple)
        assert np.array_equal(h_dev.cpu().numpy(), h_ref)
        assert np.array_equal(gn.cpu().numpy(), g_ref)
        assert np.array_equal(on.cpu().numpy(), o_ref)
    say("[control] gamma update: B=%d ok, gamma histogram %s" % (B, np.bincount(g_ref).tolist()))


def test_gamma_update_long_rounds():
    """Counts of 15..40 and a huge count: only the newest 16 outcomes are kept."""
    import rejection_sampling_verify_04_amd as sv
    torch = torch_mod()
    rng = np.random.default_rng(101)
    B = 300
    count = rng.integers(0, 17, size=B)
    hist = (rng.integers(0, 1 << 16, size=B) & ((1 << count) - 1)) | (count << 16)
    g = rng.integers(14, 42, size=B)
    n = np.array([rng.integers(13, gi + 1) for gi in g], dtype=np.int32)
    off = np.concatenate([[0], np.cumsum(g)]).astype(np.int32)
    h_dev = torch.from_numpy(hist.astype(np.int32)).cuda()
    gn, on = sv.gamma_update(h_dev, i32(n), i32(off))
    h_ref, g_ref, o_ref = OC.gamma_update(hist, n, g)
    assert np.array_equal(h_dev.cpu().numpy(), h_ref)
    assert np.array_equal(gn.cpu().numpy(), g_ref)
    assert np.array_equal(on.cpu().numpy(), o_ref)
    # a count of 2^31 - 1 (a corrupt input) pushes sixteen ones, in bounded time
    big = np.array([2 ** 31 - 1, 2 ** 31 - 1], dtype=np.int32)
    h_dev = torch.from_numpy(np.array([0, (3 << 16) | 0b101], dtype=np.int32)).cuda()
    gn, _ = sv.gamma_update(h_dev, i32(big), i32([0, 8, 16]))
    assert list(h_dev.cpu().numpy()) == [(16 << 16) | 0xFFFF] * 2
    assert list(gn.cpu().numpy()) == [8, 8]
    say("[control] gamma update, long rounds: ok")


def test_gamma_closed_loop():
    """Five rounds: draft with the controller's gammas, verify and update on the GPU."""
    import rejection_sampling_verify_04_amd as sv
    torch = torch_mod()
    rng = np.random.default_rng(101)
    B, V = 64, 512
    sigma = np.where(np.arange(B) % 2 == 0, 3.0, 0.3)
    h_dev = torch.zeros(B, dtype=torch.int32, device="cuda")
    h_ref = np.zeros(B, dtype=np.int64)
    gam = np.full(B, 4)
    T = np.ones(B, dtype=np.float32)
    for rnd in range(5):
        d = synth._linear_batch(rng, gam, V, 3.0, sigma, T, T.copy(), synth.BF16)
        gv = run_linear(d, step=rnd)
        gn, on = sv.gamma_update(h_dev, i32(gv["num_accepted"]), i32(d["offsets"]))
        h_ref, g_ref, o_ref = OC.gamma_update(h_ref, gv["num_accepted"], gam)
        assert np.array_equal(h_dev.cpu().numpy(), h_ref)
        assert np.array_equal(gn.cpu().numpy(), g_ref)
        gam = g_ref
    low = gam[sigma > 1].mean()
    high = gam[sigma < 1].mean()
    say("[control] closed loop: mean gamma sigma=3.0 rows %.2f, sigma=0.3 rows %.2f" % (low, high))
    assert high > low


@pytest.mark.parametrize("dtype,V,R,k", [(1, 1000, 40, 16), (1, 32000, 16, 4), (0, 5000, 8, 64),
                                         (1, 152064, 3, 8), (0, 777, 5, 1)])
def test_draft_topk_matches_oracle(dtype, V, R, k):
    import rejection_sampling_verify_04_amd as sv
    rng = np.random.default_rng(102 + V)
    x = rng.normal(0, 2, size=(R, V)).astype(np.float32)
    x[:, rng.integers(0, V, size=V // 10)] = x[:, :1]          # ties
    if dtype == 1:
        bits = synth.bf16_bits(x)
        vals = synth.bf16_values(bits).astype(np.float64)
        dev = logits_to_dev(bits, 1)
    else:
        vals = x.astype(np.float64)
        dev = logits_to_dev(x, 0)
    T = rng.choice([1.0, 0.7, 0.0], size=R).astype(np.float32)
    tok, lp = sv.draft_topk(dev, k, temp=f32(T))
    tok, lp = tok.cpu().numpy(), lp.cpu().numpy()
    for r in range(R):
        rt, rl = OD.topk_candidates(vals[r], k, float(T[r]))
        assert np.array_equal(tok[r], rt), (r, tok[r], rt)
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(lp[r]), fin)
        assert np.all(np.abs(lp[r][fin] - rl[fin]) <= 1e-5 * np.maximum(1.0, np.abs(rl[fin])))
    say("[control] draft top-k dtype=%d V=%d R=%d k=%d ok" % (dtype, V, R, k))


@pytest.mark.parametrize("V", [8, 1000, 8192, 32000, 32768])
def test_draft_topk_small_k_path(V):
    """k <= 4 over aligned bf16 rows of up to 32768 logits (one 256-thread work
    item per row): every k, greedy, sampled and invalid temperatures, ties at
    the k-th place, -inf logits, signed zeros, and more than 1024 logits tied
    at the top (the argmax rounds)."""
    import rejection_sampling_verify_04_amd as sv
    rng = np.random.default_rng(106 + V)
    R = 24
    x = rng.normal(0, 2, size=(R, V)).astype(np.float32)
    x[1, :] = 0.25                                           # all equal
    x[2, rng.choice(V, min(V, 1500), replace=False)] = 7.0   # many maxima (> 1024 when V allows)
    x[3, :] = -np.inf
    x[3, rng.choice(V, 3, replace=False)] = [1.0, 2.0, 1.0]  # three finite logits
    x[4, : min(V, 6)] = 9.0                                  # ties at the top, in index order
    zeros = rng.choice(V, min(V, 40), replace=False)
    x[5, zeros] = np.where(rng.random(len(zeros)) < 0.5, np.float32(-0.0), np.float32(0.0))
    x[5, np.setdiff1d(np.arange(V), zeros)] = -1.0           # signed zeros on top
    x[6] = np.round(x[6] * 2) / 2                            # coarse values: ties everywhere
    bits = synth.bf16_bits(x)
    vals = synth.bf16_values(bits).astype(np.float64)
    T = rng.choice([1.0, 0.7, 1.3, 0.0], size=R).astype(np.float32)
    T[7] = np.nan                                            # invalid: tokens -1, NaN log-probs
    T[8] = -1.0
    for k in (1, 2, 3, 4):
        tok, lp = sv.draft_topk(logits_to_dev(bits, 1), k, temp=f32(T))
        tok, lp = tok.cpu().numpy(), lp.cpu().numpy()
        for r in range(R):
            if r in (7, 8):
                assert np.all(tok[r] == -1) and np.all(np.isnan(lp[r])), (k, r)
                continue
            rt, rl = OD.topk_candidates(vals[r], k, float(T[r]))
            assert np.array_equal(tok[r], rt), (V, k, r, tok[r], rt)
            fin = np.isfinite(rl)
            assert np.array_equal(np.isfinite(lp[r]), fin), (V, k, r, lp[r], rl)
            assert np.all(np.abs(lp[r][fin] - rl[fin]) <= 1e-5 * np.maximum(1.0, np.abs(rl[fin])))
    say("[control] draft top-k, small-k path V=%d ok" % V)


def test_draft_topk_small_k_ties_within_one_wave():
    """The small-k path bounds each wave's candidates by its own k-th largest
    thread maximum and ranks all waves' candidates in one wave.  Ties at the
    top placed inside one wave's logits (logit i belongs to wave
    ((i / 8) mod 256) / 64): 16 (one ranking round per lane), 17 and 100
    (more than one candidate per ranking lane), 300 (more than one wave's
    256 slots: the whole-row rounds), ties split across two waves, and a
    lower tie value in another wave."""
    import rejection_sampling_verify_04_amd as sv
    rng = np.random.default_rng(107)
    R, V = 8, 32000
    x = rng.normal(0, 2, size=(R, V)).astype(np.float32)
    wave_of = ((np.arange(V) // 8) % 256) // 64

    def put(r, w, n, val):
        pos = rng.choice(np.flatnonzero(wave_of == w), n, replace=False)
        x[r, pos] = val

    put(0, 0, 16, 9.0)
    put(1, 1, 17, 9.0)
    put(2, 2, 100, 9.0)
    put(3, 3, 300, 9.0)
    put(4, 0, 10, 9.0)
    put(4, 3, 10, 9.0)
    put(5, 1, 3, 9.5)
    put(5, 2, 40, 9.0)
    put(6, 2, 2, 9.0)
    put(6, 0, 2, 9.0)
    bits = synth.bf16_bits(x)
    vals = synth.bf16_values(bits).astype(np.float64)
    T = np.array([1.0, 0.7, 0.0, 1.0, 1.3, 1.0, 0.0, 1.0], dtype=np.float32)
    for k in (1, 2, 3, 4):
        tok, lp = sv.draft_topk(logits_to_dev(bits, 1), k, temp=f32(T))
        tok, lp = tok.cpu().numpy(), lp.cpu().numpy()
        for r in range(R):
            rt, rl = OD.topk_candidates(vals[r], k, float(T[r]))
            assert np.array_equal(tok[r], rt), (k, r, tok[r], rt)
            fin = np.isfinite(rl)
            assert np.array_equal(np.isfinite(lp[r]), fin), (k, r, lp[r], rl)
            assert np.all(np.abs(lp[r][fin] - rl[fin]) <= 1e-5 * np.maximum(1.0, np.abs(rl[fin])))
    say("[control] draft top-k, ties within one wave ok")


def test_draft_topk_heavy_ties():
    """Rows whose top values repeat far more often than k (the whole-row path)."""
    import rejection_sampling_verify_04_amd as sv
    rng = np.random.default_rng(104)
    R, V, k = 6, 20000, 8
    x = rng.normal(0, 1, size=(R, V)).astype(np.float32)
    x[0] = 0.5                                  # every logit equal
    x[1, rng.choice(V, 3000, replace=False)] = 9.0   # 3000 copies of the maximum
    x[2, :] = -np.inf
    x[2, 5] = 1.0                               # one finite logit among -inf
    bits = synth.bf16_bits(x)
    vals = synth.bf16_values(bits).astype(np.float64)
    tok, lp = sv.draft_topk(logits_to_dev(bits, 1), k)
    tok, lp = tok.cpu().numpy(), lp.cpu().numpy()
    for r in range(R):
        rt, rl = OD.topk_candidates(vals[r], k, 1.0)
        assert np.array_equal(tok[r], rt), (r, tok[r], rt)
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(lp[r]), fin)
        assert np.all(np.abs(lp[r][fin] - rl[fin]) <= 1e-5 * np.maximum(1.0, np.abs(rl[fin])))
    say("[control] draft top-k with heavy ties ok")


def test_draft_topk_signed_zero_ties():
    """-0 and +0 are equal logits: ties between them go to the lower id, in
    the direct path (a few zeros at the top) and in the whole-row path (more
    zeros at the top than candidates are ranked directly)."""
    import rejection_sampling_verify_04_amd as sv
    rng = np.random.default_rng(105)
    R, V, k = 4, 32000, 8
    x = -np.abs(rng.normal(1, 1, size=(R, V))).astype(np.float32) - 0.5
    for r, n in enumerate([5, 12, 3000, 20000]):
        pos = rng.choice(V, n, replace=False)
        x[r, pos] = np.where(rng.random(n) < 0.5, np.float32(-0.0), np.float32(0.0))
    for dt in (1, 0):
        if dt == 1:
            bits = synth.bf16_bits(x)
            vals = synth.bf16_values(bits).astype(np.float64)
            dev = logits_to_dev(bits, 1)
        else:
            vals = x.astype(np.float64)
            dev = logits_to_dev(x, 0)
        tok, lp = sv.draft_topk(dev, k)
        tok, lp = tok.cpu().numpy(), lp.cpu().numpy()
        for r in range(R):
            rt, rl = OD.topk_candidates(vals[r], k, 1.0)
            assert np.array_equal(tok[r], rt), (dt, r, tok[r], rt)
            assert np.all(np.abs(lp[r] - rl) <= 1e-5 * np.maximum(1.0, np.abs(rl)))
    say("[control] draft top-k signed-zero ties ok")


def gpu_forest(rng, V, width, depth, B):
    """Full forests from the GPU's own top-k of random draft rows."""
    import rejection_sampling_verify_04_amd as sv
    par, tok, lq = [], [], []
    for b in range(B):
        p_b, t_b, l_b = [], [], []
        frontier = [-1]
        for _ in range(depth):
            rows = rng.normal(0, 2, size=(len(frontier), V)).astype(np.float32)
            t, l = sv.draft_topk(logits_to_dev(rows, 0), width)
            t, l = t.cpu().numpy(), l.cpu().numpy()
            nxt = []
            for j, p in enumerate(frontier):
                for c in range(width):
                    p_b.append(p)
                    t_b.append(int(t[j, c]))
                    l_b.append(float(l[j, c]))
                    nxt.append(len(p_b) - 1)
            frontier = nxt
        par.append(p_b)
        tok.append(t_b)
        lq.append(l_b)
    return (np.array(par, dtype=np.int32), np.array(tok, dtype=np.int32),
            np.array(lq, dtype=np.float32))


def test_tree_prune_matches_oracle():
    import rejection_sampling_verify_04_amd as sv
    rng = np.random.default_rng(103)
    B = 6
    par, tok, lq = gpu_forest(rng, 300, 4, 4, B)
    C = par.shape[1]
    n_cand = np.array([C, C, 200, 84, 20, 4], dtype=np.int32)
    for n_max in (1, 16, 64):
        out = sv.tree_prune(i32(par), i32(tok), f32(lq), n_max, tau=0.01, n_cand=i32(n_cand))
        got = {k: v.cpu().numpy() for k, v in out.items()}
        for b in range(B):
            c = int(n_cand[b])
            rp, rt, rc, rpass = OD.prune_tree(par[b, :c], tok[b, :c], lq[b, :c].astype(np.float64),
                                              n_max, 0.01)
            n = len(rp)
            assert got["n_nodes"][b] == n
            assert np.array_equal(got["parents"][b, :n], rp)
            assert np.array_equal(got["tokens"][b, :n], rt)
            assert np.array_equal(got["cum_logprob"][b, :n], rc.astype(np.float32))
            assert got["n_pass"][b] == rpass
            assert np.all(got["parents"][b, n:] == -1)
        say("[control] prune n_max=%d ok: nodes %s" % (n_max, got["n_nodes"].tolist()))
    bad = par.copy()
    bad[2, 10] = 50                     # a parent after its child
    out = sv.tree_prune(i32(bad), i32(tok), f32(lq), 64)
    assert out["n_nodes"].cpu().numpy()[2] == 0


def test_tree_prune_ties_at_limit():
    """1024 candidates (the limit: one thread group counts each), and forests
    of 40 and 130 (several groups share each count), whose log q come from
    three values, so that exact ties in the cumulative log-probability are
    common and the tie order (depth, parent, rank) decides the kept set."""
    import rejection_sampling_verify_04_amd as sv
    rng = np.random.default_rng(107)
    C = 1024
    par = np.array([-1] * 4 + [(i - 4) // 4 for i in range(4, C)], dtype=np.int32)
    B = 3
    pars = np.tile(par, (B, 1))
    tok = rng.integers(0, 32000, size=(B, C)).astype(np.int32)
    lq = rng.choice(np.array([-0.5, -1.0, -1.5], dtype=np.float32), size=(B, C))
    n_cand = np.array([C, 40, 130], dtype=np.int32)
    for n_max in (8, 33, 64):
        out = sv.tree_prune(i32(pars), i32(tok), f32(lq), n_max, tau=0.2, n_cand=i32(n_cand))
        got = {k: v.cpu().numpy() for k, v in out.items()}
        for b in range(B):
            c = int(n_cand[b])
            rp, rt, rc, rpass = OD.prune_tree(pars[b, :c], tok[b, :c], lq[b, :c].astype(np.float64),
                                              n_max, 0.2)
            n = len(rp)
            assert got["n_nodes"][b] == n, (n_max, b)
            assert np.array_equal(got["parents"][b, :n], rp), (n_max, b)
            assert np.array_equal(got["tokens"][b, :n], rt), (n_max, b)
            assert np.array_equal(got["cum_logprob"][b, :n], rc.astype(np.float32)), (n_max, b)
            assert got["n_pass"][b] == rpass, (n_max, b)
    say("[control] prune with ties at 1024, 40 and 130 candidates ok")


def test_drafting_full_size_sampled():
    """The drafting workloads at their full size and launch shape: top-4 of
    1024 draft rows over V=32000 bf16 (every 32nd row checked), then the
    pruning of 64 full 4-wide, 4-deep forests (340 candidates, log q from the
    library's own top-4 of random rows) to 64 nodes (every tree checked)."""
    import rejection_sampling_verify_04_amd as sv
    torch = torch_mod()
    rng = np.random.default_rng(11)
    R, V, k = 1024, 32000, 4
    bits = synth.bf16_bits(rng.standard_normal((R, V), dtype=np.float32) * np.float32(2.0))
    tok, lp = sv.draft_topk(logits_to_dev(bits, 1), k)
    tok, lp = tok.cpu().numpy(), lp.cpu().numpy()
    vals = synth.bf16_values(bits[::32]).astype(np.float64)
    for i, r in enumerate(range(0, R, 32)):
        rt, rl = OD.topk_candidates(vals[i], k, 1.0)
        assert np.array_equal(tok[r], rt), (r, tok[r], rt)
        assert np.all(np.abs(lp[r] - rl) <= 1e-5 * np.maximum(1.0, np.abs(rl))), r
    say("[control] draft top-k full size: 32 of 1024 rows checked")
    Bp, C, n_max = 64, 340, 64
    par = np.zeros((Bp, C), dtype=np.int32)
    lvl = [list(range(0, 4)), list(range(4, 20)), list(range(20, 84)), list(range(84, 340))]
    for d in range(4):
        for j, c in enumerate(lvl[d]):
            par[:, c] = -1 if d == 0 else lvl[d - 1][j // 4]
    cl = torch.from_numpy(rng.standard_normal((Bp * 85, V // 8), dtype=np.float32)).cuda()
    ct, clq = sv.draft_topk(cl, 4)
    ctok = ct.reshape(Bp, C).contiguous()
    clog = clq.reshape(Bp, C).contiguous()
    out = sv.tree_prune(i32(par), ctok, clog, n_max, tau=0.1)
    got = {kk: v.cpu().numpy() for kk, v in out.items()}
    tk, lq = ctok.cpu().numpy(), clog.cpu().numpy()
    for b in range(Bp):
        rp, rtk, rc, rpass = OD.prune_tree(par[b], tk[b], lq[b].astype(np.float64), n_max, 0.1)
        n = len(rp)
        assert got["n_nodes"][b] == n == n_max
        assert np.array_equal(got["parents"][b, :n], rp), b
        assert np.array_equal(got["tokens"][b, :n], rtk), b
        assert np.array_equal(got["cum_logprob"][b, :n], rc.astype(np.float32)), b
        assert got["n_pass"][b] == rpass, b
    say("[control] tree prune full size: 64 forests of 340 candidates -> 64 nodes")
