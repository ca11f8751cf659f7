"""HIP-graph replay of a whole drafting and verify round equals eager execution.

One captured graph holds draft top-k, tree pruning, a SAMPLED_WOR tree verify,
the KV-cache commit of its accepted paths, the dynamic-gamma update and the
tree telemetry, as the benchmark replays them.  The graph is replayed several
times; before each replay the state the round updates in place (KV cache,
gamma histories, telemetry counters) is restored eagerly, and unrelated eager
verify calls on the same workspace run between replays.  Every replay must
give the eager results bit for bit.
"""

import numpy as np
import pytest

import synth
from gpu_util import f32, i32, logits_to_dev, say, torch_mod

pytestmark = pytest.mark.gpu


def forest(rng, B, width=4, depth=3, V=32000):
    """Full candidate forests in breadth-first order (roots' parent -1)."""
    par, tok, lq = [], [], []
    for _ in range(B):
        p_b, frontier = [], [-1]
        for _ in range(depth):
            nxt = []
            for p in frontier:
                for _ in range(width):
                    p_b.append(p)
                    nxt.append(len(p_b) - 1)
            frontier = nxt
        par.append(p_b)
        tok.append(rng.integers(0, V, size=len(p_b)))
        lq.append(-rng.exponential(1.0, size=len(p_b)))
    return (np.array(par, dtype=np.int32), np.array(tok, dtype=np.int32),
            np.array(lq, dtype=np.float32))


def test_graph_round_replays_match_eager():
    torch = torch_mod()
    import rejection_sampling_verify_04_amd as sv
    rng = np.random.default_rng(130)

    # drafting inputs: top-k rows and candidate forests
    R, Vd = 64, 32000
    rows = synth.bf16_bits(rng.normal(0, 2, size=(R, Vd)).astype(np.float32))
    rows_dev = logits_to_dev(rows, 1)
    temps = f32(rng.choice([1.0, 0.7, 0.0], size=R).astype(np.float32))
    B = 8
    cpar, ctok, clq = forest(rng, B)
    cpar_d, ctok_d, clq_d = i32(cpar), i32(ctok), f32(clq)

    # the verify: SAMPLED_WOR trees of 21 nodes over V=20000 bf16
    t = synth.tree_wor(seed=131, B=B, N=21, V=20000, draft_sd=5.0, pert=1.0)
    N = t["N"]
    wor_args = (logits_to_dev(t["target"], 1), i32(t["parents"]), i32(t["tokens"]),
                f32(t["temp_target"]))
    wor_kw = dict(cand_mode=sv.SV_TREE_SAMPLED_WOR, draft_logits=logits_to_dev(t["draft"], 1),
                  temp_draft=f32(t["temp_draft"]), seed=5, step=2)
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")

    # state the round updates in place, with pristine copies
    H, d, layers = 4, 128, 2
    L0 = rng.integers(0, 40, size=B).astype(np.int32)
    S = int(L0.max()) + N + 3
    def cache():   # finite bf16 values (bitwise comparison needs no NaN)
        bits = synth.bf16_bits(rng.normal(0, 1, size=(layers, B, H, S, d)).astype(np.float32))
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    kc0, vc0 = cache(), cache()
    kc, vc = kc0.clone(), vc0.clone()
    pl = i32(L0)
    count = rng.integers(0, 17, size=B)
    hist0 = i32(((rng.integers(0, 1 << 16, size=B) & ((1 << count) - 1)) | (count << 16))
                .astype(np.int32))
    hist = hist0.clone()
    gam = rng.choice([2, 4, 8], size=B)
    off = i32(np.concatenate([[0], np.cumsum(gam)]).astype(np.int32))
    n_lin = i32(np.array([rng.integers(-1, g + 1) for g in gam], dtype=np.int32))
    tel = sv.telemetry_block()

    def round_(out):
        tk, tl = sv.draft_topk(rows_dev, 4, temp=temps)
        pr = sv.tree_prune(cpar_d, ctok_d, clq_d, 64, tau=0.05)
        v = sv.verify_tree(*wor_args, workspace=ws, outputs=out["verify"], **wor_kw)
        nl = sv.kv_commit(kc, vc, pl, v["num_accepted"], path_nodes=v["path_nodes"])
        gn, on = sv.gamma_update(hist, n_lin, off)
        sv.telemetry_tree(v["num_accepted"], v["path_nodes"], wor_args[1], tel)
        return dict(topk_tokens=tk, topk_logprob=tl, new_len=nl, gamma=gn, offsets=on, **pr)

    def restore():
        kc.copy_(kc0)
        vc.copy_(vc0)
        hist.copy_(hist0)
        tel.zero_()

    def snapshot(res, out):
        got = {k: v.clone() for k, v in res.items()}
        got.update({"verify_" + k: v.clone() for k, v in out["verify"].items()})
        got.update(k_cache=kc.clone(), v_cache=vc.clone(), history=hist.clone(),
                   telemetry=tel.clone())
        return got

    def verify_outputs():
        return dict(num_accepted=torch.empty(B, dtype=torch.int32, device="cuda"),
                    path_nodes=torch.empty((B, N - 1), dtype=torch.int32, device="cuda"),
                    out_tokens=torch.empty((B, N), dtype=torch.int32, device="cuda"),
                    row_status=torch.empty(B, dtype=torch.int32, device="cuda"),
                    p_at_node=torch.empty((B, N), dtype=torch.float32, device="cuda"))

    eager_out = dict(verify=verify_outputs())
    restore()
    torch.cuda.synchronize()
    eager = snapshot(round_(eager_out), eager_out)
    torch.cuda.synchronize()
    assert int(eager["verify_num_accepted"].max()) >= 1   # paths that move KV rows

    graph_out = dict(verify=verify_outputs())
    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graph_res = round_(graph_out)

    other = synth.linear_v32k(seed=132, B=8)
    other_args = (logits_to_dev(other["target"], 1), logits_to_dev(other["draft"], 1),
                  i32(other["offsets"]), i32(other["tokens"]), f32(other["temp_target"]),
                  f32(other["temp_draft"]))
    for rep in range(4):
        restore()
        for v in list(graph_res.values()) + list(graph_out["verify"].values()):
            v.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot(graph_res, graph_out)
        for k in eager:
            assert torch.equal(got[k], eager[k]), (rep, k)
        sv.verify_linear(*other_args, seed=rep, workspace=ws)   # eager work in between
        torch.cuda.synchronize()
    say("[graph] round of top-k, prune, SAMPLED_WOR verify, KV commit, gamma update and "
        "telemetry: 4 replays equal to eager")
