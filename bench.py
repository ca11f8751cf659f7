#!/usr/bin/env python3
"""Benchmark of the speculative-decoding verify step on one MI355X.

A step is one call of the verify hot path on one batch of synthetic input
that is already resident in device memory.  The default workload is the
largest verify configuration that one GPU holds: the bimodal-acceptance batch,
B=256 ragged rows over V=152064 bf16 with gamma in {2, 4, 8} from a 16-step
acceptance history (about 1124 draft positions and 765 MB of logits per step).
Other workloads (--workload) measure the remaining configurations.

Timing: W untimed warm-up steps, then K timed steps bracketed by
torch.cuda.synchronize(); the K steps are captured as one HIP graph and
replayed, so host launch overhead does not pace the GPU.  Before the timed
replay the graph is replayed untimed until the GPU has been busy for 0.25 s,
so that its clocks have settled (the first replays of a cold GPU run up to
20% slower).  The dominant kernel's duration comes from the same K steps run
right after, each with a pair of HIP events attached to that kernel's
dispatch on the call's own stream (the library's one-shot timing hook).
Inputs rotate over enough copies to exceed the 256 MB Infinity Cache, so
the logits come from HBM.

Prints one JSON line.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("verified draft positions/sec + achieved HBM GB/s (% of peak), "
          "B×γ×V verify")
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="bimodal_v152k",
                    choices=["linear_v1000", "linear_v32k", "linear_v128k", "bimodal_v152k",
                             "tree_v32k", "tree_wor_v32k", "attn_tree", "kv_commit",
                             "draft_topk", "tree_prune", "telemetry", "telemetry_tree",
                             "gamma_update"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the timed steps eagerly instead of replaying one HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--settle-seconds", type=float, default=0.25,
                    help="untimed work before the timed steps, so that the GPU clocks settle "
                         "(0 for counter runs, which need few dispatches)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="per-launch HBM bytes measured with rocprofv3 counters")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run device-to-device copies of this many MiB (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def calibrate_copy(mib, steps):
    """Plain device copies of a known size, for scaling HBM byte counters."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps(dict(calibration="copy", bytes_read=n, bytes_written=n, copies=steps)),
          flush=True)


def copies_for(nbytes):
    return max(1, min(64, -(-2 * MALL_BYTES // max(nbytes, 1))))


def to_dev_logits(torch, arr, dtype_code):
    if dtype_code == 1:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def cpu_baseline_linear(d, seconds):
    """The oracle on a bounded sample of the same workload: whole batch rows until ~seconds."""
    import oracle
    off = d["offsets"]
    B = len(off) - 1
    done_pos = 0
    rows = 0
    t0 = time.perf_counter()
    b = 0
    while time.perf_counter() - t0 < seconds:
        bb = b % B
        o0, o1 = int(off[bb]), int(off[bb + 1])
        t = o0 + bb
        oracle.verify_linear(d["target"][t:t + o1 - o0 + 1], d["draft"][o0:o1], d["dtype"],
                             np.array([0, o1 - o0]), d["tokens"][o0:o1],
                             d["temp_target"][bb:bb + 1], d["temp_draft"][bb:bb + 1],
                             seed=0, step=0, row_ids=np.array([bb]))
        done_pos += o1 - o0
        rows += 1
        b += 1
    dt = time.perf_counter() - t0
    es = 2 if d["dtype"] == 1 else 4
    V = d["target"].shape[1] if d["target"].ndim == 2 else d["V"]
    total = int(off[-1])
    # the logit rows of the sampled batch rows, each read once: 2 gamma_b + 1 per row
    sample_bytes = (2 * done_pos + rows) * V * es
    return dict(value=done_pos / dt, unit="verified draft positions/s", cores=1, kind="oracle",
                us_per_call=dt / done_pos * total * 1e6,
                logit_gb_per_s=sample_bytes / dt / 1e9,
                sample="%d batch rows (%d draft positions) of the same workload in %.1f s, "
                       "single-threaded NumPy float64; us_per_call scales the sample to the "
                       "whole batch" % (rows, done_pos, dt))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


_POOL_DATA = None


def _oracle_batch_row(d, bb):
    """One batch row of the workload through the oracle; returns its draft positions / nodes."""
    import oracle
    if d["kind"] == "linear":
        off = d["offsets"]
        o0, o1 = int(off[bb]), int(off[bb + 1])
        t = o0 + bb
        oracle.verify_linear(d["target"][t:t + o1 - o0 + 1], d["draft"][o0:o1], d["dtype"],
                             np.array([0, o1 - o0]), d["tokens"][o0:o1],
                             d["temp_target"][bb:bb + 1], d["temp_draft"][bb:bb + 1],
                             seed=0, step=0, row_ids=np.array([bb]))
        return o1 - o0
    if d["kind"] == "tree_wor":
        oracle.verify_tree_sampled_wor(d["target"][bb:bb + 1], d["draft"][bb:bb + 1], d["dtype"],
                                       d["parents"][bb:bb + 1], d["tokens"][bb:bb + 1],
                                       d["n_nodes"][bb:bb + 1], d["temp_target"][bb:bb + 1],
                                       d["temp_draft"][bb:bb + 1], row_ids=np.array([bb]))
    else:
        oracle.verify_tree_topk(d["target"][bb:bb + 1], d["dtype"], d["parents"][bb:bb + 1],
                                d["tokens"][bb:bb + 1], d["n_nodes"][bb:bb + 1],
                                d["temp_target"][bb:bb + 1], row_ids=np.array([bb]))
    return int(d["n_nodes"][bb]) - 1


def _pool_worker(arg):
    w, n, deadline = arg
    d = _POOL_DATA
    B = len(d["offsets"]) - 1 if d["kind"] == "linear" else d["B"]
    units = rows = 0
    b = w
    while time.monotonic() < deadline:
        units += _oracle_batch_row(d, b % B)
        rows += 1
        b += n
    return units, rows


def host_cores():
    """Cores this process may run on, the machine's count, and the CPU model."""
    return dict(affinity=len(os.sched_getaffinity(0)), machine=os.cpu_count(), model=cpu_model())


# One GPU's share of its host's CPUs: worker pools stay within it whatever
# larger count the machine reports.
HOST_SHARE = 16


def cpu_baseline_pool(d, seconds):
    """The oracle over the host cores: one process per core (at most the 16-core
    share of one GPU), forked before the GPU is touched, worker w taking batch
    rows w, w + n, ... for ~seconds.  (A thread pool gains nothing: the oracle's
    per-position work is Python that holds the interpreter lock.)"""
    import multiprocessing
    global _POOL_DATA
    hc = host_cores()
    n = min(HOST_SHARE, hc["affinity"])
    _POOL_DATA = d
    ctx = multiprocessing.get_context("fork")
    t0 = time.monotonic()
    with ctx.Pool(n) as pool:
        res = pool.map(_pool_worker, [(w, n, t0 + seconds) for w in range(n)])
    dt = time.monotonic() - t0
    _POOL_DATA = None
    units = sum(r[0] for r in res)
    rows = sum(r[1] for r in res)
    linear = d["kind"] == "linear"
    return dict(value=units / dt, unit="verified draft positions/s" if linear else "verified draft nodes/s",
                cores=n, kind="oracle", host_cores=hc,
                sample="%d batch rows (%d %s) of the same workload in %.1f s, NumPy float64 in "
                       "%d processes (%s; %d cores in this process's affinity mask, %d on the "
                       "machine; the pool is capped at one GPU's %d-core share)"
                       % (rows, units, "draft positions" if linear else "draft nodes", dt, n,
                          hc["model"], hc["affinity"], hc["machine"] or 0, HOST_SHARE))


def cpu_baseline_tree(d, seconds):
    import oracle
    B = d["B"]
    t0 = time.perf_counter()
    rows = nodes = 0
    while time.perf_counter() - t0 < seconds:
        b = rows % B
        if d["kind"] == "tree_wor":
            oracle.verify_tree_sampled_wor(d["target"][b:b + 1], d["draft"][b:b + 1], d["dtype"],
                                           d["parents"][b:b + 1], d["tokens"][b:b + 1],
                                           d["n_nodes"][b:b + 1], d["temp_target"][b:b + 1],
                                           d["temp_draft"][b:b + 1], row_ids=np.array([b]))
        else:
            oracle.verify_tree_topk(d["target"][b:b + 1], d["dtype"], d["parents"][b:b + 1],
                                    d["tokens"][b:b + 1], d["n_nodes"][b:b + 1],
                                    d["temp_target"][b:b + 1], row_ids=np.array([b]))
        nodes += int(d["n_nodes"][b]) - 1
        rows += 1
    dt = time.perf_counter() - t0
    total = int(np.sum(d["n_nodes"])) - B
    return dict(value=nodes / dt, unit="verified draft nodes/s", cores=1, kind="oracle",
                us_per_call=dt / nodes * total * 1e6,
                sample="%d trees (%d draft nodes) of the same workload in %.1f s, "
                       "single-threaded NumPy float64 (it reads every node's rows); "
                       "us_per_call scales the sample to the whole batch" % (rows, nodes, dt))


def cpu_baseline_attn(q, k, v, L, parents, seconds):
    import oracle
    B, H, N, dd = q.shape
    t0 = time.perf_counter()
    heads = 0
    while time.perf_counter() - t0 < seconds and heads < B * H:
        b, h = divmod(heads, H)
        mask = oracle.ancestor_mask(parents[b], N)
        oracle.attention_head(oracle.bf16_bits_to_f64(q[b, h]), oracle.bf16_bits_to_f64(k[b, h]),
                              oracle.bf16_bits_to_f64(v[b, h]), int(L[b]), mask, dd ** -0.5)
        heads += 1
    dt = time.perf_counter() - t0
    threads = os.environ.get("OMP_NUM_THREADS")
    return dict(value=heads * N / dt, unit="verified query tokens/s",
                cores=int(threads) if threads else len(os.sched_getaffinity(0)), kind="oracle",
                sample="%d (b, h) heads of the same workload in %.1f s, NumPy float64 "
                       "(BLAS matmul threads)" % (heads, dt))


def cpu_baseline_kv(kc, vc, L0, n_acc, path, N, seconds):
    """The oracle's commit on a bounded sample: one (batch row, all heads, all layers) slice
    at a time, copied to the host first (copy time excluded)."""
    import oracle
    layers, B = kc.shape[0], kc.shape[1]
    ks = kc[:, :, :, L0:L0 + N].float().cpu().numpy()
    vs = vc[:, :, :, L0:L0 + N].float().cpu().numpy()
    t_total = 0.0
    rows = toks = 0
    while t_total < seconds:
        b = rows % B
        t0 = time.perf_counter()
        oracle.kv_commit(ks[:, b:b + 1], vs[:, b:b + 1], np.array([0]), n_acc[b:b + 1],
                         path[b:b + 1], N)
        t_total += time.perf_counter() - t0
        toks += max(int(n_acc[b]), 0)
        rows += 1
    return dict(value=toks / t_total, unit="committed tokens/s", cores=1, kind="oracle",
                sample="%d batch rows (%d committed tokens, %d layers) of the same workload, "
                       "the %d new slots of every head, in %.2f s of NumPy copying"
                       % (rows, toks, layers, N, t_total))


def cpu_baseline_topk(rows, k, seconds):
    import oracle
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        x = oracle.bf16_bits_to_f64(rows[n % rows.shape[0]])
        oracle.draft.topk_candidates(x, k, 1.0)
        n += 1
    dt = time.perf_counter() - t0
    return dict(value=n / dt, unit="draft rows/s", cores=1, kind="oracle",
                sample="%d rows of the same workload in %.1f s, single-threaded Python/NumPy"
                       % (n, dt))


def cpu_baseline_prune(par, tok, logq, n_max, seconds):
    import oracle
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        b = n % par.shape[0]
        oracle.draft.prune_tree(par[b], tok[b], logq[b].astype(np.float64), n_max)
        n += 1
    dt = time.perf_counter() - t0
    return dict(value=n / dt, unit="pruned trees/s", cores=1, kind="oracle",
                sample="%d forests of the same workload in %.1f s, single-threaded Python"
                       % (n, dt))


def cpu_baseline_control(wl, na, off, seconds):
    """The oracle's telemetry counters (linear rows or trees) or gamma update over
    the same rows until ~seconds."""
    import oracle
    t0 = time.perf_counter()
    n = 0
    gam = np.diff(off) if wl == "gamma_update" else None
    hist = np.zeros(len(na), dtype=np.int64)
    while time.perf_counter() - t0 < seconds:
        if wl == "telemetry":
            oracle.telemetry.add_linear(oracle.telemetry.empty(), na, off)
        elif wl == "telemetry_tree":
            oracle.telemetry.add_tree(oracle.telemetry.empty(), na, off[0], off[1], None)
        else:
            hist, _, _ = oracle.control.gamma_update(hist, na, gam)
        n += len(na)
    dt = time.perf_counter() - t0
    unit = {"telemetry": "batch rows/s", "telemetry_tree": "trees/s"}.get(wl, "requests/s")
    return dict(value=n / dt, unit=unit, cores=1, kind="oracle",
                sample="%d %s (%d calls of %d) in %.1f s, single-threaded Python"
                       % (n, unit[:-2], n // len(na), len(na), dt))


def load_traffic(path, workload, kernel_sig):
    """HBM bytes per launch of the dominant kernel, from counter runs
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy of known size); None when
    absent or taken on a different build of the kernel."""
    try:
        with open(path) as f:
            t = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not t or t.get("kernel_source_sha1") != kernel_sig:
        return None
    return t.get("hbm_bytes_per_launch")


def dominant_kernel(wl):
    """The kernel whose duration the roofline reports: the vocabulary pass, which
    for linear calls of one round of (row, chunk) work items is its by-chunk form."""
    return {"attn_tree": "attn_kernel", "kv_commit": "kv_commit_kernel",
            "draft_topk": "draft_topk_small_kernel", "tree_prune": "tree_prune_kernel",
            "linear_v32k": "stats_kernel_by_chunk",
            "linear_v1000": "stats_kernel_by_chunk",
            "telemetry": "telemetry_linear_kernel",
            "telemetry_tree": "telemetry_tree_kernel",
            "gamma_update": "gamma_update_kernel"}.get(wl, "stats_kernel")


def kernel_source_sig(wl):
    """SHA-1 over the sources that the dominant kernel is compiled from (its
    own file and the headers that file includes)."""
    import hashlib
    csrc = os.path.join(ROOT, "rejection_sampling_verify_04_amd", "csrc")
    own = {"attn_tree": "sv_attn.hip", "kv_commit": "sv_kv.hip", "draft_topk": "sv_draft.hip",
           "tree_prune": "sv_draft.hip", "telemetry": "sv_telemetry.hip",
           "telemetry_tree": "sv_telemetry.hip",
           "gamma_update": "sv_control.hip"}.get(wl, "sv_stats.hip")
    names = [own, "sv_common.h", "sv_internal.h", "sv_pass.h"]
    h = hashlib.sha1()
    for name in names:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib, args.steps)
        return
    import torch
    import synth
    import rejection_sampling_verify_04_amd as sv

    wl = args.workload
    # The oracle over all host cores runs first: its worker processes are
    # forked before anything touches the GPU.
    early = None
    pool_baseline = None
    if wl in synth.WORKLOADS:
        early = synth.WORKLOADS[wl]()
        if not args.no_cpu_baseline:
            pool_baseline = cpu_baseline_pool(early, args.cpu_seconds)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    dev = torch.device("cuda", 0)

    if wl in ("draft_topk", "tree_prune"):
        # One level of tree drafting: top-4 candidates of 1024 draft rows
        # (64 trees x 16 frontier nodes) over V=32000 bf16; and the pruning of
        # 64 full 4-wide, 4-deep candidate forests (340 candidates) to 64 nodes.
        rng = np.random.default_rng(11)
        R, V, kk = 1024, 32000, 4
        rows = synth.bf16_bits(rng.standard_normal((R, V), dtype=np.float32) * np.float32(2.0))
        nrc = copies_for(R * V * 2)
        lsets = [to_dev_logits(torch, rows, 1) for _ in range(nrc)]
        Bp, C, n_max = 64, 340, 64
        par = np.zeros((Bp, C), dtype=np.int32)
        lvl = [list(range(0, 4)), list(range(4, 20)), list(range(20, 84)), list(range(84, 340))]
        for d in range(4):
            for j, c in enumerate(lvl[d]):
                par[:, c] = -1 if d == 0 else lvl[d - 1][j // 4]
        cl = torch.from_numpy(rng.standard_normal((Bp * 85, V // 8), dtype=np.float32)).cuda()
        ct, clq = sv.draft_topk(cl, 4)
        cpar = torch.from_numpy(par).cuda()
        ctok = ct.reshape(Bp, C).contiguous()
        clog = clq.reshape(Bp, C).contiguous()
        torch.cuda.synchronize()
        if wl == "draft_topk":
            alg_bytes = R * V * 2
            units = R

            def step(i, ev=None):
                sv.draft_topk(lsets[i % nrc], kk)
            config = dict(workload=wl, rows=R, V=V, k=kk, input_dtype="bf16", input_copies=nrc)
            unit = "draft rows/s"
            metric = "draft top-k: rows/sec + achieved HBM GB/s (% of peak)"
        else:
            alg_bytes = Bp * C * 12 + Bp * n_max * 12
            units = Bp

            def step(i, ev=None):
                sv.tree_prune(cpar, ctok, clog, n_max, tau=0.1)
            config = dict(workload=wl, B=Bp, candidates=C, n_max=n_max,
                          forest="4-wide, 4-deep, top-4 log q of random draft rows")
            unit = "pruned trees/s"
            metric = "tree pruning: trees/sec"
        flops = 0
    elif wl in ("telemetry", "gamma_update"):
        # The control work after a round of the bimodal batch (B=256, ragged
        # gamma): the round's counters, or the next gamma per request from the
        # 16-step history.  Outcomes from the library's own verify of it.
        bm = synth.bimodal_v152k()
        gv = sv.verify_linear(to_dev_logits(torch, bm["target"], 1), to_dev_logits(torch, bm["draft"], 1),
                              torch.from_numpy(bm["offsets"]).cuda(), torch.from_numpy(bm["tokens"]).cuda(),
                              torch.from_numpy(bm["temp_target"]).cuda(),
                              torch.from_numpy(bm["temp_draft"]).cuda())
        na_dev = gv["num_accepted"]
        off_dev = torch.from_numpy(bm["offsets"]).cuda()
        torch.cuda.synchronize()
        ctl_na, ctl_off = na_dev.cpu().numpy(), bm["offsets"]
        Bc = int(na_dev.shape[0])
        units = Bc
        if wl == "telemetry":
            acc = sv.telemetry_block()
            alg_bytes = Bc * 8 + 156 * 8

            def step(i, ev=None):
                sv.telemetry_linear(na_dev, off_dev, acc)
            unit = "batch rows/s"
            metric = "round telemetry: batch rows/sec"
        else:
            hist = torch.zeros(Bc, dtype=torch.int32, device=dev)
            alg_bytes = Bc * 24

            def step(i, ev=None):
                sv.gamma_update(hist, na_dev, off_dev)
            unit = "requests/s"
            metric = "dynamic gamma update: requests/sec"
        config = dict(workload=wl, B=Bc, gamma="ragged 2/4/8 (bimodal batch)")
        flops = 0
    elif wl == "telemetry_tree":
        # The counters after a TOPK round of the tree_v32k trees (B=64, 64
        # nodes each): outcomes from the library's own verify of them.
        tr = synth.tree_v32k()
        par_dev = torch.from_numpy(tr["parents"]).cuda()
        gv = sv.verify_tree(to_dev_logits(torch, tr["target"], 1), par_dev,
                            torch.from_numpy(tr["tokens"]).cuda(),
                            torch.from_numpy(tr["temp_target"]).cuda())
        na_dev, path_dev = gv["num_accepted"], gv["path_nodes"]
        torch.cuda.synchronize()
        Bc, Nt = tr["parents"].shape
        ctl_na = na_dev.cpu().numpy()
        ctl_off = (path_dev.cpu().numpy(), tr["parents"])
        units = Bc
        acc = sv.telemetry_block()
        alg_bytes = Bc * 4 + Bc * (Nt - 1) * 4 + Bc * Nt * 4 + 156 * 8

        def step(i, ev=None):
            sv.telemetry_tree(na_dev, path_dev, par_dev, acc)
        unit = "trees/s"
        metric = "round telemetry: trees/sec"
        config = dict(workload=wl, B=Bc, nodes=Nt, trees="tree_v32k, TOPK walk")
        flops = 0
    elif wl == "kv_commit":
        # The commit after a SAMPLED_WOR tree round: paths from the library's
        # own verify of the tree_wor_v32k trees, caches of 4 layers.
        B, H, N, dd, L0, layers = 64, 32, 64, 128, 4096, 4
        S = L0 + N
        tr = synth.tree_wor_v32k()
        g = sv.verify_tree(to_dev_logits(torch, tr["target"], 1), torch.from_numpy(tr["parents"]).cuda(),
                           torch.from_numpy(tr["tokens"]).cuda(),
                           torch.from_numpy(tr["temp_target"]).cuda(),
                           n_nodes=torch.from_numpy(tr["n_nodes"]).cuda(),
                           cand_mode=sv.SV_TREE_SAMPLED_WOR,
                           draft_logits=to_dev_logits(torch, tr["draft"], 1),
                           temp_draft=torch.from_numpy(tr["temp_draft"]).cuda())
        n_acc = g["num_accepted"]
        path = g["path_nodes"]
        torch.cuda.synchronize()
        kc = torch.empty((layers, B, H, S, dd), dtype=torch.bfloat16, device=dev).normal_()
        vc = torch.empty_like(kc).normal_()
        pl = torch.full((B,), L0, dtype=torch.int32, device=dev)
        nl = torch.empty(B, dtype=torch.int32, device=dev)
        na, pa = n_acc.cpu().numpy(), path.cpu().numpy()
        moved = 0
        for b in range(B):
            n = int(na[b])
            i0 = next((i for i in range(n) if pa[b, i] != i + 1), n)
            moved += n - i0
        alg_bytes = moved * layers * H * dd * 2 * 2 * 2    # K and V rows, read and written
        flops = 0
        units = int(np.maximum(na, 0).sum())

        def step(i, ev=None):
            if ev is not None:
                sv.profile_next(ev[0], ev[1])
            sv.kv_commit(kc, vc, pl, n_acc, path, new_len=nl)
        config = dict(workload=wl, B=B, H=H, head_dim=dd, prefix_len=L0, nodes=N, layers=layers,
                      paths="SAMPLED_WOR verify of tree_wor_v32k",
                      accepted_tokens=units, rows_moved_per_layer_head=moved, input_dtype="bf16")
        unit = "committed tokens/s"
        metric = "KV commit: committed tokens/sec + achieved HBM GB/s (% of peak)"
    elif wl == "attn_tree":
        B, H, N, dd, L = 64, 32, 64, 128, 4096
        tree = synth.tree_v32k(seed=4, B=B, N=N, V=64)
        q, k, v, pl = synth.attn_tensors(B=B, H=H, N=N, L=L)
        qd = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda()
        kd = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).cuda()
        vd = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda()
        pld = torch.from_numpy(pl).cuda()
        par = torch.from_numpy(tree["parents"]).cuda()
        outs = dict(out=torch.empty_like(qd),
                    lse=torch.empty((B, H, N), dtype=torch.float32, device=dev))
        kv_bytes = 2 * B * H * (L + N) * dd * 2
        qo_bytes = 2 * B * H * N * dd * 2
        alg_bytes = kv_bytes + qo_bytes
        flops = 0
        anc = [synth_anc(tree["parents"][b]) for b in range(B)]
        for b in range(B):
            keys = L * N + int(sum(anc[b]))
            flops += 2 * 2 * H * keys * dd
        units = B * N

        def step(i, ev=None):
            if ev is not None:
                sv.profile_next(ev[0], ev[1])
            sv.verify_attn(qd, kd, vd, pld, par, outputs=outs)
        config = dict(workload=wl, B=B, H=H, N=N, head_dim=dd, prefix_len=L,
                      mask="tree (64-node best-first top-4 trees)", input_dtype="bf16")
        unit = "verified query tokens/s"
        metric = "verify-attention query tokens/sec + achieved HBM GB/s (% of peak)"
    else:
        d = early if early is not None else synth.WORKLOADS[wl]()
        per_call = synth.logits_bytes(d)
        nc = copies_for(per_call)
        if d["kind"] == "linear":
            sets = []
            for c in range(nc):
                sets.append(dict(
                    t=to_dev_logits(torch, d["target"], d["dtype"]),
                    d=to_dev_logits(torch, d["draft"], d["dtype"])))
            off = torch.from_numpy(d["offsets"].astype(np.int32)).cuda()
            tok = torch.from_numpy(d["tokens"].astype(np.int32)).cuda()
            tt = torch.from_numpy(d["temp_target"]).cuda()
            td = torch.from_numpy(d["temp_draft"]).cuda()
            total = int(d["offsets"][-1])
            Bn = d["B"]
            outs = dict(num_accepted=torch.empty(Bn, dtype=torch.int32, device=dev),
                        out_tokens=torch.empty(total + Bn, dtype=torch.int32, device=dev),
                        p_at_draft=torch.empty(total, dtype=torch.float32, device=dev),
                        q_at_draft=torch.empty(total, dtype=torch.float32, device=dev),
                        row_status=torch.empty(Bn, dtype=torch.int32, device=dev))
            ws = torch.empty(sv.linear_workspace_size(Bn, total, d["V"], d["dtype"]),
                             dtype=torch.uint8, device=dev)
            units = total

            def step(i, ev=None):
                s = sets[i % nc]
                if ev is not None:
                    sv.profile_next(ev[0], ev[1])
                sv.verify_linear(s["t"], s["d"], off, tok, tt, td, seed=0, step=i, workspace=ws,
                                 outputs=outs)
            config = dict(workload=wl, B=Bn, gamma=("ragged 2/4/8" if wl == "bimodal_v152k"
                                                    else int(d["gammas"][0])),
                          total_draft=total, V=d["V"],
                          input_dtype="bf16" if d["dtype"] == 1 else "fp32",
                          input_copies=nc)
            unit = "verified draft positions/s"
        else:
            wor = d["kind"] == "tree_wor"
            sets = [to_dev_logits(torch, d["target"], d["dtype"]) for _ in range(nc)]
            dsets = [to_dev_logits(torch, d["draft"], d["dtype"]) for _ in range(nc)] if wor else None
            td = torch.from_numpy(d["temp_draft"]).cuda() if wor else None
            par = torch.from_numpy(d["parents"]).cuda()
            tok = torch.from_numpy(d["tokens"]).cuda()
            nn = torch.from_numpy(d["n_nodes"]).cuda()
            tt = torch.from_numpy(d["temp_target"]).cuda()
            Bn, N = d["B"], d["N"]
            outs = dict(num_accepted=torch.empty(Bn, dtype=torch.int32, device=dev),
                        path_nodes=torch.empty((Bn, N - 1), dtype=torch.int32, device=dev),
                        out_tokens=torch.empty((Bn, N), dtype=torch.int32, device=dev),
                        p_at_node=torch.empty((Bn, N), dtype=torch.float32, device=dev),
                        row_status=torch.empty(Bn, dtype=torch.int32, device=dev))
            ws = torch.empty(sv.tree_workspace_size(Bn, N, d["V"], d["dtype"]),
                             dtype=torch.uint8, device=dev)
            units = int(d["n_nodes"].sum()) - Bn

            def step(i, ev=None):
                if ev is not None:
                    sv.profile_next(ev[0], ev[1])
                sv.verify_tree(sets[i % nc], par, tok, tt, n_nodes=nn, seed=0, step=i,
                               workspace=ws, outputs=outs,
                               cand_mode=sv.SV_TREE_SAMPLED_WOR if wor else sv.SV_TREE_TOPK,
                               draft_logits=dsets[i % nc] if wor else None, temp_draft=td)
            config = dict(workload=wl, B=Bn, nodes=N, V=d["V"],
                          mode="SAMPLED_WOR" if wor else "TOPK", input_dtype="bf16",
                          input_copies=nc)
            # rows read by the vocabulary pass: those of the nodes with
            # children (a leaf's row only when a walk stops there)
            config["target_rows_read"] = synth.inner_nodes(d)
            if wor:
                config["draft_rows_read"] = synth.inner_nodes(d)
            unit = "verified draft nodes/s"
        alg_bytes = per_call
        flops = 0
        metric = METRIC

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    use_graph = not args.no_graph and wl not in ("attn_tree",)
    # The GPU's clocks ramp up over the first milliseconds of sustained work
    # (a 20-step replay of the bimodal batch runs at 180-195 us per step for
    # its first few replays, then settles at 162 us), so untimed work goes on
    # until the device has been busy for `settle` seconds before the timed
    # region.
    settle = args.settle_seconds
    if use_graph:
        # The K timed steps are captured once and replayed as one graph, so
        # the host does not pace the GPU.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(args.warmup + i)
        t_w = time.perf_counter()
        n_untimed = 0
        while n_untimed < 1 or time.perf_counter() - t_w < settle:
            graph.replay()      # untimed: the first uploads the graph
            torch.cuda.synchronize()
            n_untimed += 1
        untimed = "%d eager steps, then %d untimed replays of the timed graph (%.2f s)" % (
            args.warmup, n_untimed, time.perf_counter() - t_w)
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        t_w = time.perf_counter()
        n_untimed = 0
        while time.perf_counter() - t_w < settle:
            step(args.warmup + n_untimed)
            torch.cuda.synchronize()
            n_untimed += 1
        untimed = "%d eager steps, then %d more untimed steps (%.2f s)" % (
            args.warmup, n_untimed, time.perf_counter() - t_w)
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(args.warmup + i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    # Dominant kernel's duration: the same K steps again, each with a pair of
    # HIP events attached to that kernel's dispatch on the call's stream.
    hooked = wl not in ("draft_topk", "tree_prune", "telemetry", "telemetry_tree",
                        "gamma_update")
    # One kernel per step: a pair of events around GROUP calls in a row on the
    # current stream, divided by GROUP, so that the events' own fixed cost
    # (a few microseconds) is not charged to each launch of a short kernel.
    group = 1 if hooked else max(1, min(10, args.steps))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps // group)]
    for i, ev in enumerate(evs):
        if hooked:
            step(args.warmup + i, ev)
        else:
            ev[0].record()
            for j in range(group):
                step(args.warmup + i * group + j)
            ev[1].record()
    torch.cuda.synchronize()
    kern_ms = [a.elapsed_time(b) / group for a, b in evs]
    avg_kern_s = float(np.mean(kern_ms)) / 1e3
    ms_per_step = wall * 1e3 / args.steps
    # Hot cache, labelled as such: the same input copy every call, so inputs
    # that fit the 256 MB Infinity Cache come largely from it.
    hot = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(max(1, min(args.steps, 50) // group))]
    for ev in hot:
        if hooked:
            step(0, ev)
        else:
            ev[0].record()
            for _ in range(group):
                step(0)
            ev[1].record()
    torch.cuda.synchronize()
    hot_ms = [a.elapsed_time(b) / group for a, b in hot]

    achieved = alg_bytes / avg_kern_s / 1e9
    traffic = load_traffic(args.traffic_json, wl, kernel_source_sig(wl))
    roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(achieved / HBM_PEAK_GBS, 4),
                traffic=traffic,
                kernel=dominant_kernel(wl),
                algorithmic_bytes_per_launch=int(alg_bytes),
                avg_kernel_us=round(avg_kern_s * 1e6, 2),
                median_kernel_us=round(float(np.median(kern_ms)) * 1e3, 2),
                hot_cache_kernel_us=round(float(np.median(hot_ms)) * 1e3, 2))
    # The whole call as a caller sees it (every kernel of the step, back to
    # back in the replayed graph) against the same algorithmic bytes.
    whole = alg_bytes / (ms_per_step / 1e3) / 1e9
    roof["whole_call"] = dict(achieved=round(whole, 1), frac=round(whole / HBM_PEAK_GBS, 4),
                              us_per_call=round(ms_per_step * 1e3, 2))
    if flops:
        roof["mfma_tflops"] = round(flops / avg_kern_s / 1e12, 2)
        roof["mfma_util"] = round(flops / avg_kern_s / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)

    config["launch"] = "hip graph of %d steps" % args.steps if use_graph else "eager"
    config["untimed_warmup"] = untimed
    out = dict(metric=metric, value=round(units / (ms_per_step / 1e3), 1), unit=unit, n_gpus=1,
               steps=args.steps, warmup=args.warmup, ms_per_step=round(ms_per_step, 5),
               higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f32",
               data="synthetic", config=config, roofline=roof)
    if not args.no_cpu_baseline:
        if wl == "kv_commit":
            out["cpu_baseline"] = cpu_baseline_kv(kc, vc, L0, na, pa, N, args.cpu_seconds)
        elif wl == "draft_topk":
            out["cpu_baseline"] = cpu_baseline_topk(rows, kk, args.cpu_seconds)
        elif wl in ("telemetry", "telemetry_tree", "gamma_update"):
            out["cpu_baseline"] = cpu_baseline_control(wl, ctl_na, ctl_off, args.cpu_seconds)
        elif wl == "tree_prune":
            out["cpu_baseline"] = cpu_baseline_prune(par, ctok.cpu().numpy(), clog.cpu().numpy(),
                                                     n_max, args.cpu_seconds)
        elif wl == "attn_tree":
            out["cpu_baseline"] = cpu_baseline_attn(q, k, v, pl, tree["parents"], args.cpu_seconds)
        elif d["kind"] == "linear":
            out["cpu_baseline"] = cpu_baseline_linear(d, args.cpu_seconds)
        else:
            out["cpu_baseline"] = cpu_baseline_tree(d, args.cpu_seconds)
        out["cpu_baseline"].setdefault("host_cores", host_cores())
        if pool_baseline is not None:
            out["cpu_baseline_pool"] = pool_baseline
    print(json.dumps(out), flush=True)


def synth_anc(parents):
    """Number of visible new-token keys per query (ancestors plus itself)."""
    N = len(parents)
    out = []
    for i in range(N):
        c, j = 0, i
        while j >= 0:
            c += 1
            j = int(parents[j]) if j > 0 else -1
        out.append(c)
    return out


if __name__ == "__main__":
    main()
