"""GPU parity of spec_verify_kv_commit against the oracle (bit-exact copies).

Caches hold random bf16 bit patterns.  Paths come from the library's own
tree verify on peaked trees (deep accepted paths), from chains (linear
rounds), and from hand-made error and malformed rows.  Every slot below the
new length must equal the oracle's; every slot the commit does not write
must keep its old bits.
"""

import numpy as np
import pytest

import oracle
from oracle.kv import commit_row_plan
import synth
from gpu_util import i32, run_tree, say, torch_mod

pytestmark = pytest.mark.gpu


def rand_cache(rng, shape):
    torch = torch_mod()
    bits = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    return bits, torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def check(k_bits, v_bits, L, n_acc, path, N, label, layers_dim=True):
    import rejection_sampling_verify_04_amd as sv
    torch = torch_mod()
    kd = torch.from_numpy(k_bits.view(np.int16)).view(torch.bfloat16).cuda()
    vd = torch.from_numpy(v_bits.view(np.int16)).view(torch.bfloat16).cuda()
    if not layers_dim:
        kd, vd = kd[0], vd[0]
    nl = sv.kv_commit(kd, vd, i32(L), i32(n_acc), None if path is None else i32(path), n_new=N)
    torch.cuda.synchronize()
    kg = kd.cpu().view(torch.int16).numpy().view(np.uint16)
    vg = vd.cpu().view(torch.int16).numpy().view(np.uint16)
    if not layers_dim:
        kg, vg = kg[None], vg[None]
    k_ref, v_ref, nl_ref = oracle.kv_commit(k_bits, v_bits, L, n_acc, path, N)
    assert np.array_equal(nl.cpu().numpy(), nl_ref), (nl.cpu().numpy(), nl_ref)
    B = k_bits.shape[1]
    moved = 0
    for b in range(B):
        _, moves = commit_row_plan(int(L[b]), int(n_acc[b]), None if path is None else path[b], N,
                                   k_bits.shape[3])
        dst = {d for s, d in moves if s != d}
        moved += len(dst)
        keep = np.ones(k_bits.shape[3], dtype=bool)
        keep[list(dst)] = False
        assert np.array_equal(kg[:, b][..., keep, :], k_bits[:, b][..., keep, :]), "b=%d" % b
        assert np.array_equal(vg[:, b][..., keep, :], v_bits[:, b][..., keep, :]), "b=%d" % b
        top = max(int(nl_ref[b]), 0)
        assert np.array_equal(kg[:, b, :, :top], k_ref[:, b, :, :top]), "b=%d" % b
        assert np.array_equal(vg[:, b, :, :top], v_ref[:, b, :, :top]), "b=%d" % b
    say("[kv] %s: ok, new lengths %s, rows moved %d" % (label, nl_ref[:8].tolist(), moved))


def tree_paths(seed, B, N):
    d = synth.peaked_tree(seed=seed, B=B, N=N, V=64)
    g = run_tree(d)
    return g["num_accepted"], g["path_nodes"]


def test_commit_after_tree_verify():
    rng = np.random.default_rng(70)
    B, N, H, d = 24, 21, 4, 128
    n_acc, path = tree_paths(71, B, N)
    assert max(n_acc) >= 3
    L = rng.integers(0, 50, size=B).astype(np.int32)
    S = int(L.max()) + N + 5
    k, _ = rand_cache(rng, (2, B, H, S, d))
    v, _ = rand_cache(rng, (2, B, H, S, d))
    check(k, v, L, n_acc, path, N, "tree paths, 2 layers, d=128")


def test_commit_head_dims_and_single_layer():
    rng = np.random.default_rng(72)
    B, N, H = 16, 21, 3
    n_acc, path = tree_paths(73, B, N)
    for d in (64, 256, 8):
        L = rng.integers(0, 9, size=B).astype(np.int32)
        S = int(L.max()) + N
        k, _ = rand_cache(rng, (1, B, H, S, d))
        v, _ = rand_cache(rng, (1, B, H, S, d))
        check(k, v, L, n_acc, path, N, "d=%d, [B,H,S,d] caches" % d, layers_dim=False)


def test_linear_rounds_move_nothing():
    rng = np.random.default_rng(74)
    B, g, H, d = 8, 5, 2, 128
    L = rng.integers(0, 30, size=B).astype(np.int32)
    S = int(L.max()) + g + 1
    k, _ = rand_cache(rng, (1, B, H, S, d))
    v, _ = rand_cache(rng, (1, B, H, S, d))
    n_acc = np.array([0, 5, 3, 5, 1, 0, 2, 4], dtype=np.int32)   # all-reject, all-accept, mixed
    check(k, v, L, n_acc, None, g + 1, "linear chains")


def test_error_and_malformed_rows():
    rng = np.random.default_rng(75)
    B, N, H, d = 8, 6, 2, 64
    L = np.array([3, 3, 3, 3, 3, 10, 3, 3], dtype=np.int32)
    S = 14
    path = np.zeros((B, N - 1), dtype=np.int32)
    path[0, :2] = [2, 4]          # valid, moves both rows
    path[1, :2] = [2, 2]          # not increasing
    path[2, :2] = [1, 6]          # node id out of range
    path[3, :3] = [3, 4, 5]       # valid: slots L+3.. overlap their destinations
    path[4, :1] = [1]             # valid, nothing moves
    path[5, :1] = [2]             # L + N > S_max
    path[6, :2] = [1, 2]          # flagged row (n = -1)
    path[7, :5] = [1, 2, 3, 4, 5] # valid, depth N - 1
    n_acc = np.array([2, 2, 2, 3, 1, 1, -1, 5], dtype=np.int32)
    k, _ = rand_cache(rng, (1, B, H, S, d))
    v, _ = rand_cache(rng, (1, B, H, S, d))
    check(k, v, L, n_acc, path, N, "error and malformed rows")


def test_commit_full_size_sampled():
    """B=64, H=32, d=128, prefix 4096 + 64 new tokens: the copied rows, sampled by head."""
    import rejection_sampling_verify_04_amd as sv
    torch = torch_mod()
    B, H, N, d, L0 = 64, 32, 64, 128, 4096
    S = L0 + N
    tr = synth.tree_wor(seed=76, B=B, N=N, V=64, draft_sd=6.0, pert=1.0, dtype=synth.F32)
    g = run_tree(tr)
    n_acc, path = g["num_accepted"], g["path_nodes"]
    gen = torch.Generator(device="cuda").manual_seed(77)
    k = torch.randn((B, H, S, d), generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, H, S, d), generator=gen, device="cuda").to(torch.bfloat16)
    L = np.full(B, L0, dtype=np.int32)
    heads = [(b, (7 * b) % H) for b in range(B)]
    before = [(k[b, h, L0:].cpu().float().numpy(), v[b, h, L0:].cpu().float().numpy())
              for b, h in heads]
    nl = sv.kv_commit(k, v, i32(L), i32(n_acc), i32(path)).cpu().numpy()
    torch.cuda.synchronize()
    depth = []
    for (b, h), (kb, vb) in zip(heads, before):
        new, moves = commit_row_plan(L0, int(n_acc[b]), path[b], N, S)
        assert nl[b] == new
        ka = k[b, h, L0:].cpu().float().numpy()
        va = v[b, h, L0:].cpu().float().numpy()
        for src, dst in moves:
            assert np.array_equal(ka[dst - L0], kb[src - L0]) and np.array_equal(va[dst - L0], vb[src - L0])
        depth.append(int(n_acc[b]))
    say("[kv] full size: B=%d H=%d S=%d, depth histogram %s" % (
        B, H, S, np.bincount(np.maximum(depth, 0)).tolist()))
