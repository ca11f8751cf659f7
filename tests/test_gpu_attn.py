"""GPU parity of spec_verify_attn against the float64 oracle (2e-2 absolute on bf16 output)."""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import say, torch_mod

pytestmark = pytest.mark.gpu

ATOL = 2e-2


def bf16_dev(bits):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def decode(bits):
    return oracle.bf16_bits_to_f64(bits)


def run(q, k, v, L, parents):
    import rejection_sampling_verify_04_amd as sv
    torch = torch_mod()
    par = None if parents is None else torch.from_numpy(parents.astype(np.int32)).cuda()
    out = sv.verify_attn(bf16_dev(q), bf16_dev(k), bf16_dev(v),
                         torch.from_numpy(L.astype(np.int32)).cuda(), par)
    torch.cuda.synchronize()
    o = out["out"].view(torch.int16).cpu().numpy().view(np.uint16)
    return decode(o), out["lse"].cpu().numpy()


def rand_bits(rng, shape):
    return synth.bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def check_case(label, B, H, N, L_list, S_max, parents, seed):
    rng = np.random.default_rng(seed)
    d = 128
    q = rand_bits(rng, (B, H, N, d))
    k = rand_bits(rng, (B, H, S_max, d))
    v = rand_bits(rng, (B, H, S_max, d))
    L = np.array(L_list, dtype=np.int32)
    say("[attn] %s: B=%d H=%d N=%d L=%s S_max=%d" % (label, B, H, N, L.tolist(), S_max))
    o, lse = run(q, k, v, L, parents)
    ro, rl = oracle.verify_attention(decode(q), decode(k), decode(v), L, parents)
    err = np.max(np.abs(o - ro))
    lerr = np.max(np.abs(lse - rl))
    say("[attn] %s: max|dO|=%.3g max|dLSE|=%.3g" % (label, err, lerr))
    assert err < ATOL
    assert lerr < 1e-3
    return err


def test_tree_mask_small():
    parents = np.array([[-1, 0, 0, 1, 1, 2, 2, 3, 5, 8, 0, 10]] * 2, dtype=np.int32)
    check_case("tree small", 2, 3, 12, [100, 37], 160, parents, 1)


def test_causal_ragged_prefix():
    check_case("causal", 3, 2, 9, [0, 64, 130], 200, None, 2)


def test_single_query_plain_attention():
    check_case("N=1", 2, 4, 1, [1, 500], 600, None, 3)


def test_full_64_node_tree_two_tiles_of_new_tokens():
    rng = np.random.default_rng(4)
    d = synth.tree_v32k(seed=4, B=2, N=64, V=200)
    check_case("64-node trees", 2, 2, 64, [4096, 4000], 4160, d["parents"], 5)


def test_bad_prefix_row_gives_zeros():
    rng = np.random.default_rng(6)
    B, H, N, S = 2, 2, 4, 40
    q, k, v = rand_bits(rng, (B, H, N, 128)), rand_bits(rng, (B, H, S, 128)), rand_bits(rng, (B, H, S, 128))
    o, lse = run(q, k, v, np.array([10, 38], dtype=np.int32), None)
    assert np.all(o[1] == 0) and np.all(np.isnan(lse[1]))
    ro, _ = oracle.verify_attention(decode(q[:1]), decode(k[:1]), decode(v[:1]), np.array([10]), None)
    assert np.max(np.abs(o[0] - ro[0])) < ATOL


def test_config_tree_attention_full_size_sampled():
    """B=64, H=32, N=64, d=128, L=4096 against the oracle on sampled (b, h) slices."""
    torch = torch_mod()
    import rejection_sampling_verify_04_amd as sv
    B, H, N, L = 64, 32, 64, 4096
    tree = synth.tree_v32k(seed=4, B=B, N=N, V=64)
    say("[attn] generating full-size Q/K/V")
    q, k, v, pl = synth.attn_tensors(B=B, H=H, N=N, L=L)
    out = sv.verify_attn(bf16_dev(q), bf16_dev(k), bf16_dev(v), torch.from_numpy(pl).cuda(),
                         torch.from_numpy(tree["parents"]).cuda())
    torch.cuda.synchronize()
    o = decode(out["out"].view(torch.int16).cpu().numpy().view(np.uint16))
    lse = out["lse"].cpu().numpy()
    rng = np.random.default_rng(7)
    worst = 0.0
    for b, h in [(0, 0), (63, 31)] + [tuple(x) for x in rng.integers(0, [B, H], size=(6, 2))]:
        mask = oracle.ancestor_mask(tree["parents"][b], N)
        ro, rl = oracle.attention_head(decode(q[b, h]), decode(k[b, h]), decode(v[b, h]), L, mask,
                                       1 / np.sqrt(128))
        worst = max(worst, np.max(np.abs(o[b, h] - ro)))
        assert np.max(np.abs(lse[b, h] - rl)) < 1e-3
    say("[attn] full size sampled: max|dO|=%.3g" % worst)
    assert worst < ATOL
