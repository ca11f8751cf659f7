"""spec_verify_linear_noalloc against spec_verify_linear, through the C ABI.

The allocation-free entry point runs the same kernels with the library's
static per-GPU scratch as the workspace, so its outputs must equal the
workspace entry point's bit for bit.  Two calls in a row share the scratch:
the bimodal batch (B=256 ragged rows over V=152064 bf16, about 1.4 MB of
scratch), then a smaller one (B=32, gamma=5, V=32000), whose results must
not depend on what the first call left behind.  A request beyond the scratch
is refused before any launch.
"""

import numpy as np
import pytest

import synth
from gpu_util import logits_to_dev, i32, f32, say, torch_mod

pytestmark = pytest.mark.gpu


def _inputs(d):
    return (logits_to_dev(d["target"], d["dtype"]), logits_to_dev(d["draft"], d["dtype"]),
            i32(d["offsets"]), i32(d["tokens"]), f32(d["temp_target"]), f32(d["temp_draft"]))


def _run_both(d, seed, step):
    import rejection_sampling_verify_04_amd as sv
    torch = torch_mod()
    args = _inputs(d)
    ref = sv.verify_linear(*args, seed=seed, step=step)
    got = sv.verify_linear_noalloc(*args, seed=seed, step=step)
    torch.cuda.synchronize()
    return ({k: v.cpu().numpy() for k, v in ref.items()},
            {k: v.cpu().numpy() for k, v in got.items()})


def _assert_same(ref, got, label):
    for k in ("num_accepted", "out_tokens", "row_status", "p_at_draft", "q_at_draft"):
        assert np.array_equal(ref[k].view(np.int32), got[k].view(np.int32)), (label, k)
    say("[no-alloc] %s: identical to the workspace entry point (%d rows, accepted %d)" % (
        label, len(ref["num_accepted"]), int(np.maximum(ref["num_accepted"], 0).sum())))


def test_noalloc_matches_workspace_entry_point_two_calls():
    big = synth.bimodal_v152k()
    ref, got = _run_both(big, seed=3, step=11)
    _assert_same(ref, got, "bimodal B=256 V=152064")
    small = synth.linear_v32k()
    ref, got = _run_both(small, seed=5, step=7)
    _assert_same(ref, got, "B=32 gamma=5 V=32000")


def test_noalloc_refuses_requests_beyond_the_scratch():
    import rejection_sampling_verify_04_amd as sv
    torch = torch_mod()
    L = sv.library()
    need = L.spec_verify_linear_workspace_size(4096, 4096 * 8, 152064, 1)
    assert need > sv.SV_STATIC_SCRATCH_BYTES
    x = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    o = torch.zeros(4096 * 9 + 1, dtype=torch.int32, device="cuda")
    t = torch.ones(4096, dtype=torch.float32, device="cuda")
    st = L.spec_verify_linear_noalloc(x.data_ptr(), x.data_ptr(), 1, 4096, 152064, 4096 * 8,
                                      o.data_ptr(), o.data_ptr(), t.data_ptr(), t.data_ptr(), 0, 0,
                                      None, o.data_ptr(), o.data_ptr(), None, None, None, None)
    assert st == sv.SV_ERR_SCRATCH
