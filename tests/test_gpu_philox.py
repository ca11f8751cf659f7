"""GPU Philox words equal the oracle's, bit for bit, on 2^20 counters."""

import numpy as np
import pytest

from oracle.philox import philox4x32_10
from gpu_util import i32, say, torch_mod

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed,step", [(0, 0), (0x0123456789ABCDEF, (5 << 32) | 77)])
def test_gpu_words_match_oracle(seed, step):
    torch = torch_mod()
    import rejection_sampling_verify_04_amd as sv
    n_rows, n_slots = 16384, 64
    ids = np.random.default_rng(1).integers(0, 2 ** 32, size=n_rows, dtype=np.uint64).astype(np.uint32)
    gw = sv.philox_words(seed, step, n_rows, n_slots, row_ids=i32(ids.view(np.int32)))
    torch.cuda.synchronize()
    gw = gw.cpu().numpy().view(np.uint32)
    ctr = np.zeros((n_rows, n_slots, 4), dtype=np.uint64)
    ctr[:, :, 0] = np.arange(n_slots)[None, :]
    ctr[:, :, 1] = ids[:, None]
    ctr[:, :, 2] = step & 0xFFFFFFFF
    ctr[:, :, 3] = step >> 32
    ref = philox4x32_10(ctr.reshape(-1, 4), (seed & 0xFFFFFFFF, seed >> 32)).reshape(n_rows, n_slots, 4)
    assert np.array_equal(gw, ref)
    say("[philox] %d counters bit-exact" % (n_rows * n_slots))
