"""The error model behind the draw bound, measured on the GPU.

Every probability of the verify is formed with one hardware 2^x (v_exp_f32).
The draw bound of tests/draw_bound.py allows it a relative error of
EPS_EXP; here the library's own 2^x (spec_verify_exp2) is compared with the
exact float64 2^x on 2^24 random exponents over the range the kernels use
(offsets keep every exponent at or below about 1), on a dense grid near 0,
and on the integers, where 2^x is exact.
"""

import numpy as np
import pytest

import draw_bound as DB
from gpu_util import say, torch_mod

pytestmark = pytest.mark.gpu


def test_exp2_error_within_the_draw_bound_model():
    import rejection_sampling_verify_04_amd as sv
    torch = torch_mod()
    rng = np.random.default_rng(71)
    x = np.concatenate([
        rng.uniform(-126.0, 1.0, size=1 << 24),
        rng.uniform(-1.0, 1.0, size=1 << 22),
        np.linspace(-8.0, 1.0, 1 << 20),
        np.arange(-126, 2, dtype=np.float64),
    ]).astype(np.float32)
    y = sv.exp2_hw(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    exact = np.exp2(x.astype(np.float64))
    rel = np.abs(y - exact) / exact
    ulp = rel * 2.0 ** 23
    worst = int(np.argmax(rel))
    say("[draw bound] hardware 2^x: max relative error %.3g (%.2f float32 ulps of the result) "
        "at x=%r; the bound allows %.3g" % (rel[worst], ulp[worst], float(x[worst]), DB.EPS_EXP))
    assert rel.max() <= DB.EPS_EXP
    ints = np.arange(-126, 2)
    assert np.array_equal(y[-len(ints):], np.exp2(ints.astype(np.float64)))
