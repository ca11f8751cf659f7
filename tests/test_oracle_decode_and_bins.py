"""Pins of two small oracle pieces that every parity test leans on:

* the bf16 decode (`oracle.bf16_bits_to_f64`), against the IEEE-754 binary
  format written out field by field (bf16 is binary32 with the low 16
  fraction bits dropped: 1 sign bit, 8 exponent bits of bias 127, 7 fraction
  bits), against fixed patterns whose values follow from that definition, and
  against torch's own bfloat16 type as an independent library routine;
* the percentile bins of the telemetry summary (the lonae page's acceptance
  P50 / P95 / P99 over the per-request histogram), against the nearest-rank
  percentile of the rows the histogram counts: the q-th percentile of n rows
  is the row of rank ceil(q n / 100) in sorted order, so its bin is the first
  whose cumulative count reaches q n / 100.  Hand-built histograms put that
  count exactly on a bin edge, where a strict comparison would move the bin.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import decode as OD
from oracle import telemetry as TM


def ieee_bf16(bits):
    """Value of one bf16 pattern from the format's fields (no bit reinterpretation)."""
    s = (bits >> 15) & 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    sign = -1.0 if s else 1.0
    if e == 0xFF:
        return sign * math.inf if m == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(m, -126 - 7)            # subnormal: 0.m * 2^-126
    return sign * math.ldexp(128 + m, e - 127 - 7)      # normal: 1.m * 2^(e - 127)


FIXED = [
    (0x3F80, 1.0), (0xBF80, -1.0), (0xC040, -3.0), (0x4049, 3.140625),
    (0x3F81, 1.0 + 2.0 ** -7), (0x0080, 2.0 ** -126), (0x0001, 2.0 ** -133),
    (0x007F, 127 * 2.0 ** -133), (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),
    (0xFF7F, -(2.0 - 2.0 ** -7) * 2.0 ** 127), (0x7F80, math.inf), (0xFF80, -math.inf),
    (0x4180, 16.0), (0x3E00, 0.125),
]


@pytest.mark.parametrize("bits,want", FIXED)
def test_bf16_fixed_patterns(bits, want):
    got = oracle.bf16_bits_to_f64(np.array([bits], dtype=np.uint16))[0]
    assert got == want, "0x%04X -> %r, want %r" % (bits, got, want)


def test_bf16_signed_zero_and_nan():
    z = oracle.bf16_bits_to_f64(np.array([0x0000, 0x8000, 0x7FC0, 0xFFC1, 0x7F81], dtype=np.uint16))
    assert z[0] == 0.0 and not math.copysign(1.0, z[0]) < 0
    assert z[1] == 0.0 and math.copysign(1.0, z[1]) < 0
    assert np.all(np.isnan(z[2:]))


def test_bf16_every_pattern_matches_the_format_definition():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    want = np.array([ieee_bf16(int(b)) for b in range(65536)])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_bf16_matches_torch_bfloat16():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 65536, size=1 << 16).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_bits_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_decode_logits_fp32_is_exact_widening():
    rng = np.random.default_rng(12)
    x = rng.standard_normal(4096).astype(np.float32) * np.float32(37.0)
    got = oracle.decode_logits(x, OD.DTYPE_F32)
    assert got.dtype == np.float64 and np.array_equal(got, x.astype(np.float64))
    with pytest.raises(ValueError):
        oracle.decode_logits(x, 7)


def nearest_rank_bin(hist, q):
    """Bin of the row of rank ceil(q n / 100) when the rows are listed bin by bin."""
    rows = np.repeat(np.arange(len(hist)), hist)
    n = len(rows)
    rank = -(-q * n // 100)                              # ceil in integers
    return int(rows[rank - 1])


def summary_bins(hist):
    t = TM.empty()
    t["acc_rate_hist"][:] = hist
    s = TM.summary(t)
    return [s["acc_rate_p%d_bin" % q] for q in (50, 95, 99)]


def _hist(**bins):
    h = np.zeros(TM.ACC_BINS, dtype=np.int64)
    for k, v in bins.items():
        h[int(k[1:])] = v
    return h


@pytest.mark.parametrize("hist,want", [
    # 20 rows: P50 needs 10 rows (reached exactly at bin 3), P95 19 (exactly at
    # bin 7), P99 19.8 -> 20 (bin 12)
    (_hist(b3=10, b7=9, b12=1), [3, 7, 12]),
    # 100 rows: P50 at 50 exactly (bin 0), P95 at 95 exactly (bin 5), P99 at 99 (bin 19)
    (_hist(b0=50, b5=45, b10=4, b19=1), [0, 5, 10]),
    # 100 rows, P99 at 99 exactly: still bin 4 (a strict comparison would give 8)
    (_hist(b4=99, b8=1), [4, 4, 4]),
    # one row: every percentile is that row
    (_hist(b17=1), [17, 17, 17]),
    # two rows: P50 is the first (rank 1), P95 and P99 the second
    (_hist(b2=1, b9=1), [2, 9, 9]),
])
def test_percentile_bins_on_bin_edges(hist, want):
    assert summary_bins(hist) == want
    assert [nearest_rank_bin(hist, q) for q in (50, 95, 99)] == want


def test_percentile_bins_empty_window():
    assert summary_bins(np.zeros(TM.ACC_BINS, dtype=np.int64)) == [None, None, None]


def test_percentile_bins_match_nearest_rank_by_brute_force():
    rng = np.random.default_rng(13)
    for trial in range(400):
        n_used = rng.integers(1, 6)
        hist = np.zeros(TM.ACC_BINS, dtype=np.int64)
        hist[rng.choice(TM.ACC_BINS, size=n_used, replace=False)] = rng.integers(1, 60, size=n_used)
        if trial % 4 == 0:            # totals that are multiples of 100 and 20 (edge-heavy)
            hist[rng.integers(0, TM.ACC_BINS)] += (-hist.sum()) % 100
        assert summary_bins(hist) == [nearest_rank_bin(hist, q) for q in (50, 95, 99)], hist
