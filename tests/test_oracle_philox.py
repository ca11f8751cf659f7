"""Pins of the oracle's Philox-4x32-10.

The oracle's generator is written from the published definition (Salmon et
al., SC'11).  It is checked against an independent implementation, rocRAND's
host-callable Philox-4x32-10 engine (called through a small host program, not
copied), and against plain statistical properties of uniforms.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest
import scipy.stats

from oracle.philox import philox4x32_10, verify_uniforms, words_to_uniform

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="session")
def rocrand_words(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND reference program")
    exe = str(tmp_path_factory.mktemp("rocrand") / "philox_words")
    subprocess.run([hipcc, "-O2", "-o", exe,
                    os.path.join(HERE, "helpers", "rocrand_philox_words.cpp")],
                   check=True, capture_output=True)

    def run(counters, key):
        counters = np.asarray(counters, dtype=np.uint64)
        lines = [f"{len(counters)} {int(key[0])} {int(key[1])}"]
        lines += [" ".join(str(int(v)) for v in row) for row in counters]
        out = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True,
                             text=True, check=True).stdout
        return np.array([[int(t) for t in ln.split()] for ln in out.strip().split("\n")],
                        dtype=np.uint64)
    return run


def test_matches_rocrand_on_random_counters_and_keys(rocrand_words):
    rng = np.random.default_rng(123)
    for trial in range(4):
        ctr = rng.integers(0, 2 ** 32, size=(4096, 4), dtype=np.uint64)
        key = tuple(int(v) for v in rng.integers(0, 2 ** 32, size=2, dtype=np.uint64))
        assert np.array_equal(rocrand_words(ctr, key), philox4x32_10(ctr, key).astype(np.uint64))


def test_matches_rocrand_on_verify_layout(rocrand_words):
    # counters exactly as the verify step builds them: (slot, row_id, step_lo, step_hi)
    seed, step = 0x0123456789ABCDEF, (7 << 32) | 3
    rows = np.repeat(np.arange(64, dtype=np.uint64), 65)
    slots = np.tile(np.arange(65, dtype=np.uint64), 64)
    ctr = np.stack([slots, rows, np.full_like(rows, step & 0xFFFFFFFF),
                    np.full_like(rows, step >> 32)], axis=1)
    key = (seed & 0xFFFFFFFF, seed >> 32)
    ref = rocrand_words(ctr, key)
    ua, us = verify_uniforms(seed, step, 5, 65)
    sel = rows == 5
    assert np.array_equal(words_to_uniform(ref[sel, 0]), ua)
    assert np.array_equal(words_to_uniform(ref[sel, 1]), us)


def test_zero_counter_zero_key_is_not_degenerate():
    w = philox4x32_10(np.zeros((1, 4), dtype=np.uint64), (0, 0))
    assert np.any(w != 0)


def test_uniform_statistics():
    n = 1 << 18
    ctr = np.zeros((n, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(n) % 65
    ctr[:, 1] = np.arange(n) // 65
    w = philox4x32_10(ctr, (0, 0))
    u = words_to_uniform(w[:, 0])
    assert u.min() >= 0.0 and u.max() <= 1.0 - 2.0 ** -24
    assert np.all(u * 2 ** 24 == np.floor(u * 2 ** 24))       # on the 2^-24 grid
    assert abs(u.mean() - 0.5) < 5 * np.sqrt(1 / 12 / n)
    assert abs(u.var() - 1 / 12) < 5 * np.sqrt(1 / 180 / n)
    assert scipy.stats.kstest(u, "uniform").pvalue > 1e-4
    # every output bit of every word is balanced
    bits = (w[:, :, None] >> np.arange(32, dtype=np.uint32)) & 1
    frac = bits.mean(axis=0)
    assert np.all(np.abs(frac - 0.5) < 6 * np.sqrt(0.25 / n))
    # adjacent slots are uncorrelated
    assert abs(np.corrcoef(u[:-1], u[1:])[0, 1]) < 6 / np.sqrt(n)


def test_row_and_step_change_the_stream():
    a = verify_uniforms(0, 0, 1, 8)[0]
    b = verify_uniforms(0, 0, 2, 8)[0]
    c = verify_uniforms(0, 1, 1, 8)[0]
    d = verify_uniforms(1, 0, 1, 8)[0]
    assert not np.array_equal(a, b) and not np.array_equal(a, c) and not np.array_equal(a, d)
