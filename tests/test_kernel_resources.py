"""Register budgets that the launch decisions rely on, read from hipcc's
resource remarks for gfx950 (CPU only: device code is compiled, nothing runs).

- The by-chunk vocabulary pass is chosen for a linear call when its (row,
  chunk) work items fit one round on the GPU; at B=32, gamma=5, V=32000 that is
  1408 work items of 4 waves, so it needs 6 waves per SIMD (1536 resident).
- The attention kernel is built for 2 waves per SIMD (its K/V prefetch depth).
- Draft top-k rows re-read from memory are built for 8 waves per SIMD (two
  1024-thread rows per compute unit); the register-resident variant keeps its
  registers; the small-k variant runs four 256-thread rows per compute unit.
- No hot kernel spills registers, apart from the re-reading top-k variant and a
  few prologue values of the SAMPLED_WOR walk with its 4-chunk cache.
"""

import os
import re
import shutil
import subprocess

import pytest

from rejection_sampling_verify_04_amd import build as B

pytestmark = pytest.mark.skipif(not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")),
                                reason="hipcc is not installed")

_cache = {}


def resources(src):
    """{kernel symbol: {"vgpr", "spill", "occ"}} for one source file."""
    if src in _cache:
        return _cache[src]
    flags = [f for f in B.HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [B.hipcc_path(), *flags, "--cuda-device-only", "-c", "-I", B.INCLUDE, "-I", B.CSRC,
           os.path.join(B.CSRC, src), "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    out, cur = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        if cur is None:
            continue
        for key, pat in (("vgpr", r"remark:\s+VGPRs: (\d+)"), ("spill", r"remark:\s+VGPRs Spill: (\d+)"),
                         ("occ", r"remark:\s+Occupancy \[waves/SIMD\]: (\d+)")):
            m = re.search(pat, line)
            if m:
                cur[key] = int(m.group(1))
    _cache[src] = out
    return out


def kernels(src, prefix):
    ks = {k: v for k, v in resources(src).items() if k.startswith(prefix)}
    assert ks, (src, prefix)
    return ks


def test_by_chunk_stats_fits_one_round():
    for name, r in kernels("sv_stats.hip", "_ZN2sv21stats_kernel_by_chunk").items():
        assert r["occ"] >= 6, (name, r)
        assert r["spill"] == 0, (name, r)


def test_streaming_stats_and_finish_passes_do_not_spill():
    for src, prefix in (("sv_stats.hip", "_ZN2sv12stats_kernel"), ("sv_linear.hip", "_ZN2sv"),
                        ("sv_tree.hip", "_ZN2sv11tree_kernel"), ("sv_tree.hip", "_ZN2sv15tree_wor_kernel"),
                        ("sv_kv.hip", "_ZN2sv16kv_commit_kernel")):
        for name, r in kernels(src, prefix).items():
            if name.startswith("_ZN2sv15tree_wor_kernel") and name.endswith("Li4EEEvNS_8TreeArgsE"):
                # the SAMPLED_WOR walk with a 4-chunk cache keeps 32 draft terms per
                # thread in registers at the 128-VGPR limit of a 1024-thread work
                # item; two values spill
                assert r["spill"] <= 4, (name, r)
            else:
                assert r["spill"] == 0, (name, r)


def test_attention_four_waves_per_simd():
    """32-key tiles with one tile's loads in registers: four 256-thread work
    items per compute unit, with no spill."""
    for name, r in kernels("sv_attn.hip", "_ZN2sv11attn_kernel").items():
        assert r["occ"] == 4 and r["spill"] == 0, (name, r)


def test_draft_topk_small_k_four_rows_per_cu():
    """The small-k top-k keeps a row's 128 logits per thread packed in registers
    and runs four 256-thread rows per compute unit."""
    for name, r in kernels("sv_draft.hip", "_ZN2sv23draft_topk_small_kernel").items():
        assert r["occ"] >= 4 and r["spill"] == 0, (name, r)


def test_draft_topk_variants():
    ks = kernels("sv_draft.hip", "_ZN2sv17draft_topk_kernel")
    for name, r in ks.items():
        reg = name.endswith("ELb1EEEvPKviiPKfPiPf")
        if reg:
            assert r["spill"] == 0, (name, r)
        else:
            assert r["occ"] == 8, (name, r)
    assert sum(1 for n in ks if n.endswith("ELb1EEEvPKviiPKfPiPf")) == 2
