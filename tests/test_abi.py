"""The C-ABI library: builds, loads, exports every declared symbol, validates on the host.

No call here reaches a kernel launch, so the file runs without a GPU.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


@pytest.fixture(scope="module")
def lib():
    import rejection_sampling_verify_04_amd as sv
    if not os.path.exists(sv.LIB_PATH):
        from rejection_sampling_verify_04_amd import build
        build.build()
    return sv.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_verify_\w+)\s*\(", text)))


def test_telemetry_block_layout():
    import rejection_sampling_verify_04_amd as sv
    from oracle import telemetry as TM
    # the binding's word layout is the header's struct: 7 counters then the bins
    assert sv.TELEMETRY_WORDS == 7 + TM.ACC_BINS + TM.POS_BINS + TM.RANK_BINS
    assert sv.TELEMETRY_FIELDS == TM.FIELDS
    text = open(HEADER).read()
    assert "uint64_t rounds, error_rows, drafted, accepted, full_accepts, tree_paths, tree_paths_hit;" in text


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ["spec_verify_linear", "spec_verify_tree", "spec_verify_attn",
                 "spec_verify_version", "spec_verify_status_string",
                 "spec_verify_linear_workspace_size", "spec_verify_tree_workspace_size"]:
        assert must in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    import rejection_sampling_verify_04_amd as sv
    assert sv.version() >= 1
    assert sv.status_string(0) == "ok"
    for code in (-1, -2, -3, -4, -5):
        assert sv.status_string(code) not in ("ok", "unknown status")
    assert sv.status_string(-99) == "unknown status"


def test_workspace_sizes(lib):
    n = lib.spec_verify_linear_workspace_size(32, 160, 32000, 1)
    assert n > 0 and n % 256 == 0
    # partials (352 rows x 4 chunks x 16 B) + chunk masses (32 rows x 4 chunks x 8 B)
    assert n >= 352 * 4 * 16 + 32 * 4 * 8
    assert lib.spec_verify_linear_workspace_size(-1, 0, 10, 1) == 0
    # partials and gathers of the target and (SAMPLED_WOR) draft rows
    assert lib.spec_verify_tree_workspace_size(64, 64, 32000, 1) >= 2 * 64 * 64 * (4 * 16 + 4)


def _linear(lib, **kw):
    args = dict(target=ctypes.c_void_p(16), draft=ctypes.c_void_p(16), dtype=1, B=2, V=100,
                total=4, off=ctypes.c_void_p(16), tok=ctypes.c_void_p(16),
                tt=ctypes.c_void_p(16), td=ctypes.c_void_p(16), na=ctypes.c_void_p(16),
                out=ctypes.c_void_p(16), ws=ctypes.c_void_p(256), wsb=1 << 20)
    args.update(kw)
    return lib.spec_verify_linear(args["target"], args["draft"], args["dtype"], args["B"],
                                  args["V"], args["total"], args["off"], args["tok"], args["tt"],
                                  args["td"], 0, 0, None, args["na"], args["out"], None, None,
                                  None, args["ws"], args["wsb"], None)


def test_linear_host_validation(lib):
    assert _linear(lib, dtype=7) == -1
    assert _linear(lib, B=-1) == -1
    assert _linear(lib, V=0) == -1
    assert _linear(lib, total=2 * 64 + 1) == -1          # some gamma_b > 64
    assert _linear(lib, B=0, total=0) == 0                # empty batch: no-op
    assert _linear(lib, target=None) == -1
    assert _linear(lib, na=None) == -1
    assert _linear(lib, ws=None) == -3
    assert _linear(lib, ws=ctypes.c_void_p(128)) == -3    # misaligned workspace
    assert _linear(lib, wsb=16) == -3                     # too small
    assert _linear(lib, V=64 * 8192 + 1) == -2            # vocabulary beyond the chunk table


def test_tree_and_attn_host_validation(lib):
    p = ctypes.c_void_p(256)
    common = (p, None, 1, 4, 8, 100, p, p, None)
    tail = (p, None, 0, 0, None, p, p, p, None, None, p, 1 << 20, None)
    assert lib.spec_verify_tree(*common, 1, *tail) == -1        # SAMPLED_WOR without draft rows
    wor = (p, p, 1, 4, 8, 100, p, p, None, 1, p, None)          # ... or without temp_draft
    assert lib.spec_verify_tree(*wor, *tail[2:]) == -1
    assert lib.spec_verify_tree(*common, 5, *tail) == -1
    assert lib.spec_verify_tree(p, None, 1, 4, 65, 100, p, p, None, 0, *tail) == -1
    assert lib.spec_verify_attn(p, p, p, p, None, 2, 4, 8, 64, 100, 0.1, p, None, None) == -2
    assert lib.spec_verify_attn(p, p, p, p, None, 2, 4, 65, 128, 100, 0.1, p, None, None) == -1
    assert lib.spec_verify_attn(p, p, p, p, None, 2, 4, 8, 128, 4, 0.1, p, None, None) == -1
    assert lib.spec_verify_attn(p, p, p, p, None, 0, 4, 8, 128, 100, 0.1, p, None, None) == 0
    kv = lambda *a: lib.spec_verify_kv_commit(p, p, *a)
    # layers, layer_stride, prefix_len, num_accepted, path, stride, B, H, N, d, S_max, new_len, stream
    assert kv(1, 0, p, p, None, 0, 0, 4, 8, 128, 100, p, None) == 0       # empty batch: no-op
    assert kv(1, 0, p, p, None, 0, 2, 4, 65, 128, 100, p, None) == -1     # N > 64
    assert kv(1, 0, p, p, None, 0, 2, 4, 8, 100, 100, p, None) == -1     # d not a multiple of 8
    assert kv(1, 0, p, p, None, 0, 2, 4, 8, 128, 4, p, None) == -1       # S_max < N
    assert kv(2, 16, p, p, None, 0, 2, 4, 8, 128, 100, p, None) == -1     # layer stride too small
    assert kv(1, 0, p, p, p, 3, 2, 4, 8, 128, 100, p, None) == -1         # path stride < N - 1
    assert kv(1, 0, None, p, None, 0, 2, 4, 8, 128, 100, p, None) == -1   # no prefix lengths
    assert lib.spec_verify_telemetry_linear(p, p, 0, p, None) == 0          # empty: no-op
    assert lib.spec_verify_telemetry_linear(p, None, 4, p, None) == -1
    assert lib.spec_verify_telemetry_linear(p, p, 4, ctypes.c_void_p(260), None) == -1   # misaligned
    assert lib.spec_verify_telemetry_tree(p, p, p, None, 4, 65, p, None) == -1     # N > 64
    assert lib.spec_verify_telemetry_tree(p, None, p, None, 4, 8, p, None) == -1   # no paths
    assert lib.spec_verify_telemetry_summary(None, p, None) == -1
    assert lib.spec_verify_draft_topk(p, 1, 0, 100, 4, None, p, p, None) == 0        # empty
    assert lib.spec_verify_draft_topk(p, 1, 2, 100, 65, None, p, p, None) == -1      # k > 64
    assert lib.spec_verify_draft_topk(p, 1, 2, 3, 4, None, p, p, None) == -1         # k > V
    assert lib.spec_verify_draft_topk(p, 5, 2, 100, 4, None, p, p, None) == -1       # dtype
    prune = lib.spec_verify_tree_prune
    assert prune(p, p, p, None, 2, 1025, 64, ctypes.c_double(0.1), p, p, p, p, None, None) == -1
    assert prune(p, p, p, None, 2, 10, 65, ctypes.c_double(0.1), p, p, p, p, None, None) == -1
    assert prune(p, p, p, None, 2, 10, 64, ctypes.c_double(-1.0), p, p, p, p, None, None) == -1
    assert prune(p, p, p, None, 0, 10, 64, ctypes.c_double(0.1), p, p, p, p, None, None) == 0
    gu = lib.spec_verify_gamma_update
    assert gu(p, p, p, None, 1, 4, p, None, None) == -1     # coupling without temperatures
    assert gu(p, p, p, None, 0, 0, p, None, None) == 0      # empty
    assert lib.spec_verify_exp2(p, p, -1, None) == -1
    assert lib.spec_verify_exp2(None, p, 4, None) == -1
    assert lib.spec_verify_exp2(None, None, 0, None) == 0
    assert lib.spec_verify_philox_words(0, 0, None, 0, 5, None, None) == 0
    assert lib.spec_verify_philox_words(0, 0, None, 3, 5, None, None) == -1
    assert lib.spec_verify_philox_words(0, 0, None, 3, 5, ctypes.c_void_p(8), None) == -1


def test_noalloc_host_validation(lib):
    """The allocation-free linear verify refuses, before any launch, what the
    workspace entry point refuses, and requests beyond its static scratch."""
    import rejection_sampling_verify_04_amd as sv
    p = ctypes.c_void_p(256)
    call = lambda dtype, B, V, total, target=p: lib.spec_verify_linear_noalloc(
        target, p, dtype, B, V, total, p, p, p, p, 0, 0, None, p, p, None, None, None, None)
    assert call(7, 2, 100, 4) == -1                 # dtype
    assert call(1, 2, 100, 129) == -1               # some gamma_b > 64
    assert call(1, 0, 100, 0) == 0                  # empty batch: no-op
    assert call(1, 2, 100, 4, target=None) == -1
    assert call(1, 2, 64 * 8192 + 1, 4) == -2       # vocabulary beyond the chunk table
    need = lib.spec_verify_linear_workspace_size(4096, 4096 * 8, 152064, 1)
    assert need > sv.SV_STATIC_SCRATCH_BYTES
    assert call(1, 4096, 152064, 4096 * 8) == sv.SV_ERR_SCRATCH
    # the configurations it is for fit
    assert lib.spec_verify_linear_workspace_size(256, 1130, 152064, 1) <= sv.SV_STATIC_SCRATCH_BYTES
    assert lib.spec_verify_linear_workspace_size(128, 1024, 128256, 1) <= sv.SV_STATIC_SCRATCH_BYTES
