"""Build libspecverify.so (the verify kernels and their C ABI) for gfx950 with hipcc.

Usage: python -m rejection_sampling_verify_04_amd.build  (or build() from Python).
The library is written next to this file so that it travels with the tree.
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspecverify.so")
SOURCES = ["sv_api.hip", "sv_stats.hip", "sv_linear.hip", "sv_tree.hip", "sv_attn.hip",
           "sv_kv.hip", "sv_telemetry.hip", "sv_control.hip",
           "sv_draft.hip"]
HEADERS = ["sv_common.h", "sv_internal.h", "sv_finish.h"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc_path():
    p = shutil.which("hipcc")
    if p:
        return p
    p = "/opt/rocm/bin/hipcc"
    if os.path.exists(p):
        return p
    raise RuntimeError("hipcc not found: the verify library cannot be built")


def build(verbose=False):
    """Compile every source into LIB (always recompiles)."""
    cmd = [hipcc_path(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
