"""The C ABI's host-side validation under the host sanitizers, without a GPU.

`tests/helpers/abi_host_check.cpp` drives every entry point's argument checks,
the workspace-size queries and the per-thread timing hook from eight threads
at once, with extreme sizes (INT_MAX, LLONG_MAX) that must be rejected before
any launch.  It is built with the library sources twice: with AddressSanitizer
and UndefinedBehaviorSanitizer (out-of-bounds access, signed overflow in the
size arithmetic), and with ThreadSanitizer (data races between host threads).
Only host code is instrumented: each sanitizer flag is passed to the host pass
alone, and the device code is built as in the library.
"""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rejection_sampling_verify_04_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "helpers", "abi_host_check.cpp")
OUT = os.path.join(ROOT, "tests", "helpers", "_build")

VARIANTS = {
    "asan_ubsan": ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-sanitize-recover=all",
                   "-Xarch_host", "-fno-omit-frame-pointer"],
    "tsan": ["-Xarch_host", "-fsanitize=thread"],
}


def _hipcc():
    from rejection_sampling_verify_04_amd import build
    try:
        return build.hipcc_path()
    except RuntimeError:
        pytest.skip("hipcc not available")


@pytest.fixture(scope="module")
def binaries():
    from rejection_sampling_verify_04_amd import build
    hipcc = _hipcc()
    os.makedirs(OUT, exist_ok=True)
    sources = [os.path.join(CSRC, s) for s in build.SOURCES]
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC", "-O3")]
    procs = {}
    for name, san in VARIANTS.items():
        exe = os.path.join(OUT, "abi_host_check_" + name)
        cmd = [hipcc, "-O1", "-g", *flags, *san, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               *sources, DRIVER, "-o", exe, "-lpthread"]
        procs[name] = (exe, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                             text=True))
    out = {}
    for name, (exe, p) in procs.items():
        log, _ = p.communicate(timeout=600)
        assert p.returncode == 0, "%s build failed:\n%s" % (name, log[-4000:])
        out[name] = exe
    return out


@pytest.mark.parametrize("variant", sorted(VARIANTS))
def test_abi_validation_under_sanitizers(binaries, variant):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["TSAN_OPTIONS"] = "halt_on_error=1"
    res = subprocess.run([binaries[variant]], capture_output=True, text=True, timeout=300, env=env)
    text = res.stdout + res.stderr
    assert res.returncode == 0, text[-4000:]
    assert "abi host check ok" in res.stdout
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "WARNING: ThreadSanitizer"):
        assert marker not in text, text[-4000:]
