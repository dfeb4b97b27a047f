"""The host-checked build: ABI layer under ASan/UBSan with launch-arithmetic checks.

hybrid_sparse_attention_flash_amd/build.py builds _build/checked/libhys_checked.so
with the host code under AddressSanitizer and UndefinedBehaviorSanitizer and
the ABI layer's launch-arithmetic checks enabled (-DHYS_DEBUG; device code is
compiled as usual and never runs here).  This test runs the CPU tests of the
ABI (tests/test_abi.py: validation and workspace queries) and the valid-call
sweep (tests/test_launch_configs.py: every entry point taken up to its
launch) against that library, in a subprocess that preloads the ASan runtime.
Any sanitizer report aborts the subprocess; any failed launch-arithmetic check
fails a test with HYS_ERR_INTERNAL.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "hybrid_sparse_attention_flash_amd"))
import build as hys_build  # noqa: E402


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _checked_lib():
    lib = hys_build.CHECKED_LIB
    newest = max(os.path.getmtime(f) for f in hys_build.sources())
    if not os.path.exists(lib) or os.path.getmtime(lib) < newest:
        hys_build.build(verbose=False, checked=True)
    return lib


@pytest.mark.skipif(_asan_runtime() is None, reason="no ASan runtime in this toolchain")
def test_abi_and_launch_configs_under_sanitizers():
    lib = _checked_lib()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": _asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1:detect_odr_violation=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "HYS_TEST_LIB": lib,
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_launch_configs.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert " passed" in out and "skipped" not in out, out[-2000:]
