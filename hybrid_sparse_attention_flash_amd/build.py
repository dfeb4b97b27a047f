"""Build libhys.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Every source under csrc/ is compiled by hipcc to an object in _build/ (in
parallel), then linked into hybrid_sparse_attention_flash_amd/libhys.so.

build(checked=True) makes the host-checked variant instead,
_build/checked/libhys_checked.so: the host code under AddressSanitizer and
UndefinedBehaviorSanitizer (device code is compiled as usual) and the ABI
layer's launch-arithmetic checks enabled (-DHYS_DEBUG).  It is for CPU-side
test runs that preload the ASan runtime; it is never the product library.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libhys.so")
ARCH = os.environ.get("HYS_OFFLOAD_ARCH", "gfx950")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.exists(c) or c == "hipcc":
            return c


# host-only sanitizers: each -fsanitize= goes to the host compilation alone
CHECKED_FLAGS = [
    "-DHYS_DEBUG",
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
]
CHECKED_DIR = os.path.join(BUILD, "checked")
CHECKED_LIB = os.path.join(CHECKED_DIR, "libhys_checked.so")


def _compile(src, out_dir=BUILD, extra=()):
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *CFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-4000:]}")
    return obj


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")) +
                  [os.path.join(os.path.dirname(HERE), "include", "hys.h")])


def build(verbose: bool = True, checked: bool = False) -> str:
    out_dir, lib, extra = (CHECKED_DIR, CHECKED_LIB, CHECKED_FLAGS) if checked else (BUILD, LIB, [])
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, out_dir, extra), srcs))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources")
    return lib


if __name__ == "__main__":
    build(checked="--checked" in sys.argv[1:])
    sys.exit(0)
