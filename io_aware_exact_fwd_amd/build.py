"""Build libfa_mi355x.so (the HIP kernels and the C ABI) for gfx950.

    python -m io_aware_exact_fwd_amd.build            # libfa_mi355x.so
    python -m io_aware_exact_fwd_amd.build --debug    # libfa_mi355x_debug.so

Compiles every ``csrc/*.hip`` with hipcc for --offload-arch=gfx950 (in
parallel, objects under ``_build/``) and links the shared library next to this
file, where the binding loads it.  Cross-compiles without a GPU.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfa_mi355x.so")
# the debug build (include/fa_debug.h): NaN-filled LDS and tile-visit counters
LIB_DEBUG = os.path.join(HERE, "libfa_mi355x_debug.so")
ARCH = "gfx950"

# Packed-fp32 instructions are disabled for all device code.
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa_mi355x)")


def _compile(src: str, hipcc: str, build_dir: str, defines) -> str:
    obj = os.path.join(build_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc, *HIP_FLAGS, *[f"-D{d}" for d in defines], "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True, defines=(), out: str = LIB, debug: bool = False) -> str:
    """Compile and link; `defines` are extra preprocessor definitions passed
    to every source, `out` the library path; debug=True builds the debug
    library (FA_DEBUG_BUILD=1) as libfa_mi355x_debug.so."""
    hipcc = _hipcc()
    if debug:
        defines = (*defines, "FA_DEBUG_BUILD=1")
        out = LIB_DEBUG if out == LIB else out
    build_dir = BUILD if out == LIB else (BUILD + "_debug" if out == LIB_DEBUG else out + ".objs")
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    workers = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "8"))))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, build_dir, defines), srcs))
    tmp = out + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(debug="--debug" in sys.argv[1:])
    sys.exit(0)
