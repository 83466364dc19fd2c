"""Build the host-only sanitizer check of the C ABI (tests/abi_sanitize).

    python tests/abi_sanitize/build_check.py

Compiles io_aware_exact_fwd_amd/csrc/fa_api.hip (the argument checks,
workspace layout and dispatch of include/fa.h) together with stand-in kernel
launchers and the fuzz driver, host code only, with AddressSanitizer and
UndefinedBehaviorSanitizer (every sanitizer flag is given through -Xarch_host,
so no device code is instrumented), into io_aware_exact_fwd_amd/_build/abi_fuzz.
tests/test_abi_sanitize.py runs it on the CPU.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(ROOT, "io_aware_exact_fwd_amd", "_build", "abi_fuzz")

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = True) -> str:
    hipcc = _hipcc()
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    objs = []
    srcs = [os.path.join(ROOT, "io_aware_exact_fwd_amd", "csrc", "fa_api.hip"),
            os.path.join(HERE, "launch_stubs.cpp"), os.path.join(HERE, "abi_fuzz.cpp")]
    for src in srcs:
        obj = os.path.join(os.path.dirname(OUT), "abi_fuzz_" + os.path.basename(src) + ".o")
        lang = [] if src.endswith(".hip") else ["-x", "hip"]
        cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *SAN, *lang, "-c", src,
               "-o", obj, "-Wno-unused-command-line-argument"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        objs.append(obj)
    cmd = [hipcc, "--offload-arch=gfx950", *SAN, *objs, "-o", OUT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
