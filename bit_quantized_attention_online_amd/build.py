"""Build libqk4v8.so (all HIP sources, gfx950 only) in-tree with hipcc.

Usage: python -m bit_quantized_attention_online_amd.build  (or build()).
Objects go to <repo>/_build/, the library to this package's directory, where
``ops`` loads it from.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqk4v8.so")
SOURCES = ["qk4v8_api.hip", "quantize.hip", "prefill.hip", "decode.hip", "append.hip"]
# the peak microbenchmarks (include/qk4v8_peaks.h) are a library of their own
PEAKS_LIB = os.path.join(PKG, "libqk4v8_peaks.so")
PEAKS_SOURCES = ["peaks.hip"]
ARCH = "gfx950"


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def flags():
    return [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
            "-I", os.path.join(ROOT, "include"),
            # NaN inputs are outside the contract: lets max/min skip IEEE quieting
            "-fno-honor-nans",
            # packed FP32 VALU instructions are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    return obj, msgs


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def build(verbose=False):
    """Compile every HIP source for gfx950 and link libqk4v8.so and
    libqk4v8_peaks.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        results = list(ex.map(_compile, SOURCES + PEAKS_SOURCES))
    for _, msgs in results:
        if verbose and msgs.strip():
            print(msgs, file=sys.stderr)
    _link([o for o, _ in results[:len(SOURCES)]], LIB)
    _link([o for o, _ in results[len(SOURCES):]], PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
