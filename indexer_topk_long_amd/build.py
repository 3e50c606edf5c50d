"""Build the gfx950 HIP libraries in-tree: indexer_topk_long_amd/_lib/liblitetopk.so (the
fused Indexer-TopK) and indexer_topk_long_amd/_lib/libltkpeak.so (the achievable-peak
microbenchmarks the benchmark reports beside the vendor peaks).

    python -m indexer_topk_long_amd.build [-v]
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_lib")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "liblitetopk.so"
PEAK_SRC = os.path.join(PKG, "peak", "peak.hip")
PEAK_LIB = "libltkpeak.so"
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    # packed fp32 VALU forms stay off: scalar fp32 only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def lib_path() -> str:
    return os.path.join(OUT_DIR, LIB_NAME)


def peak_lib_path() -> str:
    return os.path.join(OUT_DIR, PEAK_LIB)


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if verbose and msg.strip():
        print(msg)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link the shared library. Returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs) + 1, 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs + [PEAK_SRC]))
    peak_obj = objs.pop()
    for out, inputs in ((lib_path(), objs), (peak_lib_path(), [peak_obj])):
        tmp = out + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *inputs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
        os.replace(tmp, out)
    return lib_path()


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
