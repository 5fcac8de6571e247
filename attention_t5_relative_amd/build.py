"""Build libfat5attn.so for gfx950 in-tree with hipcc.

    python -m attention_t5_relative_amd.build [--jobs N] [--debug]

Every source under csrc/ is compiled to an object in _build/ (in parallel),
then linked into attention_t5_relative_amd/libfat5attn.so.  hipcc
cross-compiles, so no GPU is needed.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfat5attn.so")
ARCH = "gfx950"

# Packed fp32 VALU forms are kept out of the device code.  Device code is
# also built without NaN semantics: the kernels never produce or consume NaN
# (masked scores are -inf, which keeps its meaning), and IEEE NaN handling
# would put a canonicalising max in front of every fmaxf of the softmax.
# Host code (the argument checks in api.cpp) keeps full IEEE semantics.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Xarch_device", "-fno-honor-nans"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfat5attn)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str, debug: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-c", src, "-o", obj, "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
           "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"] + DEVICE_FLAGS
    cmd += ["-O1", "-g"] if debug else ["-O3"]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, debug: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, debug), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--debug", action="store_true")
    a = ap.parse_args(argv)
    build(a.jobs, a.debug, verbose=True)


if __name__ == "__main__":
    sys.exit(main())
