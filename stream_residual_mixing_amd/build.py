"""Build libhc.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m stream_residual_mixing_amd.build

compiles every source under csrc/ with hipcc into stream_residual_mixing_amd/libhc.so.
hipcc cross-compiles for gfx950 without a GPU present.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhc.so")
ARCH = "gfx950"

# Packed fp32 VALU instructions are disabled for every HIP file; hipcc's host
# pass warns that it does not know this target feature, which is harmless.
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: cannot build libhc for gfx950")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile all HIP sources and link libhc.so; returns its path."""
    cc = hipcc()
    objs = []
    with tempfile.TemporaryDirectory(prefix="hcbuild_") as tmp:
        procs = []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [cc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
            if len(procs) >= jobs:
                _wait(procs.pop(0), verbose)
        for p in procs:
            _wait(p, verbose)
        tmp_lib = LIB + ".tmp"
        cmd = [cc, *HIP_FLAGS, "-shared", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if out.returncode != 0:
            raise RuntimeError(f"link of libhc.so failed:\n{out.stdout}")
        os.replace(tmp_lib, LIB)
    return LIB


def _wait(item, verbose):
    src, proc = item
    out, _ = proc.communicate()
    text = out.decode(errors="replace")
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{text}")
    if verbose and text.strip():
        print(text, flush=True)


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
