"""Build librr.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

Run as ``python -m jagged_candidate_isolated_amd.build``; ``__graft_entry__.build()``
calls ``build()``.  Every call recompiles.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librr.so")
ARCH = "gfx950"

# Packed fp32 VALU instructions are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librr)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    out_tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}",
           *DEVICE_FLAGS, "-o", out_tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with status {r.returncode}")
    noise = [ln for ln in (r.stdout + r.stderr).splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln and "not a recognized feature" not in ln]
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
