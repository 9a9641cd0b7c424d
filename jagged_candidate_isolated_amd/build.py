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
# Per-file flags.  The MFMA attention kernel never forms a NaN, so it is compiled
# without NaN support: max chains then map to v_max3_f32 with no canonicalisation.
FILE_FLAGS = {"attn_mfma.hip": ["-fno-honor-nans"]}
BUILD_DIR = os.path.join(ROOT, "_build")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librr)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
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


# The forward attention kernels' device code: the digest of their gfx950 assembly is built
# into the library (rr_forward_fingerprint), so measurements taken on one build can be
# matched to another with the same machine code.
FINGERPRINT_SOURCES = ("attn_mfma.hip",)


def _fingerprint_source(common, verbose) -> str:
    import hashlib
    h = hashlib.sha256()
    for name in FINGERPRINT_SOURCES:
        src = os.path.join(CSRC, name)
        asm = os.path.join(BUILD_DIR, name + ".s")
        _run(common + FILE_FLAGS.get(name, []) + ["--cuda-device-only", "-S", src, "-o", asm], verbose)
        with open(asm, encoding="utf-8", errors="replace") as f:
            for line in f:
                # compilation-unit ids and file/tool stamps differ between otherwise equal builds
                if "__hip_cuid" in line or line.lstrip().startswith((".file", ".ident")):
                    continue
                h.update(line.encode())
    out = os.path.join(BUILD_DIR, "rr_fingerprint.cpp")
    with open(out, "w", encoding="utf-8") as f:
        f.write('extern "C" const char* rr_forward_fingerprint(void) { return "%s"; }\n' % h.hexdigest()[:16])
    return out


def build(verbose: bool = False) -> str:
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD_DIR, exist_ok=True)
    common = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
              "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}", *DEVICE_FLAGS]
    jobs = []
    for src in sources():
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        jobs.append((common + FILE_FLAGS.get(os.path.basename(src), []) + ["-c", src, "-o", obj], obj))
    fp = _fingerprint_source(common, verbose)
    fp_obj = os.path.join(BUILD_DIR, "rr_fingerprint.o")
    jobs.append(([hipcc(), "-O2", "-fPIC", "-c", "-x", "c++", fp, "-o", fp_obj], fp_obj))
    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        list(ex.map(lambda j: _run(j[0], verbose), jobs))
    out_tmp = LIB + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp] + [o for _, o in jobs],
         verbose)
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
