"""Build libparallax.so (HIP for gfx950) in-tree with hipcc.

    python -m parallax_covariance_corrected_amd.build [--verbose]

Every call recompiles all sources (cross-compiles without a GPU). The library
lands next to this file, where the ctypes binding loads it from.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libparallax.so")
SOURCES = ["api.hip", "decode_mfma.hip", "decode_generic.hip", "merge.hip", "probe.hip",
           "prefill_mfma.hip", "readbench.hip"]

ARCH = "gfx950"
# Packed-fp32 VALU forms are disabled: the compiler would otherwise emit them
# from plain float code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form",
             # leading scalar kernel arguments arrive in SGPRs (no argument load)
             "-mllvm", "-amdgpu-kernarg-preload-count=14",
             "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libparallax)")


def _compile(src: str, obj: str, verbose: bool) -> str:
    cmd = [hipcc(), *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; drop that line
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libparallax.so; return its path."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        for s in SOURCES:
            src = os.path.join(CSRC, s)
            obj = os.path.join(objdir, s.replace(".hip", ".o"))
            jobs.append(ex.submit(_compile, src, obj, verbose))
        objs = [j.result() for j in jobs]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
