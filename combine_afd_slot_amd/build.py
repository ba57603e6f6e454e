"""Build libafd.so in-tree with hipcc for gfx950.

    python -m combine_afd_slot_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libafd.so")
SOURCES = ["afd_kernels.hip", "afd_host.cpp"]
ARCH = os.environ.get("AFD_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile every source and link libafd.so (always recompiles)."""
    out_tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}",
           "-x", "hip"] + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", out_tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
