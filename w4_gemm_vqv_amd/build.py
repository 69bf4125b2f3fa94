"""Build libvqv.so in-tree for gfx950 with hipcc.

    python -m w4_gemm_vqv_amd.build

The library is compiled as one shared object from the HIP sources in csrc/.
Packed fp32 instructions are disabled for the device pass; hipcc's host pass
warns that it does not know that feature, which is harmless.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["vqv_api.hip", "qgemm.hip", "qgemm_m16.hip", "verify.hip"]
LIB = os.path.join(PKG, "libvqv.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libvqv)")


def command(out: str) -> list[str]:
    return [hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-command-line-argument",
            *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def build(verbose: bool = True) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in r.stderr.splitlines() if "is not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError("libvqv build failed:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
