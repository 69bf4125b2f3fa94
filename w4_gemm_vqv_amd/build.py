"""Build libvqv.so in-tree for gfx950 with hipcc.

    python -m w4_gemm_vqv_amd.build

The HIP sources in csrc/ are compiled to objects in parallel and linked into
one shared object.
Packed fp32 instructions are disabled for the device pass; hipcc's host pass
warns that it does not know that feature, which is harmless.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["vqv_api.hip", "qgemm.hip", "qgemm_m8.hip", "qgemm_m16.hip", "qgemm_v.hip",
           "verify.hip"]
LIB = os.path.join(PKG, "libvqv.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libvqv)")


def flags() -> list[str]:
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-command-line-argument"]


def _run(cmd: list[str]) -> tuple[int, list[str]]:
    r = subprocess.run(cmd, capture_output=True, text=True)
    return r.returncode, [ln for ln in r.stderr.splitlines()
                          if "is not a recognized feature" not in ln]


def build(verbose: bool = True) -> str:
    """Compile every source to an object (in parallel), then link the shared
    library; the previous library is replaced only when both steps succeed."""
    objdir = tempfile.mkdtemp(prefix="vqv_build_")
    try:
        objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
        cmds = [[hipcc(), *flags(), "-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
            results = list(ex.map(_run, cmds))
        errs = [ln for _, e in results for ln in e]
        if any(rc != 0 for rc, _ in results):
            raise RuntimeError("libvqv build failed:\n" + "\n".join(errs))
        tmp = LIB + ".tmp"
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        rc, lerrs = _run(link)
        if rc != 0:
            raise RuntimeError("libvqv link failed:\n" + "\n".join(lerrs))
        if verbose and (errs or lerrs):
            print("\n".join(errs + lerrs), file=sys.stderr)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build())
