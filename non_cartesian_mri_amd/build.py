"""Build the gfx950 HIP library libncmri_fhd.so in-tree with hipcc.

Usage: python -m non_cartesian_mri_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libncmri_fhd.so")
SOURCES = ["fhd_kernels.hip", "fhd_mfma.hip", "fhd_half.hip", "fhd_forward.hip", "fhd_forward_half.hip", "fhd_lines.hip", "fhd_cg.hip",
           "fhd_grid.hip", "fhd_api.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # no contraction: every fused multiply-add in the kernels is written out
    "-ffp-contract=off",
    # keep the compiler from emitting packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def build_library(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link the shared library (always rebuilds)."""
    hipcc = _hipcc()
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, src + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        if verbose:
            print(" ".join(cmd))
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


ISSUE_RATES = os.path.join(PKG, "issue_rates")


def build_issue_rates() -> str:
    """Compile the standalone issue-rate microbenchmark (csrc/issue_rates.hip)."""
    tmp = ISSUE_RATES + f".tmp{os.getpid()}"
    cmd = [_hipcc(), *HIPCC_FLAGS, os.path.join(CSRC, "issue_rates.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for issue_rates.hip:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, ISSUE_RATES)
    return ISSUE_RATES


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
    print(build_issue_rates())
