"""Build libdflash.so (the drafter's HIP kernels + host runtime) for gfx950 with hipcc.

    python -m block_diffusion_draft_02_amd.build        # or build() from Python

Objects go to _build/ at the repository root; the shared library lands next to this file.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdflash.so")
SOURCES = ["k_gemm.hip", "k_gemm_wide.hip", "k_gemm_tiled.hip", "k_attn.hip", "k_misc.hip", "k_markov.hip", "k_dflash2.hip", "runtime.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _quiet(text: str) -> str:
    # the host pass does not know the packed-fp32 feature and says so once per file
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = _quiet(r.stdout + r.stderr).strip()
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{msg}")
    if msg:
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    # -z defs: a symbol no object defines fails the link, not the first load
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{_quiet(r.stdout + r.stderr)}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
