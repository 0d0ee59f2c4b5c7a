"""Build libdflash.so (the drafter's HIP kernels + host runtime) for gfx950 with hipcc.

    python -m block_diffusion_draft_02_amd.build        # or build() from Python

Objects go to _build/ at the repository root; the shared library lands next to this file.
build_host_check() also links tests/host/abi_check: the runtime's host code compiled with
AddressSanitizer and UndefinedBehaviorSanitizer (the host pass only), the library's kernel
objects as they are, and a driver that calls every entry point.
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


HOST_CHECK_DIR = os.path.join(ROOT, "tests", "host")
HOST_CHECK = os.path.join(HOST_CHECK_DIR, "abi_check")
# sanitizers for the host compilation pass only (device code is built as in the library)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
LINK_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def clangxx() -> str:
    for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("amdclang++")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("clang++ of the ROCm toolchain not found")


def _run(cmd, what):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{what} failed: {' '.join(cmd)}\n{_quiet(r.stdout + r.stderr)}")


def build_host_check(verbose: bool = True) -> str:
    os.makedirs(os.path.join(BUILD, "san"), exist_ok=True)
    kernels = [s for s in SOURCES if s != "runtime.hip"]
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in kernels]
    if not all(os.path.exists(o) for o in objs):
        with cf.ThreadPoolExecutor(max_workers=min(8, len(kernels))) as ex:
            objs = list(ex.map(_compile, kernels))
    rt = os.path.join(BUILD, "san", "runtime.o")
    _run([hipcc(), *FLAGS, "-O1", "-g", *HOST_SAN, "-c", os.path.join(CSRC, "runtime.hip"), "-o", rt],
         "sanitized runtime compile")
    drv = os.path.join(BUILD, "san", "abi_check.o")
    _run([clangxx(), "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", *LINK_SAN, "-D__HIP_PLATFORM_AMD__",
          "-Wno-c++20-extensions", "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
          os.path.join(HOST_CHECK_DIR, "abi_check.cpp"), "-o", drv], "host check compile")
    tmp = HOST_CHECK + ".tmp"
    _run([clangxx(), *LINK_SAN, "-o", tmp, drv, rt, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib"], "host check link")
    os.replace(tmp, HOST_CHECK)
    if verbose:
        print(f"built {HOST_CHECK}")
    return HOST_CHECK


if __name__ == "__main__":
    build()
    if "--host-check" in sys.argv:
        build_host_check()
