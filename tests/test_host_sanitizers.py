"""The runtime's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/host/abi_check is the library's kernel objects linked with a copy of the host runtime
compiled with both sanitizers (host pass only) and a driver that calls every entry point of
dflash.h (block_diffusion_draft_02_amd/build.py, build_host_check). Any invalid host access,
leak of the runtime's own allocations or undefined operation ends the run with a report.

  * without a device: every configuration refusal, the NULL-handle paths, and create's
    unwind when no device can be used;
  * on the GPU: bf16 (YaRN, a window, the LDS attention path), FP8, Markov-head and DFlash2
    drafters through appends, batched appends, forwards at gamma 16, 5 and 2 (each band bit
    for bit equal alone, the no-allocation forward bit for bit equal), the capture seam,
    timing, resets, pool exhaustion and every argument refusal, which must leave every
    sequence's state unchanged."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
BIN = os.path.join(HOST, "abi_check")


def _env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1:abort_on_error=0:verify_asan_link_order=0"
    env["LSAN_OPTIONS"] = "suppressions=" + os.path.join(HOST, "lsan.supp")
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def _run(mode, timeout):
    r = subprocess.run([BIN, mode], capture_output=True, text=True, timeout=timeout, env=_env(), cwd=HOST)
    print(r.stdout[-4000:], r.stderr[-8000:])
    assert r.returncode == 0, f"abi_check {mode} exited {r.returncode}"
    assert f"abi_check {mode} ok" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr


def test_host_runtime_sanitized_without_device():
    if not os.path.exists(BIN):
        from block_diffusion_draft_02_amd import build as b
        b.build_host_check()
    _run("cpu", 120)


@pytest.mark.gpu
def test_host_runtime_sanitized_on_gpu():
    assert os.path.exists(BIN), "tests/host/abi_check is not built (block_diffusion_draft_02_amd.build.build_host_check)"
    _run("gpu", 200)
