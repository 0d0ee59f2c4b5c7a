"""DFlash block-diffusion drafter, gamma-block forward, for AMD Instinct MI355X (gfx950).

The compute path is libdflash.so (hand-written HIP kernels + a C++ runtime behind the C ABI
in include/dflash.h); `binding` is its ctypes binding.
"""
from .binding import Drafter, DflashError, lib  # noqa: F401
