"""1-bit Adam compression-phase step on AMD Instinct MI355X (gfx950).

The kernels and the C ABI live in libob.so (sources in csrc/, declarations in
include/ob.h at the repository root); binding.py is a thin ctypes layer over
it.  Build with ``python -m error_compensated_bit_02_amd.build``.
"""
from .binding import OneBitAdam, OneBitError, layout, load_library  # noqa: F401

__all__ = ["OneBitAdam", "OneBitError", "layout", "load_library"]
