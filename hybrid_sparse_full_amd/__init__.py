"""MI355X-native hybrid-head prefill attention (Elastic Attention).

The computation lives in libea.so (HIP kernels for gfx950 behind the C ABI
of include/ea.h).  This package holds the build script, the ctypes binding
(`ea`) and the device-memory plumbing (`layer`).
"""

from . import ea  # noqa: F401

__all__ = ["ea"]
