"""MI355X (gfx950) Mamba-2 chunked-SSD forward.

The computation lives in ``libmamba_ssd.so`` (hand-written HIP kernels behind
the C ABI of ``include/ssd.h``); this package holds its build script, a ctypes
binding with the ABI's names (``ops``) and the seeded input recipe
(``inputs``).  Build with ``python -m mamba_ssd_scan_chunk_amd.build``.
"""
from ._lib import LIB_PATH, SSDError, SSDShape, load_library  # noqa: F401

__all__ = ["LIB_PATH", "SSDError", "SSDShape", "load_library"]
