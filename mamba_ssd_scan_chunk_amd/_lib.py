"""ctypes binding of ``libmamba_ssd.so`` (the C ABI in ``include/ssd.h``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  Torch tensors serve as device buffers and torch's
current stream as the launch stream.  There is no fallback: when the library
is missing or the tensors are not on the GPU, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmamba_ssd.so")

SSD_OK = 0
STATUS_NAMES = {0: "SSD_OK", 1: "SSD_ERR_NULL", 2: "SSD_ERR_SHAPE", 3: "SSD_ERR_DTYPE",
                4: "SSD_ERR_UNSUPPORTED", 5: "SSD_ERR_WORKSPACE", 6: "SSD_ERR_ALIGN", 7: "SSD_ERR_HIP",
                8: "SSD_ERR_SCRATCH"}
SSD_F32, SSD_BF16 = 0, 1
SSD_MMA_BF16, SSD_MMA_F32 = 0, 1
MMA = {"bf16": SSD_MMA_BF16, "f32": SSD_MMA_F32}


class SSDShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk", ctypes.c_int64)]

    @classmethod
    def make(cls, batch, seqlen, nheads, headdim, dstate, ngroups, chunk) -> "SSDShape":
        return cls(batch, seqlen, nheads, headdim, dstate, ngroups, chunk)

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


_P = ctypes.c_void_p
_S = ctypes.POINTER(SSDShape)
_E = ctypes.c_int  # enums

_SIGNATURES = {
    "ssd_chunk_cumsum": (ctypes.c_int, [_S, _P, _P, _P, _P, _P]),
    "ssd_chunk_state": (ctypes.c_int, [_S, _P, _P, _E, _P, _P, _P, _E, _E, _P]),
    "ssd_chunk_cumsum_state": (ctypes.c_int, [_S, _P, _P, _E, _P, _P, _P, _P, _P, _E, _E, _P]),
    "ssd_state_passing": (ctypes.c_int, [_S, _P, _E, _P, _E, _P, _P, _P, _P]),
    "ssd_chunk_scan": (ctypes.c_int, [_S, _P, _P, _P, _E, _P, _P, _P, _E, _P, _P, _E, _E, _P]),
    "ssd_chunk_state_passing": (ctypes.c_int, [_S, _P, _P, _E, _P, _P, _P, _P, _E, _P, _E, _P]),
    "ssd_decode_step": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _E, _P, _P, _E, _P]),
    "ssd_workspace_bytes": (ctypes.c_size_t, [_S]),
    "ssd_workspace_bytes_varlen": (ctypes.c_size_t, [_S]),
    "ssd_forward_varlen": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _E, _P, _P, _P, _E, _P, ctypes.c_int64, _P, _P,
                                          _P, ctypes.c_size_t, _E, _P]),
    "ssd_forward": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _E, _P, _P, _E, _P, _P, ctypes.c_size_t, _E, _P]),
    "ssd_forward_noalloc": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _E, _P, _P, _E, _P, _E, _P]),
    "ssd_backward": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _E, _P, _P, _E, _P, _P, _P, _P, _P, _P, _P, _P,
                                    _P, ctypes.c_size_t, _E, _P]),
    "ssd_backward_workspace_bytes": (ctypes.c_size_t, [_S]),
    "ssd_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ssd_abi_version": (ctypes.c_int, []),
}

_LIB: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _LIB
    if _LIB is not None and path == LIB_PATH:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path}; run `python -m mamba_ssd_scan_chunk_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _LIB = lib
    return lib


class SSDError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


def check(code: int) -> None:
    if code != SSD_OK:
        lib = load_library()
        raise SSDError(code, lib.ssd_status_string(code).decode())
