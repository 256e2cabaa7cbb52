"""ctypes view of libsharq.so (the C ABI declared in include/sharq.h).

Only argument marshalling lives here. Every step of the hot path runs in the
HIP library; if the library cannot be loaded, loading fails loudly.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsharq.so")

SHARQ_OK = 0
SHARQ_EINVAL = -1
SHARQ_EALIGN = -2
SHARQ_EUNSUPPORTED = -3
SHARQ_EHIP = -4
SHARQ_ENOTIMPL = -5
SHARQ_ESCRATCH = -6
SCRATCHFREE_MAX_BYTES = 32 << 20  # SHARQ_SCRATCHFREE_MAX_BYTES

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int

# name -> (restype, argtypes); mirrors include/sharq.h
SIGNATURES = {
    "sharq_status_string": (ctypes.c_char_p, [_INT]),
    "sharq_abi_version": (_INT, []),
    "sharq_prepare": (_INT, [_P, _I64, _I64, _I64, _P, _INT, _INT, _P, _P, _P, _P, _P, _P]),
    "sharq_prepare_rms": (_INT, [_P, _I64, _I64, _I64, _P, ctypes.c_float, _INT, _INT, _P, _P, _P, _P, _P, _P,
                                 _P]),
    "sharq_quantize_mxfp4": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "sharq_pack_stage_major": (_INT, [_P, _P, _I64, _I64, _INT, _P, _P, _P]),
    "sharq_unpack_stage_major": (_INT, [_P, _P, _I64, _I64, _INT, _P, _P, _P]),
    "sharq_prepare_nvfp4": (_INT, [_P, _I64, _I64, _I64, _P, _INT, _INT, ctypes.c_float, _P, _P, _P, _P, _P, _P]),
    "sharq_quantize_nvfp4": (_INT, [_P, _I64, _I64, _I64, ctypes.c_float, _P, _P, _P]),
    "sharq_linear_nvfp4": (_INT, [_P, _P, _P, _P, ctypes.c_float, _P, _P, ctypes.c_float, _I64, _I64, _I64, _P,
                                  _I64, _P]),
    "sharq_linear": (_INT, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P]),
    "sharq_linear_workspace_bytes": (_I64, [_I64, _I64, _I64]),
    "sharq_linear_silu_prepare_workspace_bytes": (_I64, [_I64, _I64, _I64]),
    "sharq_linear_scratchfree": (_INT, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P]),
    "sharq_linear_ws": (_INT, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P]),
    "sharq_linear_grouped": (_INT, [_P, _P, _P, _P, _I64, _P, _P, ctypes.c_int32, _P, _P, _I64, _I64, _I64, _P,
                                    _P]),
    "sharq_linear_silu_prepare": (_INT, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _INT, _INT, _P, _P, _P, _P,
                                         _P, _P, _P]),
    "sharq_linear_silu_prepare_ws": (_INT, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _INT, _INT, _P, _P, _P, _P,
                                            _P, _P, _P, _I64, _P]),
    "sharq_linear_grouped_silu_prepare": (_INT, [_P, _P, _P, _P, _I64, _P, _P, ctypes.c_int32, _P, _P, _I64, _I64,
                                                 _I64, _INT, _INT, _P, _P, _P, _P, _P, _P, _P]),
    "sharq_backbone_meta_row_bytes": (_I64, [_I64, _INT, _INT]),
    "sharq_compress_backbone": (_INT, [_P, _P, _I64, _I64, _INT, _INT, _P, _P, _P]),
    "sharq_expand_backbone": (_INT, [_P, _P, _I64, _I64, _INT, _INT, _P, _P, _P]),
    "sharq_moe_combine": (_INT, [_P, _I64, _I64, _P, _P, _I64, ctypes.c_int32, _P, _P, _P]),
    "sharq_silu_mul": (_INT, [_P, _I64, _I64, _P, _P]),
}

_lib = None


class SharqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Load libsharq.so once. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m activation_sparsity_fp4_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().sharq_status_string(status).decode()


def check(fn: str, status: int) -> None:
    if status != SHARQ_OK:
        raise SharqError(fn, status)


def call(name: str, *args) -> int:
    """Call an ABI entry point with raw integers (device addresses) and return its status."""
    return getattr(lib(), name)(*args)
