"""Loading of liblowbit.so and its C signatures.  There is no fallback: if the library is
not built, every call raises."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

# Entry points declared in include/lowbit.h, with (restype, argtypes).
_VP, _I64, _INT = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
SIGNATURES = {
    "lowbit_pack": (_INT, [_VP, _VP, _I64, _I64, _INT, _VP, _VP]),
    "lowbit_unpack": (_INT, [_VP, _VP, _I64, _I64, _INT, _VP]),
    "lowbit_pack_u4": (_INT, [_VP, _VP, _I64, _I64, _VP, _VP]),
    "lowbit_gemm_affine": (_INT, [_VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _INT, _VP]),
    "lowbit_affine_workspace_size": (ctypes.c_size_t, [_I64, _I64, _I64, _INT]),
    "lowbit_gemm_affine_ex": (_INT, [_VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _INT, _VP, ctypes.c_size_t, _VP]),
    "lowbit_import_ternary": (_INT, [_VP, _INT, _INT, _VP, _I64, _I64, _VP, _VP]),
    "lowbit_import_binary_gemlite": (_INT, [_VP, _VP, _I64, _I64, _VP]),
    "lowbit_gemm": (_INT, [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _INT, _INT, _VP]),
    "lowbit_gemm_batched": (_INT, [_VP, _INT, _VP]),
    "lowbit_gemm_swiglu": (_INT, [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _INT, _INT, _VP]),
    "lowbit_gemm_residual": (_INT, [_VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _INT, _INT, _VP]),
    "lowbit_workspace_size": (ctypes.c_size_t, [_I64, _I64, _I64, _INT, _INT]),
    "lowbit_gemm_ex": (_INT, [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _INT, _INT, _VP, ctypes.c_size_t, _VP]),
    "lowbit_gemm_noalloc": (_INT, [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _INT, _INT, _VP]),
    "lowbit_batched_workspace_size": (ctypes.c_size_t, [_VP, _INT]),
    "lowbit_gemm_batched_ex": (_INT, [_VP, _INT, _VP, ctypes.c_size_t, _VP]),
    "lowbit_check_gemm_args": (_INT, [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _INT, _INT]),
    "lowbit_gemm_variant": (ctypes.c_char_p, [_I64, _I64, _I64, _INT, _INT]),
    "lowbit_status_string": (ctypes.c_char_p, [_INT]),
    "lowbit_last_hip_error": (_INT, []),
    "lowbit_device_supported": (_INT, [_INT]),
    "lowbit_version": (_INT, []),
}


class LowbitError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def library_path() -> str:
    return os.environ.get("LOWBIT_LIBRARY") or os.path.join(_HERE, "liblowbit.so")


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"liblowbit.so not found at {path}: build it with "
                               "`python -m binary_bit_gemm_amd.build` (there is no CPU fallback)")
        L = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB
