"""ctypes loader for libgptq_mi355x.so (argument marshalling only; no compute happens here)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgptq_mi355x.so")

GPTQ_OK = 0
GPTQ_ERR_INVALID_ARG = -1
GPTQ_ERR_UNSUPPORTED = -2
GPTQ_ERR_NOT_SPD = -3
GPTQ_ERR_NONFINITE = -4
GPTQ_ERR_WORKSPACE = -5
GPTQ_ERR_HIP = -6

GPTQ_F32 = 0
GPTQ_BF16 = 1

GPTQ_FACTOR_REVERSED = 0  # the default route
GPTQ_FACTOR_INVERSE_RECHOL = 1
GPTQ_FACTOR_R_FORM = 2  # R = U^-1 and U's 128 x 128 diagonal blocks, for gptq_quantize_layer_r

GPTQ_GRID_SYMMETRIC = 0
GPTQ_GRID_ASYMMETRIC = 1

# every symbol the header declares, with its ctypes signature
_c_int64 = ctypes.c_int64
_vp = ctypes.c_void_p
SIGNATURES = {
    "gptq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "gptq_version": (ctypes.c_char_p, []),
    "gptq_hessian_workspace_bytes": (ctypes.c_size_t, [_c_int64, _c_int64, ctypes.c_int]),
    "gptq_hessian_accumulate": (ctypes.c_int, [_vp, ctypes.c_int, _c_int64, _c_int64, _c_int64, _vp, _vp,
                                               ctypes.POINTER(_c_int64), _vp, ctypes.c_size_t, _vp]),
    "gptq_prepare_workspace_bytes": (ctypes.c_size_t, [_c_int64]),
    "gptq_prepare_chol": (ctypes.c_int, [_vp, _vp, _c_int64, _c_int64, ctypes.c_double, ctypes.c_int,
                                         ctypes.c_uint, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "gptq_quantize_workspace_bytes": (ctypes.c_size_t, [_c_int64, _c_int64]),
    "gptq_quantize_r_workspace_bytes": (ctypes.c_size_t, [_c_int64, _c_int64]),
    "gptq_quantize_layer": (ctypes.c_int, [_vp, ctypes.c_int, _c_int64, _c_int64, _c_int64, _vp, _vp, _vp,
                                           ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                           _vp]),
    "gptq_quantize_layer_ex": (ctypes.c_int, [_vp, ctypes.c_int, _c_int64, _c_int64, _c_int64, _vp, _vp, _vp,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _vp, _vp,
                                              _vp, ctypes.c_size_t, _vp]),
    "gptq_quantize_layer_r": (ctypes.c_int, [_vp, ctypes.c_int, _c_int64, _c_int64, _c_int64, _vp, _vp, _vp,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _vp, _vp,
                                             _vp, ctypes.c_size_t, _vp]),
    "gptq_hessian_accumulate_noalloc": (ctypes.c_int, [_vp, ctypes.c_int, _c_int64, _c_int64, _c_int64, _vp, _vp,
                                                       ctypes.POINTER(_c_int64), _vp]),
    "gptq_packed_words_per_row": (_c_int64, [_c_int64, ctypes.c_int]),
    "gptq_pack_codes": (ctypes.c_int, [_vp, _c_int64, _c_int64, ctypes.c_int, ctypes.c_int, _vp, _vp]),
    "gptq_dequant_matmul": (ctypes.c_int, [_vp, ctypes.c_int, _c_int64, _c_int64, _c_int64, _vp, _vp, _vp, _vp,
                                           _c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, ctypes.c_int,
                                           _vp, _c_int64, _vp]),
}

_lib = None


class GPTQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m post_weight_quantization_05_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().gptq_status_string(int(status)).decode()


def check(status: int, what: str) -> None:
    if status != GPTQ_OK:
        raise GPTQError(status, what)
