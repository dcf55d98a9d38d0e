"""ctypes loader for libmxq.so, the HIP library behind this package.

Loads the in-tree ``libmxq.so`` and declares the C signatures of
``include/mxq.h``.  There is no fallback: if the library is missing or cannot
be loaded, using any op raises.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxq.so")

# mxq_dtype / mxq_format codes (include/mxq.h)
MXQ_F32, MXQ_BF16, MXQ_F16 = 0, 1, 2
MXQ_FMT_FP8, MXQ_FMT_MXFP4, MXQ_FMT_NVFP4 = 0, 1, 2
MXQ_ERR_OFFS = -9

EXPORTS = (
    "quantize_mxfp4", "dequantize_mxfp4", "quantize_cache", "quantize_cache_bwd", "quantize_nvfp4", "dequantize_nvfp4",
    "quantize_cache_packed", "dequantize_cache_packed", "quantize_nvfp4_mse",
    "mxfp4_grouped_mm_fwd", "mxfp4_grouped_mm_bwd_x", "mxfp4_grouped_mm_fwd_w4a4", "mxfp4_grouped_mm_fwd_w4a8",
    "mxq_validate_offs", "mxq_status_string",
)

_lib = None

_vp, _i64, _i32, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
_SIGS = {
    "quantize_mxfp4": ([_vp, _int, _i64, _i64, _vp, _vp, _vp], _int),
    "dequantize_mxfp4": ([_vp, _vp, _i64, _i64, _vp, _int, _vp], _int),
    "quantize_cache": ([_vp, _vp, _int, _i64, _i64, _int, _i32, _vp], _int),
    "quantize_cache_bwd": ([_vp, _vp, _int, _i64, _vp], _int),
    "quantize_nvfp4": ([_vp, _int, _i64, _i64, _vp, _vp, _vp, _vp], _int),
    "dequantize_nvfp4": ([_vp, _vp, _vp, _i64, _i64, _vp, _int, _vp], _int),
    "quantize_nvfp4_mse": ([_vp, _int, _i64, _i64, _vp, _vp, _vp, _vp], _int),
    "quantize_cache_packed": ([_vp, _int, _i64, _i64, _int, _i32, _vp, _vp, _vp], _int),
    "dequantize_cache_packed": ([_vp, _vp, _i64, _i64, _int, _i32, _vp, _int, _vp], _int),
    "mxfp4_grouped_mm_fwd": ([_vp, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _vp, _vp], _int),
    "mxfp4_grouped_mm_bwd_x": ([_vp, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _vp, _vp], _int),
    "mxfp4_grouped_mm_fwd_w4a4": ([_vp, _vp, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _vp, _vp], _int),
    "mxfp4_grouped_mm_fwd_w4a8": ([_vp, _vp, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _vp, _vp], _int),
    "mxq_validate_offs": ([_vp, _i64, _i64, _vp, _vp], _int),
    "mxq_status_string": ([_int], ctypes.c_char_p),
}


class MxqError(RuntimeError):
    """A libmxq entry point returned a non-zero status."""


def lib():
    """The loaded library (loads it on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m nvfp4_quantization_grouped_amd.build` "
                "(hipcc for gfx950).  There is no fallback implementation.")
        l = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(l, name)
            f.argtypes = args
            f.restype = res
        _lib = l
    return _lib


def check(status, fn):
    if status != 0:
        msg = lib().mxq_status_string(status).decode()
        raise MxqError(f"{fn}: status {status} ({msg})")
