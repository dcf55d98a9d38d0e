"""MI355X-native block-scaled microscaling quantization and MXFP4 grouped GEMM.

All compute runs in hand-written HIP kernels for gfx950 behind the C ABI in
``include/mxq.h`` (``libmxq.so``, built by ``python -m
nvfp4_quantization_grouped_amd.build``).  This package is the PyTorch-facing
binding: argument checks, output allocation and the current stream.
"""

from ._lib import LIB_PATH, EXPORTS, MxqError, lib
from .ops import (
    MXFP4_BLOCK_SIZE,
    CacheQuantization,
    MXFP4GroupedMM,
    dequantize_mxfp4,
    dequantize_nvfp4,
    mxfp4_grouped_mm_bwd_x,
    mxfp4_grouped_mm_fwd,
    mxfp4_grouped_mm_fwd_w4a4,
    mxfp4_grouped_mm_fwd_w4a4_quantized,
    mxfp4_grouped_mm_fwd_w4a8,
    mxfp4_grouped_mm_fwd_w4a8_quantized,
    quantize_cache,
    quantize_cache_bwd,
    quantize_cache_forward,
    quantize_cache_packed,
    dequantize_cache_packed,
    quantize_mxfp4,
    quantize_nvfp4,
    quantize_nvfp4_mse,
    validate_offs,
)

__all__ = [
    "LIB_PATH", "EXPORTS", "MxqError", "lib",
    "MXFP4_BLOCK_SIZE", "CacheQuantization", "MXFP4GroupedMM",
    "dequantize_mxfp4", "mxfp4_grouped_mm_bwd_x", "mxfp4_grouped_mm_fwd",
    "mxfp4_grouped_mm_fwd_w4a4", "mxfp4_grouped_mm_fwd_w4a4_quantized",
    "mxfp4_grouped_mm_fwd_w4a8", "mxfp4_grouped_mm_fwd_w4a8_quantized",
    "quantize_cache", "quantize_cache_bwd", "quantize_cache_forward", "quantize_mxfp4",
    "quantize_nvfp4", "dequantize_nvfp4", "quantize_cache_packed", "dequantize_cache_packed",
    "quantize_nvfp4_mse", "validate_offs",
]
