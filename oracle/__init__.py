"""CPU oracle for block-scaled microscaling quantization and the MXFP4 grouped GEMM.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct
NumPy / PyTorch-CPU restatement of what the pages compute.  It exists so that
the HIP path can be checked against something written independently of it.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product path (``nvfp4_quantization_grouped_amd``)
never imports, calls or links anything here, and nothing here imports the
product path; the two share only the seeded input generators in ``synth/``.

Sources (page title, then the section on that page):

* "nemo_automodel.components.quantization.mxfp4" (NeMo AutoModel API):
  module docstring (nibble order, 32 columns per E8M0 scale), ``quantize_mxfp4``
  (floor scale rule), ``dequantize_mxfp4``, ``MXFP4GroupedMM`` and the Data
  entries ``_FP4_E2M1_TABLE``, ``_FP4_E2M1_MIDPOINTS``, ``_FP4_BYTE_TABLE``,
  ``MXFP4_BLOCK_SIZE``.
* "nemo_automodel.components.models.deepseek_v41.quantization" (NeMo AutoModel
  API): ``quantize_cache``, ``_CacheQuantization.forward/backward``,
  ``_power_of_two_ceiling``.
* "NVIDIA Model Optimizer: from mtq.quantize to a 4.95-bit DeepSeek-R1":
  section "NVFP4 in the code: two scales and a nibble" (tie rule of the e2m1
  cast, the E4M3 range 448 and smallest scale 2^-9, packing expression, and
  the two-level NVFP4 format of ``oracle/nvfp4.py``); section "Where the
  scales come from" (the MSE block-scale sweep); section "The claims,
  marked reported" (W4A4 and W4A8).

Every function is pinned by tests under ``tests/test_oracle_*.py`` against facts
the pages print, closed forms, invariants, library routines for special cases
(PyTorch's float8_e4m3fn and float8_e8m0fnu casts) and brute force.  Readings
of points the pages leave open are listed in the module that takes them.
"""

from .formats import (
    E2M1_TABLE,
    E2M1_MIDPOINTS,
    MXFP4_BLOCK_SIZE,
    E4M3_MAX,
    e2m1_encode,
    e2m1_byte_table,
    e4m3_round,
    e8m0_decode,
    to_dtype_bits,
    from_dtype_bits,
)
from .mxfp4 import quantize_mxfp4, dequantize_mxfp4, floor_scale_exponent
from .cache import (power_of_two_ceiling, cache_scale, quantize_cache, quantize_cache_backward, quantize_cache_packed,
                    dequantize_cache_packed)
from .nvfp4 import (global_scale as nvfp4_global_scale, e4m3_bits, e4m3_decode, encode_with_global_scale as nvfp4_encode,
                    quantize_nvfp4, dequantize_nvfp4_values, dequantize_nvfp4, block_sq_errors as nvfp4_block_sq_errors,
                    mse_block_scales as nvfp4_mse_block_scales, quantize_nvfp4_mse)
from .grouped_mm import (dequantize_expert_weights, grouped_mm_fwd, grouped_mm_bwd_x, grouped_mm_rows, segments,
                         w4a4_activations, grouped_mm_fwd_w4a4, w4a8_activations, grouped_mm_fwd_w4a8)

__all__ = [
    "E2M1_TABLE", "E2M1_MIDPOINTS", "MXFP4_BLOCK_SIZE", "E4M3_MAX",
    "e2m1_encode", "e2m1_byte_table", "e4m3_round", "e8m0_decode",
    "to_dtype_bits", "from_dtype_bits",
    "quantize_mxfp4", "dequantize_mxfp4", "floor_scale_exponent",
    "power_of_two_ceiling", "cache_scale", "quantize_cache", "quantize_cache_backward",
    "quantize_cache_packed", "dequantize_cache_packed",
    "dequantize_expert_weights", "grouped_mm_fwd", "grouped_mm_bwd_x", "grouped_mm_rows", "segments",
    "w4a4_activations", "grouped_mm_fwd_w4a4", "w4a8_activations", "grouped_mm_fwd_w4a8",
    "nvfp4_global_scale", "e4m3_bits", "e4m3_decode", "nvfp4_encode", "quantize_nvfp4", "dequantize_nvfp4_values",
    "dequantize_nvfp4", "nvfp4_block_sq_errors", "nvfp4_mse_block_scales", "quantize_nvfp4_mse",
]
