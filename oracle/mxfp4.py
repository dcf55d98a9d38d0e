"""quantize_mxfp4 / dequantize_mxfp4, as "nemo_automodel.components.quantization.mxfp4"
defines them.

Test infrastructure only (see ``oracle/__init__.py``).

Readings taken where the page is open:

* ``floor(log2(amax))`` is read as mathematics: the exact binade of amax,
  taken from its float64 exponent (fp32 and bf16 inputs, subnormals included,
  are normal float64 numbers, so frexp is exact).  A rounded fp32 log2 would
  misplace amax values just below a power of two.
* An all-zero block (amax = 0) gets scale byte 0x00, the bottom of the E8M0
  range, which is where a vanishing amax tends; its codes are 0 whatever the
  scale.  The scale exponent is clamped to the E8M0 range [-127, 127].
* Inputs must be finite.
"""

import numpy as np

from .formats import MXFP4_BLOCK_SIZE, E2M1_TABLE, e2m1_encode, e2m1_byte_table, e8m0_decode, to_dtype_bits

E8M0_MIN_EXP = -127
E8M0_MAX_EXP = 127


def floor_scale_exponent(amax):
    """Scale exponent of a block: floor(log2(amax)) - 2, clamped to the E8M0
    range; amax == 0 maps to the bottom of the range ("quantize_mxfp4")."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)                 # amax = f * 2^ex with f in [0.5, 1), exact
    e = (ex.astype(np.int64) - 1) - 2      # floor(log2 amax) = ex - 1
    e = np.where(amax == 0, E8M0_MIN_EXP, e)
    return np.clip(e, E8M0_MIN_EXP, E8M0_MAX_EXP)


def quantize_mxfp4(x):
    """x: float64 array [..., K] (exact values of an fp32/bf16/fp16 tensor),
    K divisible by 32.  Returns (packed int8 [..., K/2], scales uint8 [..., K/32]).

    Steps, in the page's order: view the last dim as [K/32, 32] blocks; take
    each block's amax; scale 2^(floor(log2 amax) - 2); divide (exact: a power
    of two); cast every element to the nearest e2m1 code by the midpoints;
    pack code pairs with the even column in the low nibble; store the scale
    exponent biased by 127 as the E8M0 byte.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize_mxfp4: non-finite input")
    K = x.shape[-1]
    if K % MXFP4_BLOCK_SIZE != 0:
        raise ValueError("quantize_mxfp4: K must be divisible by 32")
    lead = x.shape[:-1]
    blocks = x.reshape(lead + (K // MXFP4_BLOCK_SIZE, MXFP4_BLOCK_SIZE))
    amax = np.max(np.abs(blocks), axis=-1)
    e = floor_scale_exponent(amax)
    q = blocks / np.ldexp(1.0, e)[..., None]
    codes = e2m1_encode(q).reshape(lead + (K,)).astype(np.uint8)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    scales = (e + 127).astype(np.uint8)
    return packed.view(np.int8), scales


def dequantize_mxfp4_values(packed, scales):
    """Exact float64 values of a packed mxfp4 tensor: each byte looks up its
    (even, odd) column pair in the byte table, and each run of 32 columns is
    multiplied by its E8M0 scale 2^(b-127) (NaN for 0xFF)."""
    p = np.asarray(packed).view(np.uint8) if np.asarray(packed).dtype == np.int8 else np.asarray(packed, dtype=np.uint8)
    s = np.asarray(scales, dtype=np.uint8)
    lead = p.shape[:-1]
    K = p.shape[-1] * 2
    if s.shape != lead + (K // MXFP4_BLOCK_SIZE,):
        raise ValueError("dequantize_mxfp4: scales must be [..., K/32]")
    pairs = e2m1_byte_table()[p.astype(np.int64)]          # [..., K/2, 2]
    vals = pairs.reshape(lead + (K,))
    scale = np.repeat(e8m0_decode(s), MXFP4_BLOCK_SIZE, axis=-1)
    with np.errstate(invalid="ignore", over="ignore"):
        return vals * scale


def dequantize_mxfp4(packed, scales, dtype):
    """Values as ``dequantize_mxfp4_values``, rounded nearest-even to ``dtype``
    ('f32' | 'bf16' | 'f16'); returns raw bit patterns of that dtype."""
    return to_dtype_bits(dequantize_mxfp4_values(packed, scales), dtype)


__all__ = ["quantize_mxfp4", "dequantize_mxfp4", "dequantize_mxfp4_values",
           "floor_scale_exponent", "E2M1_TABLE"]
