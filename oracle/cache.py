"""quantize_cache and its straight-through backward, as
"nemo_automodel.components.models.deepseek_v41.quantization" defines them.

Test infrastructure only (see ``oracle/__init__.py``).

Readings taken where the page is open:

* Scale rule.  The block scale is the power-of-two ceiling of amax / fmax,
  where fmax is the largest value of the element format (6 for e2m1, 448 for
  E4M3, "NVFP4 in the code: two scales and a nibble").  ``_power_of_two_ceiling``
  is documented for positive normal FP32 inputs, so the ratio is formed in
  fp32 and floored at the smallest positive normal fp32 value, 2^-126, before
  the ceiling (an all-zero block then gets scale 2^-126 and stays zero).
* nvfp4 stores its scale as E4M3; the powers of two E4M3 can hold are
  2^-9 .. 2^8, so the nvfp4 scale is clamped to that range.  mxfp4 stores
  E8M0, which holds every scale the rule can produce.  fp8's scale storage is
  not stated; since only the round-tripped values are returned it is an fp32
  power of two.  (No clamp binds on the seeded workloads.)
* A final partial group is padded with zeros (page: ``quantize_cache``,
  parameter ``values``); padding cannot change a group's amax, and is dropped
  again from the output.
* e2m1 elements decode through the table, so a code-8 element comes back as
  +0.0; fp8 keeps the sign of zero.  The fake-quant value (grid value times
  scale) is rounded nearest-even to the input dtype.
* Any block size is accepted for every format; the page uses 32 for SWA and the
  indexer and 16 for compressed KV.
* Packed storage (``quantize_cache_packed``): the page keeps only the
  round-tripped values.  Storing the codes and the per-group scale bytes that
  round trip passes through (e2m1 nibbles or E4M3 bytes; E8M0 or E4M3 scale
  bytes) is the plainest packed form; it needs whole groups, and decoding it
  gives the fake-quantized tensor bit for bit.
"""

import numpy as np

from .formats import E2M1_TABLE, E2M1_MAX, E4M3_MAX, e2m1_encode, e4m3_round, to_dtype_bits

FORMAT_FMAX = {"fp8": E4M3_MAX, "mxfp4": E2M1_MAX, "nvfp4": E2M1_MAX}
SMALLEST_NORMAL_F32 = 2.0 ** -126
NVFP4_SCALE_MIN = 2.0 ** -9   # smallest power of two E4M3 holds (a subnormal)
NVFP4_SCALE_MAX = 2.0 ** 8    # largest power of two E4M3 holds


def power_of_two_ceiling(value):
    """``_power_of_two_ceiling``: the smallest integer power of two that is >= value,
    for positive normal fp32 values."""
    v = np.asarray(value, dtype=np.float64)
    if np.any(~(v >= SMALLEST_NORMAL_F32)) or np.any(~np.isfinite(v)):
        raise ValueError("power_of_two_ceiling: needs positive normal finite inputs")
    f, ex = np.frexp(v)                     # v = f * 2^ex, f in [0.5, 1)
    # v is already a power of two exactly when f == 0.5
    return np.where(f == 0.5, v, np.ldexp(1.0, ex))


def cache_scale(amax, fmt):
    """Per-block scale of ``quantize_cache`` for format ``fmt``."""
    amax32 = np.asarray(amax, dtype=np.float32)
    ratio = (amax32 / np.float32(FORMAT_FMAX[fmt])).astype(np.float64)   # fp32 division
    s = power_of_two_ceiling(np.maximum(ratio, SMALLEST_NORMAL_F32))
    if fmt == "nvfp4":
        s = np.clip(s, NVFP4_SCALE_MIN, NVFP4_SCALE_MAX)
    return s


def quantize_cache_values(x, fmt, block_size):
    """Fake-quantized values (exact, float64) of x: float64 [..., C].

    Steps in the page's order: zero-pad the channel dim to whole groups of
    ``block_size``; per group take amax and the power-of-two scale; divide;
    round each element to the format's grid (e2m1 via the midpoint cast and the
    table, or E4M3); multiply the scale back; drop the padding.
    """
    if fmt not in FORMAT_FMAX:
        raise ValueError("quantize_cache: format must be fp8, mxfp4 or nvfp4")
    if block_size <= 0:
        raise ValueError("quantize_cache: block_size must be positive")
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize_cache: non-finite input")
    C = x.shape[-1]
    lead = x.shape[:-1]
    groups = -(-C // block_size)
    padded = np.zeros(lead + (groups * block_size,), dtype=np.float64)
    padded[..., :C] = x
    blocks = padded.reshape(lead + (groups, block_size))
    amax = np.max(np.abs(blocks), axis=-1) if C else np.zeros(lead + (0,))
    s = cache_scale(amax, fmt)[..., None]
    q = blocks / s                                # exact: s is a power of two
    if fmt == "fp8":
        grid = e4m3_round(q)
    else:
        grid = E2M1_TABLE[e2m1_encode(q)]
    out = (grid * s).reshape(lead + (groups * block_size,))
    return out[..., :C]


def quantize_cache(x, fmt, block_size, dtype):
    """``quantize_cache`` on exact input values x (float64 [..., C]) of a tensor
    of ``dtype`` ('f32' | 'bf16' | 'f16'); returns raw bit patterns of a new
    tensor of the same shape and dtype.  The input array is not modified."""
    return to_dtype_bits(quantize_cache_values(x, fmt, block_size), dtype)


def quantize_cache_packed(x, fmt, block_size):
    """The encoding ``quantize_cache`` rounds through, stored instead of
    multiplied back (packed KV-cache storage): x float64 [..., C] with whole
    groups only (C % block_size == 0; even block_size for the fp4 formats).

    Returns (codes, scales):
    * mxfp4 / nvfp4: codes uint8 [..., C/2], e2m1, two per byte with the even
      channel in the low nibble, sign bit for x < 0 (as ``quantize_mxfp4``);
      fp8: codes uint8 [..., C], E4M3 (FN) bit patterns, sign kept;
    * scales uint8 [..., C/block_size]: the group's power-of-two scale 2^k as
      an E8M0 byte k + 127 (mxfp4, fp8) or as E4M3 bits (nvfp4, whose scales
      are clamped into E4M3's powers of two 2^-9..2^8).
    Reading: the page keeps only the round-tripped values; storing the codes
    and scales the round trip goes through is the packed form, and
    ``dequantize_cache_packed`` of it equals ``quantize_cache`` bit for bit."""
    from .nvfp4 import e4m3_bits
    if fmt not in FORMAT_FMAX:
        raise ValueError("quantize_cache_packed: format must be fp8, mxfp4 or nvfp4")
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize_cache_packed: non-finite input")
    C = x.shape[-1]
    if block_size <= 0 or C % block_size or (fmt != "fp8" and block_size % 2):
        raise ValueError("quantize_cache_packed: whole groups of a positive (even for fp4) block size")
    lead = x.shape[:-1]
    blocks = x.reshape(lead + (C // block_size, block_size))
    amax = np.max(np.abs(blocks), axis=-1)
    s = cache_scale(amax, fmt)
    q = blocks / s[..., None]                      # exact: s is a power of two
    if fmt == "fp8":
        v = e4m3_round(q).reshape(lead + (C,))
        codes = (e4m3_bits(np.abs(v)) | (np.signbit(v).astype(np.uint8) << 7)).astype(np.uint8)
    else:
        c = e2m1_encode(q).reshape(lead + (C,))
        codes = (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
    if fmt == "nvfp4":
        scales = e4m3_bits(s)
    else:
        _, ex = np.frexp(s)                        # s = 2^(ex-1)
        scales = (ex.astype(np.int64) - 1 + 127).astype(np.uint8)
    return codes, scales


def dequantize_cache_packed(codes, scales, fmt, block_size, dtype):
    """Values of the packed form: code value (e2m1 table, code 8 -> +0.0; or
    E4M3) times the group's scale, rounded to ``dtype``; raw bit patterns."""
    from .nvfp4 import e4m3_decode
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    if fmt == "fp8":
        vals = e4m3_decode(codes)
    else:
        vals = np.stack([E2M1_TABLE[codes & 15], E2M1_TABLE[codes >> 4]], axis=-1).reshape(
            codes.shape[:-1] + (codes.shape[-1] * 2,))
    s = e4m3_decode(scales) if fmt == "nvfp4" else np.ldexp(1.0, scales.astype(np.int64) - 127)
    C = vals.shape[-1]
    out = vals.reshape(vals.shape[:-1] + (C // block_size, block_size)) * s[..., None]
    return to_dtype_bits(out.reshape(vals.shape), dtype)


def quantize_cache_backward(grad):
    """``_CacheQuantization.backward``: the incoming gradient passes through
    unchanged (straight-through); block_size and format get no gradient."""
    return grad, None, None
