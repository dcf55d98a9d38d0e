"""Two-level NVFP4 quantization and dequantization, as "NVIDIA Model Optimizer:
from mtq.quantize to a 4.95-bit DeepSeek-R1", section "NVFP4 in the code: two
scales and a nibble", defines them.

Test infrastructure only (see ``oracle/__init__.py``).

For a tensor x and its blocks b of 16 consecutive elements along the last
dimension:

* g = max|x| / (6 * 448), an FP32 per-tensor scale (6 the largest e2m1
  value, 448 the largest E4M3 value);
* s_b = E4M3(max_{i in b} |x_i| / (6 g)), an FP8 block scale: a zero scale
  becomes 1.0, then the value is clamped to [2^-9, 448] and cast to E4M3;
* x_hat_i = E2M1(x_i / (s_b g)) * s_b g, the e2m1 cast by the midpoints with
  ties to the even code; two codes per byte, the even column in the low nibble
  (the page's packing expression).

Readings (the page gives the formulas, not the arithmetic):

* FP32 throughout, each operation rounded nearest-even in the order written:
  g = fl(amax / 2688); the block ratio fl(amax_b / fl(6 g)); the element
  divisor d_b = fl(s_b g); q_i = fl(x_i / d_b); the dequantized value
  fl(E2M1 value * d_b), then rounded to the output dtype.
* The E4M3 cast rounds to nearest-even (the clamp keeps it finite).
* A tensor whose max |x| is 0 has g = 0, where the formula would divide by
  zero: every block scale is then 1.0 (the zero-scale rule) and every code 0.
  *Parity unpinned by the page*; the kernels take the same reading.

The MSE block-scale rule (same page, section "Where the scales come from",
the paragraph on NVFP4's own rules): instead of the
max rule, each block tries every positive finite E4M3 value (codes 0x01 ..
0x7E, 126 of them) as s_b and keeps the one whose quantized block has the
least squared error against x.  Readings:

* g is the max rule's global scale; for each candidate the codes and the
  dequantized values are the two-level ones above (d = fl(s g), codes of
  fl(x / d), x_hat = fl(e2m1 * d)).
* The error is computed in fp32 in a fixed order: e_i = x_i - e2m1_i * d
  rounded once (a fused multiply-add; x_hat_i itself is not rounded first),
  fl(e_i * e_i), summed i = 0 .. 15 left to right, each sum rounded.  The
  fused e_i is exact to emulate: e2m1_i * d has at most 26 significant bits
  and x_i and e2m1_i * d are at most about 2^18 apart, so their difference is
  exact in float64 and one cast rounds it as the fused operation does.  The candidate chosen is the first, in increasing
  code order, with an error strictly below every earlier one; candidates
  whose d underflows to 0 are skipped.  An all-zero block therefore gets
  code 0x01 (every candidate is exact), and g = 0 gives the max rule's
  result (scales 1.0, codes 0).
"""

import numpy as np

from .formats import E2M1_MAX, E2M1_TABLE, E4M3_MAX, e2m1_encode, e4m3_round, to_dtype_bits

NVFP4_BLOCK = 16
NVFP4_SCALE_MIN = 2.0 ** -9     # smallest positive E4M3 value (a subnormal)
_F32 = np.float32


def global_scale(x):
    """g = fl32(max|x| / (6 * 448)) as a float32 (6 * 448 = 2688 exactly)."""
    amax = _F32(np.max(np.abs(np.asarray(x, dtype=np.float64)))) if np.asarray(x).size else _F32(0)
    return _F32(amax / _F32(E2M1_MAX * E4M3_MAX))


def e4m3_bits(v):
    """Non-negative E4M3 values (already on the grid) -> their FN-variant bit
    patterns: exponent bias 7, 3 mantissa bits, subnormals below 2^-6."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or np.any(v > E4M3_MAX):
        raise ValueError("e4m3_bits: outside [0, 448]")
    _, ex = np.frexp(v)                                # v = f 2^ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 1
    normal = v >= 2.0 ** -6
    mant_n = np.rint((v / np.ldexp(1.0, np.where(normal, e, 0)) - 1.0) * 8.0).astype(np.int64)
    bits_n = ((e + 7) << 3) | mant_n
    bits_s = np.rint(v / 2.0 ** -9).astype(np.int64)    # subnormal: mantissa counts 2^-9
    return np.where(normal, bits_n, bits_s).astype(np.uint8)


def e4m3_decode(bits):
    """E4M3 (FN) bit patterns -> float64 values (0x7F / 0xFF are NaN)."""
    b = np.asarray(bits).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 15
    m = b & 7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    return np.where((b & 0x7F) == 0x7F, np.nan, s * val)


def _codes_for_scales(blocks, g, s):
    """e2m1 codes of fp32 blocks [..., nb, 16] under scales s [..., nb]
    (E4M3 values) and global scale g: codes of fl(x / fl(s g))."""
    d = (s.astype(_F32) * _F32(g)).astype(_F32)          # element divisor, fp32
    q = (blocks / d[..., None]).astype(_F32)             # fp32 division, nearest-even
    return e2m1_encode(q.astype(np.float64))


def encode_with_global_scale(x, g):
    """Block scales and codes of x [..., K] (K % 16 == 0) given the tensor's
    global scale g (float32).  Returns (packed uint8 [..., K/2], block scale
    bits uint8 [..., K/16]).  Rows are independent given g, so a subset of rows
    of a large tensor can be encoded on its own."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize_nvfp4: non-finite input")
    K = x.shape[-1]
    if K % NVFP4_BLOCK != 0:
        raise ValueError("quantize_nvfp4: K must be divisible by 16")
    lead = x.shape[:-1]
    xf = x.astype(_F32)                                  # exact: x holds fp32/bf16/fp16 values
    blocks = xf.reshape(lead + (K // NVFP4_BLOCK, NVFP4_BLOCK))
    amax_b = np.max(np.abs(blocks), axis=-1)
    g = _F32(g)
    if g == 0:
        s = np.ones(amax_b.shape)
        codes = np.zeros(blocks.shape, np.uint8)
    else:
        ratio = (amax_b / _F32(_F32(E2M1_MAX) * g)).astype(_F32)
        ratio = np.where(ratio == 0, _F32(1.0), ratio)
        ratio = np.clip(ratio, _F32(NVFP4_SCALE_MIN), _F32(E4M3_MAX))
        s = e4m3_round(ratio.astype(np.float64))
        codes = _codes_for_scales(blocks, g, s)
    codes = codes.reshape(lead + (K,))
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, e4m3_bits(s)


def block_sq_errors(blocks, g, s):
    """fp32 squared error of each block [..., 16] quantized with scale s [...]
    (E4M3 values) and global scale g, in the reading's order.  Returns
    (errors float32 [...], divisor d float32 [...])."""
    d = (s.astype(_F32) * _F32(g)).astype(_F32)
    codes = _codes_for_scales(blocks, g, s)
    vd = E2M1_TABLE[codes.astype(np.int64)] * d.astype(np.float64)[..., None]      # exact in float64
    e = (blocks.astype(np.float64) - vd).astype(_F32)                               # one rounding (fused)
    sq = (e * e).astype(_F32)
    acc = np.zeros(sq.shape[:-1], _F32)
    with np.errstate(over="ignore"):
        for i in range(sq.shape[-1]):
            acc = (acc + sq[..., i]).astype(_F32)
    return acc, d


def mse_block_scales(x, g):
    """The MSE rule's block scale codes (E4M3 bits, uint8 [..., K/16]) of x
    [..., K] under global scale g (float32, nonzero)."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    blocks = x.astype(_F32).reshape(x.shape[:-1] + (K // NVFP4_BLOCK, NVFP4_BLOCK))
    best = np.zeros(blocks.shape[:-1], np.uint8)
    best_err = np.zeros(best.shape, _F32)
    for code in range(1, 0x7F):
        s = np.full(best.shape, e4m3_decode(np.uint8(code)))
        err, d = block_sq_errors(blocks, g, s)
        take = (d != 0) & ((best == 0) | (err < best_err))
        best = np.where(take, np.uint8(code), best)
        best_err = np.where(take, err, best_err)
    return best


def quantize_nvfp4_mse(x):
    """Two-level NVFP4 with MSE-searched block scales: x [..., K] (K % 16 ==
    0) -> (packed uint8 [..., K/2], block scale bits uint8 [..., K/16], g
    float32); dequantized by ``dequantize_nvfp4``."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize_nvfp4_mse: non-finite input")
    K = x.shape[-1]
    if K % NVFP4_BLOCK != 0:
        raise ValueError("quantize_nvfp4_mse: K must be divisible by 16")
    g = global_scale(x)
    if g == 0:
        packed, scales = encode_with_global_scale(x, g)
        return packed, scales, g
    scales = mse_block_scales(x, g)
    blocks = x.astype(_F32).reshape(x.shape[:-1] + (K // NVFP4_BLOCK, NVFP4_BLOCK))
    codes = _codes_for_scales(blocks, g, e4m3_decode(scales)).reshape(x.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, scales, g


def quantize_nvfp4(x):
    """x [..., K] float64 (exact values of an fp32/bf16/fp16 tensor) ->
    (packed uint8 [..., K/2], block scale E4M3 bits uint8 [..., K/16],
    global scale g float32)."""
    g = global_scale(x)
    packed, scales = encode_with_global_scale(x, g)
    return packed, scales, g


def dequantize_nvfp4_values(packed, scale_bits, g):
    """Exact float64 values of fl32(E2M1 value * fl32(s_b g)): the
    dequantized tensor in fp32."""
    p = np.asarray(packed, dtype=np.uint8)
    lead = p.shape[:-1]
    K = p.shape[-1] * 2
    sb = np.asarray(scale_bits, dtype=np.uint8)
    if sb.shape != lead + (K // NVFP4_BLOCK,):
        raise ValueError("dequantize_nvfp4: block scales must be [..., K/16]")
    codes = np.stack([p & 15, p >> 4], axis=-1).reshape(lead + (K,))
    vals = E2M1_TABLE[codes.astype(np.int64)].astype(_F32)
    d = (e4m3_decode(sb).astype(_F32) * _F32(g)).astype(_F32)
    with np.errstate(invalid="ignore", over="ignore"):
        out = (vals.reshape(lead + (K // NVFP4_BLOCK, NVFP4_BLOCK)) * d[..., None]).astype(_F32)
    return out.reshape(lead + (K,)).astype(np.float64)


def dequantize_nvfp4(packed, scale_bits, g, dtype):
    """Values as ``dequantize_nvfp4_values``, rounded nearest-even to ``dtype``
    ('f32' | 'bf16' | 'f16'); returns raw bit patterns of that dtype."""
    return to_dtype_bits(dequantize_nvfp4_values(packed, scale_bits, g), dtype)


__all__ = ["NVFP4_BLOCK", "global_scale", "e4m3_bits", "e4m3_decode", "encode_with_global_scale",
           "quantize_nvfp4", "dequantize_nvfp4_values", "dequantize_nvfp4", "block_sq_errors",
           "mse_block_scales", "quantize_nvfp4_mse"]
