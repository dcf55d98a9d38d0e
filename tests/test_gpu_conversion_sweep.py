"""Exhaustive encode sweep of the element casts through the library's entry
points: every finite bf16 and f16 bit pattern under every scale exponent it
can share a block with, bit for bit against the oracle.

The element step of every codec is gfx950's scaled conversion (x divided by a
power-of-two block scale, rounded to the e2m1 grid or to E4M3, nearest-even),
plus the sign-of-zero fix-ups of the pages' conventions: a code's sign bit
stands for x < 0, and the e2m1 table ("nemo_automodel.components.quantization.
mxfp4", Data: _FP4_E2M1_TABLE) decodes code 8 to +0.0.  The scale comes from
the block maximum, so each block here holds one element that pins it and 31
(or B - 1) test values that cannot move it:

* quantize_mxfp4 ("nemo_automodel.components.quantization.mxfp4",
  quantize_mxfp4; floor rule e = floor(log2 amax) - 2): pin 2^(e+2), values
  with |x| < 2^(e+3), so x / 2^e spans (-8, 8) -- every e2m1 code, every
  midpoint and tie, and saturation above 6;
* quantize_cache_packed, fp8 ("nemo_automodel.components.models.
  deepseek_v41.quantization", quantize_cache: power-of-two ceiling of amax /
  448): pin 448 * 2^k, values with |x| <= 448 * 2^k, so x / 2^k spans the
  whole E4M3 range, subnormals included;
* quantize_cache_packed, mxfp4 (same rule with 6): pin 6 * 2^k, values with
  |x| <= 6 * 2^k.
The decode side (every code byte under every scale byte) is swept by
test_gpu_codec.py and test_gpu_cache_packed.py."""

import numpy as np
import pytest
import torch

import oracle
import nvfp4_quantization_grouped_amd as mxq
from tests.gpu_util import assert_bits_equal, from_gpu_bits, to_gpu_bits

pytestmark = pytest.mark.gpu


def finite_patterns(dtype):
    """All finite bit patterns of bf16 / f16 with their exact values."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp_all_ones = ((bits >> 7) & 0xFF) == 0xFF if dtype == "bf16" else ((bits >> 10) & 0x1F) == 0x1F
    bits = bits[~exp_all_ones]
    return bits, oracle.from_dtype_bits(bits, dtype)


def pinned_blocks(dtype, block, pins):
    """Rows of `block` elements: element 0 is the pin of its row, the rest are
    test values (zero padding at the end of each pin's group).  pins: list of
    (pin value, bound, inclusive); values with |x| < bound (or <= bound) are
    swept under that pin.  Returns bf16/f16 bits [rows, block]."""
    bits, vals = finite_patterns(dtype)
    rows = []
    for pin, bound, inclusive in pins:
        keep = bits[np.abs(vals) <= bound] if inclusive else bits[np.abs(vals) < bound]
        per = block - 1
        n = -(-len(keep) // per)
        body = np.zeros(n * per, np.uint16)
        body[: len(keep)] = keep
        pin_bits = oracle.to_dtype_bits(np.array([pin]), dtype)[0]
        assert oracle.from_dtype_bits(pin_bits, dtype) == pin, (dtype, pin)   # the pin is exact
        rows.append(np.concatenate([np.full((n, 1), pin_bits, np.uint16), body.reshape(n, per)], axis=1))
    return np.concatenate(rows)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_quantize_mxfp4_every_pattern_every_exponent(dtype):
    # e = floor(log2 amax) - 2; a pin 2^(e+2) must be representable: bf16 e in
    # [-127, 125] (e = -127 is also where every smaller amax clamps), f16 [-26, 13]
    es = range(-127, 126) if dtype == "bf16" else range(-26, 14)
    pins = [(2.0 ** (e + 2), 2.0 ** (e + 3), False) for e in es]
    bits = pinned_blocks(dtype, 32, pins)
    x = oracle.from_dtype_bits(bits, dtype)
    want_p, want_s = oracle.quantize_mxfp4(x)
    assert np.array_equal(np.unique(want_s), np.array(sorted(e + 127 for e in es), np.uint8))
    p, s = mxq.quantize_mxfp4(to_gpu_bits(bits, dtype))
    assert_bits_equal(from_gpu_bits(s), want_s, f"{dtype} scales")
    assert_bits_equal(from_gpu_bits(p).view(np.uint8), want_p.view(np.uint8), f"{dtype} packed codes")
    # the sign-of-zero conventions are part of what was compared: -0.0 and
    # negatives that round to zero both occur in every sweep
    codes = np.stack([want_p.view(np.uint8) & 15, want_p.view(np.uint8) >> 4], -1).reshape(x.shape)
    assert np.any((codes == 8) & (x < 0)) and np.any((codes == 0) & (x == 0) & np.signbit(x))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_quantize_cache_packed_every_pattern_every_exponent(dtype, fmt):
    fmax = 448.0 if fmt == "fp8" else 6.0
    # s = 2^k exactly when amax = fmax * 2^k (k >= -126, the floor of the
    # rule); the pin must be representable in the input dtype
    lo, hi = (-126, 127 - (8 if fmt == "fp8" else 2)) if dtype == "bf16" else \
        ((-30, 7) if fmt == "fp8" else (-25, 13))
    pins = [(fmax * 2.0 ** k, fmax * 2.0 ** k, True) for k in range(lo, hi + 1)]
    bits = pinned_blocks(dtype, 32, pins)
    x = oracle.from_dtype_bits(bits, dtype)
    want_c, want_s = oracle.quantize_cache_packed(x, fmt, 32)
    c, s = mxq.quantize_cache_packed(to_gpu_bits(bits, dtype), fmt, 32)
    assert_bits_equal(from_gpu_bits(s), want_s, f"{fmt} {dtype} scales")
    assert_bits_equal(from_gpu_bits(c), want_c, f"{fmt} {dtype} codes")
