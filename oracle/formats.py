"""Element formats: e2m1 (fp4), E4M3 (fp8), E8M0 scales, and float casts.

Test infrastructure only (see ``oracle/__init__.py``).  Plain NumPy, float64.

Readings taken where the pages are open or garbled:

* The printed ``_FP4_E2M1_TABLE`` ("nemo_automodel.components.quantization.mxfp4",
  Data) is cut off after its -2 entry.  The three remaining entries are read
  as -3, -4, -6: the negative half mirrors the positive grid {0, .5, 1, 1.5,
  2, 3, 4, 6} that "NVFP4 in the code: two scales and a nibble" gives.
  Entry 8 is printed as +0.0 and is kept so: code 8 decodes to +0.0.
* The page lists the seven midpoints but no tie rule.  "NVFP4 in the code:
  two scales and a nibble" says ModelOpt's cast moves ties at 0.75, 1.75 and
  3.5 up, i.e. round-half-to-even on the grid; the oracle does the same, so a
  tie at 0.25, 1.25, 2.5 or 5 stays at the lower grid value.
* The sign bit of a code is set for x < 0 (so -0.0 encodes as code 0 and a
  small negative that rounds to zero magnitude encodes as code 8).
"""

import numpy as np

# Data entry MXFP4_BLOCK_SIZE: columns sharing one E8M0 scale.
MXFP4_BLOCK_SIZE = 32

# Data entry _FP4_E2M1_TABLE, completed by sign symmetry (see module docstring).
E2M1_TABLE = np.array(
    [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
     0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], dtype=np.float64)

# Data entry _FP4_E2M1_MIDPOINTS: decision bounds between neighbouring grid values.
E2M1_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float64)

# Midpoints whose ties are moved up to the next grid value (the even code):
# 0.75 -> 1.0, 1.75 -> 2.0, 3.5 -> 4.0.
_TIE_MOVES_UP = np.array([False, True, False, True, False, True, False])

# Largest finite E4M3 value ("NVFP4 in the code": 448 is the top of E4M3's range).
E4M3_MAX = 448.0
# Largest e2m1 magnitude.
E2M1_MAX = 6.0


def e2m1_encode(q):
    """Map already-scaled values q onto 4-bit e2m1 codes.

    The magnitude code is the number of midpoints that |q| has passed
    (searchsorted against ``_FP4_E2M1_MIDPOINTS``), with an exact hit on 0.75,
    1.75 or 3.5 counted as passed.  Anything beyond the last midpoint lands on
    code 7 (6.0), i.e. the cast saturates.  Bit 3 is the sign.
    """
    q = np.asarray(q, dtype=np.float64)
    if not np.all(np.isfinite(q)):
        raise ValueError("e2m1_encode: non-finite input (outside the method's domain)")
    m = np.abs(q)
    below = np.searchsorted(E2M1_MIDPOINTS, m, side="left")  # midpoints strictly below m
    at = np.minimum(below, len(E2M1_MIDPOINTS) - 1)
    tie_up = (below < len(E2M1_MIDPOINTS)) & (E2M1_MIDPOINTS[at] == m) & _TIE_MOVES_UP[at]
    mag = below + tie_up.astype(np.int64)
    sign = (q < 0).astype(np.int64)
    return (mag | (sign << 3)).astype(np.uint8)


def e2m1_byte_table():
    """Data entry _FP4_BYTE_TABLE as a [256, 2] array: byte -> (low-nibble value,
    high-nibble value).  The low nibble holds the even column, the high nibble
    the following odd column (module docstring of the mxfp4 page)."""
    b = np.arange(256)
    return np.stack([E2M1_TABLE[b & 15], E2M1_TABLE[b >> 4]], axis=1)


def e8m0_decode(byte):
    """E8M0 scale byte -> float64 value 2^(b-127); 0xFF is NaN (the
    float8_e8m0fnu type has no zero, no sign and no infinity)."""
    b = np.asarray(byte).astype(np.int64)
    out = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, out)


def round_to_format(v, mant_bits, emin, max_finite, overflow_to_inf=True):
    """Round float64 values to a binary floating-point format, nearest-even.

    A format is given by its stored mantissa bits, the exponent of its smallest
    normal binade (subnormals below it keep the spacing 2^(emin-mant_bits)) and
    its largest finite value.  Values whose rounding exceeds ``max_finite``
    become +-inf when ``overflow_to_inf`` (IEEE formats); otherwise they raise.
    Exact for every float64 input (scaling by powers of two and rint are exact).
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    nan = np.isnan(v)
    inf = np.isinf(v)
    fin = ~(nan | inf)
    a = np.abs(v[fin])
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(a)                 # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, emin)            # binade exponent, clamped into the subnormal range
    ulp = np.ldexp(1.0, e - mant_bits)
    r = np.rint(a / ulp) * ulp              # rint is round-half-to-even
    big = r > max_finite
    if np.any(big):
        if not overflow_to_inf:
            raise OverflowError("round_to_format: value beyond the largest finite value")
        r = np.where(big, np.inf, r)
    out[fin] = np.copysign(r, v[fin])
    out[nan] = np.nan
    out[inf] = v[inf]
    return out


# (stored mantissa bits, smallest normal exponent, largest finite value, storage dtype)
_FORMATS = {
    "f32": (23, -126, float(np.finfo(np.float32).max), np.float32, np.uint32),
    "f16": (10, -14, 65504.0, np.float16, np.uint16),
    "bf16": (7, -126, float.fromhex("0x1.fep127"), None, np.uint16),
}


def to_dtype_bits(values, dtype):
    """Round float64 values to ``dtype`` ('f32' | 'f16' | 'bf16') nearest-even
    and return the raw bit patterns (uint32 for f32, uint16 otherwise)."""
    mant, emin, mx, npdt, bits_t = _FORMATS[dtype]
    r = round_to_format(values, mant, emin, mx)
    if dtype == "bf16":
        # every bf16 value is exactly an fp32 value; bf16 bits are its top half
        return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return r.astype(npdt).view(bits_t)


def from_dtype_bits(bits, dtype):
    """Raw bit patterns of ``dtype`` -> exact float64 values."""
    bits = np.asarray(bits)
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def e4m3_round(q):
    """Round to the E4M3 (fp8, "FN" variant: no infinities) grid, nearest-even,
    keeping the sign (so -0.0 is possible).  3 mantissa bits, smallest normal
    2^-6, subnormal spacing 2^-9, largest finite 448.  The cache scale rule keeps
    |q| <= 448, so a value past it is outside the method's domain and raises."""
    return round_to_format(q, 3, -6, E4M3_MAX, overflow_to_inf=False)
