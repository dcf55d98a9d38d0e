"""MXFP4GroupedMM forward and activation backward, as
"nemo_automodel.components.quantization.mxfp4" (class ``MXFP4GroupedMM``) defines them.

Test infrastructure only (see ``oracle/__init__.py``).  float64 throughout.

* Weights are [E, N, K] packed along K ([E, N, K/2] int8 plus [E, N, K/32]
  E8M0) and dequantized exactly (``dequantize_mxfp4``).
* ``offs`` holds cumulative token counts: expert e owns rows
  [offs[e-1], offs[e]) of the activations, with offs[-1] read as 0.
* Forward: y[rows_e] = x[rows_e] @ W_e^T.  Backward: grad_x[rows_e] =
  grad_out[rows_e] @ W_e, from a fresh dequantization; no weight gradient.
* Reading: rows at or past offs[E-1] belong to no expert; they are returned as
  zeros (the page leaves them unspecified).
"""

import numpy as np

from .mxfp4 import dequantize_mxfp4_values, quantize_mxfp4
from .cache import quantize_cache_packed
from .nvfp4 import e4m3_decode


def segments(offs, tokens):
    """[(e, start, end)] for every expert; checks the offsets' preconditions
    (non-decreasing, non-negative, last <= tokens)."""
    offs = np.asarray(offs, dtype=np.int64)
    out = []
    start = 0
    for e, end in enumerate(offs.tolist()):
        if end < start or end > tokens:
            raise ValueError("offs must be non-decreasing cumulative counts <= tokens")
        out.append((e, start, end))
        start = end
    return out


def _covered(offs):
    """Number of leading rows that belong to some expert (offs[E-1], or 0)."""
    offs = np.asarray(offs, dtype=np.int64)
    return int(offs[-1]) if offs.size else 0


def dequantize_expert_weights(packed, scales, expert):
    """Exact float64 W_e [N, K] of one expert."""
    return dequantize_mxfp4_values(packed[expert], scales[expert])


def grouped_mm_fwd(x, packed, scales, offs, rows=None):
    """y = x @ W_e^T per expert segment.  x: float64 [T, K].  Returns float64 [T, N].

    ``rows`` (optional sorted int array) restricts the computation to those
    output rows (others are left as NaN) so full-size workloads can be sampled.
    """
    x = np.asarray(x, dtype=np.float64)
    T, K = x.shape
    E, N, K2 = packed.shape
    if K2 * 2 != K:
        raise ValueError("grouped_mm_fwd: packed must be [E, N, K/2]")
    y = np.zeros((T, N)) if rows is None else np.full((T, N), np.nan)
    if rows is not None:
        y[rows[rows >= _covered(offs)]] = 0.0
    for e, s, t in segments(offs, T):
        sel = np.arange(s, t) if rows is None else rows[(rows >= s) & (rows < t)]
        if len(sel) == 0:
            continue
        w = dequantize_expert_weights(packed, scales, e)           # [N, K]
        y[sel] = x[sel] @ w.T
    return y


def grouped_mm_bwd_x(grad_out, packed, scales, offs, rows=None):
    """grad_x = grad_out @ W_e per expert segment.  grad_out: float64 [T, N].
    Returns float64 [T, K]; ``rows`` as in ``grouped_mm_fwd``."""
    g = np.asarray(grad_out, dtype=np.float64)
    T, N = g.shape
    E, N2, K2 = packed.shape
    if N2 != N:
        raise ValueError("grouped_mm_bwd_x: packed must be [E, N, K/2]")
    K = 2 * K2
    gx = np.zeros((T, K)) if rows is None else np.full((T, K), np.nan)
    if rows is not None:
        gx[rows[rows >= _covered(offs)]] = 0.0
    for e, s, t in segments(offs, T):
        sel = np.arange(s, t) if rows is None else rows[(rows >= s) & (rows < t)]
        if len(sel) == 0:
            continue
        w = dequantize_expert_weights(packed, scales, e)           # [N, K]
        gx[sel] = g[sel] @ w
    return gx


def w4a4_activations(x):
    """Exact float64 values of activations x [T, K] after MXFP4 quantization
    by ``quantize_mxfp4`` (per token row, 32-blocks along K, floor scale rule).

    Reading: "NVIDIA Model Optimizer: from mtq.quantize to a 4.95-bit
    DeepSeek-R1", section "The claims, marked reported" (weight-only 4-bit
    against W4A4), names the weight-and-activation FP4 form as the one that
    runs on the FP4 matrix units, and "nemo_automodel.components.quantization.mxfp4" has one MXFP4
    quantizer, ``quantize_mxfp4``; the activations of the W4A4 forward are
    taken to be quantized by it.  Each row is independent, so a subset of
    rows can be quantized on its own."""
    xq, xs = quantize_mxfp4(np.asarray(x, dtype=np.float64))
    return dequantize_mxfp4_values(xq, xs)


def grouped_mm_fwd_w4a4(x, packed, scales, offs, rows=None):
    """W4A4 forward: y[rows_e] = q(x)[rows_e] @ W_e^T, with q the MXFP4
    round trip of ``w4a4_activations``, then ``grouped_mm_fwd`` on those
    exact values (float64).  ``rows`` as in ``grouped_mm_fwd``."""
    return grouped_mm_fwd(w4a4_activations(x), packed, scales, offs, rows=rows)


def w4a8_activations(x):
    """Exact float64 values of activations x [T, K] after fp8 quantization:
    E4M3 codes with one E8M0 power-of-two scale per 32 consecutive columns,
    the form ``quantize_cache_packed(x, "fp8", 32)`` stores (scale = power-of-
    two ceiling of fl32(amax / 448), floored at 2^-126; elements rounded to
    E4M3 nearest-even).

    Reading: "NVIDIA Model Optimizer: from mtq.quantize to a 4.95-bit
    DeepSeek-R1", section "NVFP4 in the code: two scales and a nibble", has
    activation scales computed at run time, and its "The claims, marked
    reported" section names W4A8 beside W4A4 among the weight-and-activation
    forms; the pages define one fp8 activation encoding with power-of-two
    block scales, the fp8 form of "nemo_automodel.components.models.
    deepseek_v41.quantization" quantize_cache, taken here at the 32-column
    block of the MXFP4 weights (the block the block-scaled MFMA scales by).
    Each row is independent, so a subset of rows can be quantized alone."""
    codes, sc = quantize_cache_packed(np.asarray(x, dtype=np.float64), "fp8", 32)
    return e4m3_decode(codes) * np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=-1)


def grouped_mm_fwd_w4a8(x, packed, scales, offs, rows=None):
    """W4A8 forward: y[rows_e] = q8(x)[rows_e] @ W_e^T, with q8 the fp8
    round trip of ``w4a8_activations``, then ``grouped_mm_fwd`` on those
    exact values (float64).  ``rows`` as in ``grouped_mm_fwd``."""
    return grouped_mm_fwd(w4a8_activations(x), packed, scales, offs, rows=rows)


def grouped_mm_rows(rows, packed, scales, offs, x_rows=None, g_rows=None):
    """Forward and/or activation-backward restricted to the given token rows,
    for sampling full-size workloads: ``rows`` (sorted ints), ``x_rows`` =
    x[rows] ([R, K]) and/or ``g_rows`` = grad_out[rows] ([R, N]).  Each expert's
    weight is dequantized once for both products.  Returns (y[rows], grad_x[rows])
    (None for a product not asked for); rows no expert owns give zeros."""
    rows = np.asarray(rows, dtype=np.int64)
    E, N, K2 = packed.shape
    K = 2 * K2
    y = None if x_rows is None else np.zeros((len(rows), N))
    gx = None if g_rows is None else np.zeros((len(rows), K))
    for e, s, t in _segments_unbounded(offs):
        sel = np.flatnonzero((rows >= s) & (rows < t))
        if len(sel) == 0:
            continue
        w = dequantize_expert_weights(packed, scales, e)
        if y is not None:
            y[sel] = np.asarray(x_rows, dtype=np.float64)[sel] @ w.T
        if gx is not None:
            gx[sel] = np.asarray(g_rows, dtype=np.float64)[sel] @ w
    return y, gx


def _segments_unbounded(offs):
    offs = np.asarray(offs, dtype=np.int64)
    return segments(offs, int(offs[-1]) if offs.size else 0)
