"""Pins for oracle/grouped_mm.py: a pure-Python triple loop on tiny inputs, a
row-by-row formulation that finds each row's expert from the offsets, exact
one-hot weights, the adjoint identity <fwd(x), g> = <x, bwd(g)>, empty experts
and uncovered rows."""

import bisect

import numpy as np
import pytest

import oracle
from oracle.mxfp4 import dequantize_mxfp4_values


def rand_weights(g, E, N, K, lo=117, hi=123):
    packed = g.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8).view(np.int8)
    scales = g.integers(lo, hi + 1, size=(E, N, K // 32), dtype=np.uint8)
    return packed, scales


def test_single_expert_matches_triple_loop():
    g = np.random.default_rng(0)
    T, N, K = 5, 3, 64
    packed, scales = rand_weights(g, 1, N, K)
    x = g.standard_normal((T, K))
    W = dequantize_mxfp4_values(packed[0], scales[0])
    y = oracle.grouped_mm_fwd(x, packed, scales, np.array([T], np.int32))
    for t in range(T):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += x[t, k] * W[n, k]
            assert abs(y[t, n] - acc) <= 1e-12 * max(1.0, abs(acc))
    go = g.standard_normal((T, N))
    gx = oracle.grouped_mm_bwd_x(go, packed, scales, np.array([T], np.int32))
    for t in range(T):
        for k in range(K):
            acc = sum(go[t, n] * W[n, k] for n in range(N))
            assert abs(gx[t, k] - acc) <= 1e-12 * max(1.0, abs(acc))


def test_rowwise_formulation_with_empty_experts():
    g = np.random.default_rng(1)
    E, T, N, K = 4, 23, 6, 96
    packed, scales = rand_weights(g, E, N, K)
    offs = np.array([7, 7, 19, 21], np.int32)        # expert 1 empty; rows 21, 22 uncovered
    x = g.standard_normal((T, K))
    go = g.standard_normal((T, N))
    y = oracle.grouped_mm_fwd(x, packed, scales, offs)
    gx = oracle.grouped_mm_bwd_x(go, packed, scales, offs)
    Ws = [dequantize_mxfp4_values(packed[e], scales[e]) for e in range(E)]
    for t in range(T):
        e = bisect.bisect_right(offs.tolist(), t)   # first expert whose end is past t
        if e == E:
            assert np.all(y[t] == 0) and np.all(gx[t] == 0)
            continue
        assert np.allclose(y[t], Ws[e] @ x[t], rtol=1e-12, atol=1e-12)
        assert np.allclose(gx[t], go[t] @ Ws[e], rtol=1e-12, atol=1e-12)


def test_one_hot_weights_are_exact():
    """W_e[n, (n+e) mod K] = 2^(s_e - 127) (code 2 = 1.0), everything else code 0:
    every output is one input times a power of two."""
    E, T, N, K = 3, 12, 40, 64
    g = np.random.default_rng(2)
    codes = np.zeros((E, N, K), np.uint8)
    sbyte = np.array([120, 127, 131], np.uint8)
    for e in range(E):
        for n in range(N):
            codes[e, n, (n + e) % K] = 2
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8).view(np.int8)
    scales = np.repeat(sbyte[:, None, None], N, axis=1).repeat(K // 32, axis=2)
    offs = np.array([4, 9, 12], np.int32)
    x = g.standard_normal((T, K))
    y = oracle.grouped_mm_fwd(x, packed, scales, offs)
    start = 0
    for e in range(E):
        for t in range(start, offs[e]):
            for n in range(N):
                assert y[t, n] == x[t, (n + e) % K] * 2.0 ** (int(sbyte[e]) - 127)
        start = offs[e]
    go = g.standard_normal((T, N))
    gx = oracle.grouped_mm_bwd_x(go, packed, scales, offs)
    start = 0
    for e in range(E):
        for t in range(start, offs[e]):
            want = np.zeros(K)
            for n in range(N):
                want[(n + e) % K] += go[t, n] * 2.0 ** (int(sbyte[e]) - 127)
            assert np.array_equal(gx[t], want)
        start = offs[e]


def test_adjoint_identity():
    """Forward and activation-backward are adjoint per segment:
    sum(fwd(x) * g) == sum(x * bwd(g)).  A transposed operand breaks it when N != K."""
    g = np.random.default_rng(3)
    E, T, N, K = 3, 50, 48, 160
    packed, scales = rand_weights(g, E, N, K)
    offs = np.array([10, 30, 50], np.int32)
    x, go = g.standard_normal((T, K)), g.standard_normal((T, N))
    lhs = np.sum(oracle.grouped_mm_fwd(x, packed, scales, offs) * go)
    rhs = np.sum(x * oracle.grouped_mm_bwd_x(go, packed, scales, offs))
    assert abs(lhs - rhs) <= 1e-9 * max(1.0, abs(lhs))


def test_sampled_rows_match_full():
    g = np.random.default_rng(4)
    E, T, N, K = 3, 40, 16, 64
    packed, scales = rand_weights(g, E, N, K)
    offs = np.array([5, 5, 33], np.int32)
    x = g.standard_normal((T, K))
    full = oracle.grouped_mm_fwd(x, packed, scales, offs)
    rows = np.array([0, 4, 5, 20, 32, 33, 39])
    part = oracle.grouped_mm_fwd(x, packed, scales, offs, rows=rows)
    assert np.array_equal(part[rows], full[rows])


def test_row_restricted_form_matches_full():
    g = np.random.default_rng(6)
    E, T, N, K = 4, 60, 24, 96
    packed, scales = rand_weights(g, E, N, K)
    offs = np.array([10, 10, 41, 55], np.int32)
    x, go = g.standard_normal((T, K)), g.standard_normal((T, N))
    rows = np.array([0, 9, 10, 40, 41, 54, 55, 59])
    y, gx = oracle.grouped_mm_rows(rows, packed, scales, offs, x_rows=x[rows], g_rows=go[rows])
    assert np.array_equal(y, oracle.grouped_mm_fwd(x, packed, scales, offs)[rows])
    assert np.array_equal(gx, oracle.grouped_mm_bwd_x(go, packed, scales, offs)[rows])


def test_offsets_preconditions():
    g = np.random.default_rng(5)
    packed, scales = rand_weights(g, 2, 4, 32)
    x = g.standard_normal((6, 32))
    with pytest.raises(ValueError):
        oracle.grouped_mm_fwd(x, packed, scales, np.array([4, 3], np.int32))
    with pytest.raises(ValueError):
        oracle.grouped_mm_fwd(x, packed, scales, np.array([4, 7], np.int32))


# ---- W4A4 forward (activations through quantize_mxfp4 as well)

_GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # e2m1 magnitudes by code


def _brute_mxfp4_value(v, e):
    """Nearest e2m1 grid value of v / 2^e, ties to the even code, times 2^e,
    by search over the grid."""
    q = abs(v) / 2.0 ** e
    best = min(range(8), key=lambda c: (abs(q - _GRID[c]), c % 2))
    return (-1.0 if v < 0 else 1.0) * _GRID[best] * 2.0 ** e


def _brute_floor_exponent(amax):
    if amax == 0:
        return -127
    e = -200
    while 2.0 ** (e + 1) <= amax:   # largest e with 2^e <= amax
        e += 1
    return max(-127, min(127, e - 2))


def test_w4a4_matches_brute_force():
    """Per-element scalar quantization (exponent by search, nearest grid value
    with ties to the even code) and an explicit triple loop, on 2 experts."""
    g = np.random.default_rng(5)
    E, T, N, K = 2, 5, 3, 64
    packed, scales = rand_weights(g, E, N, K)
    x = g.standard_normal((T, K)) * np.repeat(2.0 ** g.integers(-6, 7, size=(T, K // 32)), 32, axis=1)
    # planted ties on the e2m1 grid (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 times the block scale),
    # filling the whole block, so its maximum 5 * 2^-3 fixes the scale exponent at -3
    x[0, :32] = np.tile([4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], 4) * 2.0 ** -3
    x[1, 32:] = 0.0                                          # an all-zero block
    x[2, 40] = 7.5 * 2.0 ** 4                                # saturating block maximum
    offs = np.array([2, 5], np.int32)
    y = oracle.grouped_mm_fwd_w4a4(x, packed, scales, offs)
    for t in range(T):
        e_t = 0 if t < 2 else 1
        xv = []
        for b in range(K // 32):
            blk = x[t, 32 * b:32 * b + 32]
            e = _brute_floor_exponent(max(abs(v) for v in blk))
            xv += [_brute_mxfp4_value(v, e) for v in blk]
        for n in range(N):
            acc = 0.0
            for k in range(K):
                byte = int(packed[e_t, n, k // 2]) & 0xFF
                nib = byte & 0xF if k % 2 == 0 else byte >> 4
                w = (-1.0 if nib & 8 else 1.0) * _GRID[nib & 7] * 2.0 ** (int(scales[e_t, n, k // 32]) - 127)
                acc += xv[k] * w
            assert abs(y[t, n] - acc) <= 1e-12 * max(1.0, abs(acc)), (t, n, y[t, n], acc)


def test_w4a4_on_grid_values_is_the_plain_forward():
    """Activations already on the MXFP4 grid (one round trip) are fixed points
    of the quantizer, so the W4A4 forward equals the plain forward exactly;
    off-grid activations do not."""
    g = np.random.default_rng(6)
    E, T, N, K = 3, 40, 16, 128
    packed, scales = rand_weights(g, E, N, K)
    offs = np.array([10, 10, 33], np.int32)
    x0 = g.standard_normal((T, K))
    xg = oracle.w4a4_activations(x0)
    assert np.array_equal(oracle.w4a4_activations(xg), xg)
    assert np.array_equal(oracle.grouped_mm_fwd_w4a4(xg, packed, scales, offs),
                          oracle.grouped_mm_fwd(xg, packed, scales, offs))
    assert not np.allclose(oracle.grouped_mm_fwd_w4a4(x0, packed, scales, offs),
                           oracle.grouped_mm_fwd(x0, packed, scales, offs))


# ----------------------------------------------------------------- W4A8
def _e4m3_grid():
    """All non-negative finite E4M3 (FN) values with their codes: subnormals
    m * 2^-9, normals (1 + m/8) * 2^(e-7), e = 1..15, without (15, 7) (NaN)."""
    vals = [(m * 2.0 ** -9, m) for m in range(8)]
    vals += [((1 + m / 8) * 2.0 ** (e - 7), (e << 3) | m) for e in range(1, 16) for m in range(8) if (e, m) != (15, 7)]
    return vals


def _brute_fp8_value(v, s):
    """v / s rounded to the nearest E4M3 value (ties to the even code) times s."""
    q = abs(v) / s
    best = min(_e4m3_grid(), key=lambda gc: (abs(q - gc[0]), gc[1] % 2))
    return (-1.0 if v < 0 else 1.0) * best[0] * s


def _brute_ceil_scale(amax):
    """Smallest power of two >= fl32(amax / 448), at least 2^-126, by search."""
    r = float(np.float32(np.float32(amax) / np.float32(448.0)))
    j = -126
    while 2.0 ** j < r:
        j += 1
    return 2.0 ** j


def test_w4a8_matches_brute_force():
    """Per-element scalar fp8 quantization (scale by search, nearest E4M3
    value with ties to the even code, subnormals included) and an explicit
    triple loop, on 2 experts."""
    g = np.random.default_rng(15)
    E, T, N, K = 2, 5, 3, 64
    packed, scales = rand_weights(g, E, N, K)
    x = g.standard_normal((T, K)) * np.repeat(2.0 ** g.integers(-30, 30, size=(T, K // 32)), 32, axis=1)
    # ties of the E4M3 grid (midpoints between neighbours, 1.0625 = 1 + 1/16)
    # under a block maximum 448 that fixes the scale at 1
    x[0, :32] = np.tile([448.0, 1.0625, 1.1875, 3.0 * 2.0 ** -10, 0.5 * 2.0 ** -9, 9.0, 17.0, 240.0], 4)
    x[1, 32:] = 0.0                                          # an all-zero block
    x[2, :32] *= 2.0 ** -140                                 # tiny block: the 2^-126 floor
    offs = np.array([2, 5], np.int32)
    y = oracle.grouped_mm_fwd_w4a8(x, packed, scales, offs)
    for t in range(T):
        e_t = 0 if t < 2 else 1
        xv = []
        for b in range(K // 32):
            blk = x[t, 32 * b:32 * b + 32]
            s = _brute_ceil_scale(max(abs(v) for v in blk))
            xv += [_brute_fp8_value(v, s) for v in blk]
        for n in range(N):
            acc = 0.0
            for k in range(K):
                byte = int(packed[e_t, n, k // 2]) & 0xFF
                nib = byte & 0xF if k % 2 == 0 else byte >> 4
                w = (-1.0 if nib & 8 else 1.0) * _GRID[nib & 7] * 2.0 ** (int(scales[e_t, n, k // 32]) - 127)
                acc += xv[k] * w
            assert abs(y[t, n] - acc) <= 1e-12 * max(1.0, abs(acc)), (t, n, y[t, n], acc)


def test_w4a8_activations_are_the_fp8_cache_round_trip():
    """The activations equal quantize_cache's fp8 fake-quant at block 32
    (the values its packed form decodes to), and sit within half an E4M3
    step of x: |q - x| <= 2^-4 |x| for normal values, <= 2^-10 s below."""
    g = np.random.default_rng(16)
    x = g.standard_normal((64, 256)) * np.repeat(2.0 ** g.integers(-20, 20, size=(64, 8)), 32, axis=1)
    q = oracle.w4a8_activations(x)
    assert np.array_equal(q, oracle.cache.quantize_cache_values(x, "fp8", 32))
    s = np.repeat(oracle.cache_scale(np.max(np.abs(x.reshape(64, 8, 32)), axis=-1), "fp8"), 32, axis=1)
    normal = np.abs(x) >= 2.0 ** -6 * s
    assert np.all(np.abs(q - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal])
    assert np.all(np.abs(q - x)[~normal] <= 2.0 ** -10 * s[~normal])


def test_w4a8_on_grid_values_is_the_plain_forward():
    """Activations already on the fp8 grid (one round trip) are fixed points
    of the quantizer, so the W4A8 forward equals the plain forward exactly;
    off-grid activations do not."""
    g = np.random.default_rng(17)
    E, T, N, K = 3, 40, 16, 128
    packed, scales = rand_weights(g, E, N, K)
    offs = np.array([10, 10, 33], np.int32)
    x0 = g.standard_normal((T, K))
    xg = oracle.w4a8_activations(x0)
    assert np.array_equal(oracle.w4a8_activations(xg), xg)
    assert np.array_equal(oracle.grouped_mm_fwd_w4a8(xg, packed, scales, offs),
                          oracle.grouped_mm_fwd(xg, packed, scales, offs))
    assert not np.allclose(oracle.grouped_mm_fwd_w4a8(x0, packed, scales, offs),
                           oracle.grouped_mm_fwd(x0, packed, scales, offs))
