"""Pins for oracle/mxfp4.py: hand-worked blocks, the floor rule's closed form and
invariant, the exact round trip the page claims for representable values,
exhaustive dequantization, and the error bound of the cast."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.mxfp4 import dequantize_mxfp4_values

HAND = os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")


def _num(v):
    return float.fromhex(v) if isinstance(v, str) else float(v)


def _block(nonzero, n=32):
    b = np.zeros(n)
    for k, v in nonzero.items():
        b[int(k)] = _num(v)
    return b


with open(HAND) as _f:
    _HAND = json.load(_f)


@pytest.mark.parametrize("case", _HAND["floor_rule"], ids=lambda c: c["name"])
def test_hand_worked_blocks(case):
    x = _block(case["nonzero"])[None, :]
    packed, scales = oracle.quantize_mxfp4(x)
    assert scales.tolist() == [[case["scale_byte"]]]
    assert packed.view(np.uint8).tobytes().hex() == case["packed_hex"]
    deq = dequantize_mxfp4_values(packed, scales)[0]
    want = _block(case["dequant_nonzero"])
    assert np.array_equal(deq, want)
    assert not np.any(np.signbit(deq[want == 0]))   # code 8 decodes to +0.0
    bits = oracle.dequantize_mxfp4(packed, scales, "f32")
    assert np.array_equal(bits.view(np.float32)[0].astype(np.float64), want)


def test_shapes_and_block_contract():
    x = np.random.default_rng(0).standard_normal((3, 5, 64))
    p, s = oracle.quantize_mxfp4(x)
    assert p.shape == (3, 5, 32) and p.dtype == np.int8
    assert s.shape == (3, 5, 2) and s.dtype == np.uint8
    with pytest.raises(ValueError):
        oracle.quantize_mxfp4(np.zeros((2, 48)))
    with pytest.raises(ValueError):
        oracle.quantize_mxfp4(np.array([[np.nan] * 32]))


def all_positive_finite_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint32)
    return (bits << 16).view(np.float32).astype(np.float64)


def test_floor_rule_invariant_exhaustive_bf16_amax():
    amax = all_positive_finite_bf16()
    e = oracle.floor_scale_exponent(amax)
    q = amax / np.ldexp(1.0, e)
    # the clamp at -127 binds exactly when floor(log2 amax) - 2 < -127, i.e. amax < 2^-125
    unclamped = amax >= 2.0 ** -125
    assert np.all((q[unclamped] >= 4) & (q[unclamped] < 8))
    assert np.all(e[~unclamped] == -127) and np.all(q[~unclamped] < 4)


def test_floor_rule_is_exact_below_powers_of_two():
    # largest fp32 below 8: an fp32 log2 rounds to 3.0; the exact floor is 2
    a = float(np.nextafter(np.float32(8.0), np.float32(0)))
    assert np.floor(np.log2(np.float32(a))) == 3.0
    assert oracle.floor_scale_exponent(np.array([a]))[0] == 0
    assert oracle.floor_scale_exponent(np.array([8.0]))[0] == 1


def test_zero_block_scale_and_clamp_range():
    assert oracle.floor_scale_exponent(np.array([0.0]))[0] == -127
    assert oracle.floor_scale_exponent(np.array([float(np.finfo(np.float32).max)]))[0] == 125


def test_representable_values_round_trip_exactly():
    """The page's reason for the floor rule: blocks whose values already lie on
    the e2m1 grid times a power of two come back value-exactly."""
    g = np.random.default_rng(3)
    grid = oracle.E2M1_TABLE
    for _ in range(200):
        t = int(g.integers(-120, 120))
        codes = g.integers(0, 16, size=(4, 32))
        x = grid[codes] * np.ldexp(1.0, t)
        p, s = oracle.quantize_mxfp4(x)
        assert np.array_equal(dequantize_mxfp4_values(p, s), x + 0.0)


def test_cast_error_bound():
    """|q - grid(q)| is at most half the grid spacing around q when q <= 6,
    and q - 6 when 6 < q < 8 (saturation)."""
    g = np.random.default_rng(4)
    x = g.standard_normal((64, 256)) * np.exp2(g.integers(-20, 20, (64, 1)))
    p, s = oracle.quantize_mxfp4(x)
    xh = dequantize_mxfp4_values(p, s)
    scale = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=-1)
    q, qh = np.abs(x) / scale, np.abs(xh) / scale
    half = np.where(q < 2, 0.25, np.where(q < 4, 0.5, 1.0))
    inside = q <= 6
    assert np.all(np.abs(q - qh)[inside] <= half[inside])
    assert np.all(qh[~inside] == 6.0)
    assert np.all(np.sign(xh) * np.sign(x) >= 0)


def e2m1_value_from_bits(code):
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = np.where(e == 0, m * 0.5, np.exp2(e - 1.0) * (1 + m * 0.5))
    return np.where(s == 1, -mag, mag) + 0.0   # +0.0 for code 8 (page table)


def test_dequant_exhaustive_bytes_times_scales():
    """All 256 packed bytes x all 256 scale bytes: 131072 values, against the
    e2m1 bit-field definition times PyTorch's float8_e8m0fnu decode."""
    b = np.arange(256, dtype=np.uint8)
    packed = np.repeat(b[None, :], 256, axis=0)           # [256 scales, 256 bytes]
    packed = packed.reshape(256, 16, 16)                  # 16 blocks of 16 bytes per row
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 16, axis=1)
    packed = packed.reshape(256, 256)
    got = dequantize_mxfp4_values(packed.view(np.int8), scales)           # [256, 512]
    lo = e2m1_value_from_bits(packed.astype(np.int64) & 15)
    hi = e2m1_value_from_bits(packed.astype(np.int64) >> 4)
    vals = np.stack([lo, hi], axis=-1).reshape(256, 512)
    sc = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    with np.errstate(invalid="ignore"):
        want = vals * sc[:, None]
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    # fp32 / bf16 / fp16 outputs against PyTorch's nearest-even casts of the fp32 values
    f32 = oracle.dequantize_mxfp4(packed.view(np.int8), scales, "f32").view(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        want32 = want.astype(np.float32)
    assert np.array_equal(np.isnan(f32), np.isnan(want32))
    assert np.array_equal(f32[ok], want32[ok])
    assert np.array_equal(np.signbit(f32[ok]), np.signbit(want32[ok]))
    t32 = torch.from_numpy(want32)
    bf = oracle.dequantize_mxfp4(packed.view(np.int8), scales, "bf16")
    want_bf = t32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf[ok], want_bf[ok])
    f16 = oracle.dequantize_mxfp4(packed.view(np.int8), scales, "f16")
    want_f16 = t32.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f16[ok], want_f16[ok])


def test_layout_size_ratio():
    """One scale byte per 16 packed bytes (32 columns), the mxfp4 analogue of
    the 1:8 ratio the ModelOpt article measures for nvfp4's 16-column blocks."""
    x = np.random.default_rng(5).standard_normal((7, 1024))
    p, s = oracle.quantize_mxfp4(x)
    assert p.size == 16 * s.size
