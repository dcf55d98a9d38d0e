"""Pins for oracle/cache.py: hand-worked blocks, the ceiling rule's closed form
and invariant, fixed points, PyTorch's float8_e4m3fn cast for the fp8 element
step, the zero-padded partial group, and the straight-through backward."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.cache import quantize_cache_values, FORMAT_FMAX

HAND = os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")
with open(HAND) as _f:
    _HAND = json.load(_f)


def _num(v):
    return float.fromhex(v) if isinstance(v, str) else float(v)


def _block(nonzero, n):
    b = np.zeros(n)
    for k, v in nonzero.items():
        b[int(k)] = _num(v)
    return b


@pytest.mark.parametrize("case", _HAND["ceil_rule"], ids=lambda c: c["name"])
def test_hand_worked_blocks(case):
    n = case["block"]
    x = _block(case["nonzero"], n)[None, :]
    out = quantize_cache_values(x, case["format"], n)[0]
    assert np.array_equal(out, _block(case["out_nonzero"], n))


def test_power_of_two_ceiling_exhaustive_bf16_normals():
    bits = np.arange(0x0080, 0x7F80, dtype=np.uint32)           # positive normal bf16
    v = (bits << 16).view(np.float32).astype(np.float64)
    s = oracle.power_of_two_ceiling(v)
    m, _ = np.frexp(s)
    assert np.all(m == 0.5)                                      # powers of two
    assert np.all(s >= v) and np.all(s / 2 < v)                  # the smallest such
    with pytest.raises(ValueError):
        oracle.power_of_two_ceiling(np.array([2.0 ** -127]))     # not a normal fp32


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "nvfp4"])
def test_ceiling_rule_invariant(fmt):
    """amax / s lies in (fmax/2, fmax] unless the 2^-126 floor or the nvfp4
    clamp binds, so an element never saturates."""
    fmax = FORMAT_FMAX[fmt]
    bits = np.arange(1, 0x7F80, dtype=np.uint32)
    bf = (bits << 16).view(np.float32).astype(np.float64)
    g = np.random.default_rng(7)
    rnd = np.abs(g.standard_normal(200000) * np.exp2(g.integers(-140, 127, 200000))).astype(np.float32)
    amax = np.concatenate([bf, rnd[rnd > 0].astype(np.float64)])
    s = oracle.cache_scale(amax, fmt)
    r = amax / s
    free = amax / fmax > 2.0 ** -126
    if fmt == "nvfp4":
        free &= (s > 2.0 ** -9) & (s < 2.0 ** 8)
    assert np.all((r[free] > fmax / 2) & (r[free] <= fmax))
    assert np.all(r <= fmax) if fmt != "nvfp4" else np.all(r[amax <= 6 * 256] <= fmax)


def test_fp32_ratio_agrees_with_exact_ceiling():
    """The ratio is formed in fp32 (the helper is specified on FP32 values);
    over every fp32 mantissa the result equals the exact smallest power of two
    2^k with fmax * 2^k >= amax."""
    mant = np.arange(1 << 23, dtype=np.uint32)
    for fmt in ("fp8", "mxfp4"):
        fmax = FORMAT_FMAX[fmt]
        for exp_field in (1, 90, 127, 200):
            amax = ((np.uint32(exp_field) << 23) | mant).view(np.float32).astype(np.float64)
            s = oracle.cache_scale(amax, fmt)
            k = np.ceil(np.log2(amax / fmax))           # float64 guess, then fixed exactly
            k = np.where(fmax * np.exp2(k - 1) >= amax, k - 1, k)
            k = np.where(fmax * np.exp2(k) < amax, k + 1, k)
            exact = np.maximum(np.exp2(k), 2.0 ** -126)
            assert np.array_equal(s, exact)


@pytest.mark.parametrize("fmt,block", [("fp8", 128), ("mxfp4", 32), ("nvfp4", 16)])
def test_grid_values_are_fixed_points(fmt, block):
    g = np.random.default_rng(8)
    for _ in range(100):
        t = int(g.integers(-8, 8))
        if fmt == "fp8":
            codes = g.integers(0, 256, size=(3, block)).astype(np.uint8)
            codes[(codes & 0x7F) == 0x7F] = 0
            grid = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        else:
            grid = oracle.E2M1_TABLE[g.integers(0, 16, size=(3, block))]
        x = grid * np.ldexp(1.0, t)
        out = quantize_cache_values(x, fmt, block)
        assert np.array_equal(out, x)


def test_fp8_elements_vs_torch_cast():
    g = np.random.default_rng(9)
    x = (g.standard_normal((64, 512)) * np.exp2(g.integers(-30, 30, (64, 1)))).astype(np.float32).astype(np.float64)
    out = quantize_cache_values(x, "fp8", 128)
    blocks = x.reshape(64, 4, 128)
    s = oracle.cache_scale(np.max(np.abs(blocks), axis=-1), "fp8")[..., None]
    q = torch.from_numpy((blocks / s).astype(np.float32))
    want = (q.to(torch.float8_e4m3fn).to(torch.float64).numpy() * s).reshape(64, 512)
    assert np.array_equal(out, want)
    assert np.array_equal(np.signbit(out), np.signbit(want))


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "nvfp4"])
def test_partial_group_equals_own_group(fmt):
    """A final partial group is zero-padded, which leaves its amax unchanged:
    it quantizes like a tensor holding just that group."""
    g = np.random.default_rng(10)
    x = g.standard_normal((5, 70))
    full = quantize_cache_values(x, fmt, 32)
    assert full.shape == x.shape
    head = quantize_cache_values(x[:, :64], fmt, 32)
    tail = quantize_cache_values(x[:, 64:], fmt, 6)
    assert np.array_equal(full[:, :64], head)
    assert np.array_equal(full[:, 64:], tail)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "nvfp4"])
def test_output_contract_and_error_bound(fmt):
    g = np.random.default_rng(11)
    xb = g.standard_normal((8, 256)).astype(np.float32)
    bits = torch.from_numpy(xb).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    x = oracle.from_dtype_bits(bits, "bf16")
    before = x.copy()
    out = oracle.quantize_cache(x, fmt, 16, "bf16")
    assert out.shape == x.shape and out.dtype == np.uint16
    assert np.array_equal(x, before)                              # input not modified
    y = oracle.from_dtype_bits(out, "bf16")
    blocks = x.reshape(8, 16, 16)
    s = np.repeat(oracle.cache_scale(np.max(np.abs(blocks), -1), fmt), 16, axis=-1)
    err = np.abs(y - x) / s
    bound = 1.0 if fmt != "fp8" else 16.0    # half the widest grid step (2 in [4,6]; 32 in [256,448])
    assert np.all(err <= bound)


def test_nvfp4_scale_clamp_to_e4m3_range():
    x = np.zeros((1, 16))
    x[0, 0] = 6000.0                  # amax/6 = 1000 -> ceiling 1024, clamped to 256
    out = quantize_cache_values(x, "nvfp4", 16)
    assert out[0, 0] == 6 * 256.0     # saturates at the largest e2m1 value
    x[0, 0] = 2.0 ** -20              # ceiling 2^-22 -> clamped up to 2^-9
    out = quantize_cache_values(x, "nvfp4", 16)
    assert out[0, 0] == 0.0


def test_straight_through_backward_identity():
    g = np.random.default_rng(12).standard_normal((4, 3, 32))
    gi, b, f = oracle.quantize_cache_backward(g)
    assert gi is g and b is None and f is None


def test_bad_arguments():
    with pytest.raises(ValueError):
        quantize_cache_values(np.zeros((2, 32)), "int4", 32)
    with pytest.raises(ValueError):
        quantize_cache_values(np.zeros((2, 32)), "fp8", 0)


# ---- packed KV-cache storage: the codes and scales the fake-quant goes through

PACKED_CASES = [("fp8", 8), ("fp8", 24), ("fp8", 128), ("mxfp4", 8), ("mxfp4", 32), ("mxfp4", 512),
                ("nvfp4", 16), ("nvfp4", 64), ("nvfp4", 6)]


def _wide(seed, rows, cols, block, spread=40):
    g = np.random.default_rng(seed)
    t = g.integers(-spread, spread, (rows, cols // block))
    x = g.standard_normal((rows, cols)) * np.repeat(np.exp2(t), block, axis=1)
    x[g.random((rows, cols)) < 0.01] = 0.0
    x[g.random((rows, cols)) < 0.01] = -0.0
    return x.astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("fmt,block", PACKED_CASES)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_packed_round_trip_equals_fake_quant(fmt, block, dtype):
    """Decoding the stored codes and scales (table / E4M3 decode / 2^(b-127))
    gives the fake-quantized tensor bit for bit, signed zeros included."""
    x = _wide(block + len(fmt), 6, 48 * block, block)
    if dtype == "f16":
        x = np.clip(x, -6e4, 6e4)
    xb = oracle.to_dtype_bits(x, dtype)
    xv = oracle.from_dtype_bits(xb, dtype)
    codes, scales = oracle.quantize_cache_packed(xv, fmt, block)
    assert codes.shape == (6, 48 * block // (1 if fmt == "fp8" else 2)) and scales.shape == (6, 48)
    assert codes.dtype == np.uint8 and scales.dtype == np.uint8
    back = oracle.dequantize_cache_packed(codes, scales, fmt, block, dtype)
    assert np.array_equal(back, oracle.quantize_cache(xv, fmt, block, dtype))


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "nvfp4"])
def test_packed_scale_bytes_hold_the_ceiling(fmt):
    """The stored scale is the smallest power of two s with amax <= s * fmax
    (floored at 2^-126; nvfp4 clamped to 2^-9 .. 2^8), read back from its byte
    independently: E8M0 as 2^(b-127), E4M3 through PyTorch's float8_e4m3fn."""
    x = _wide(3, 16, 512, 32, spread=12 if fmt == "nvfp4" else 40)
    codes, scales = oracle.quantize_cache_packed(x, fmt, 32)
    if fmt == "nvfp4":
        s = torch.from_numpy(scales).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    else:
        s = np.ldexp(1.0, scales.astype(np.int64) - 127)
    fmax = FORMAT_FMAX[fmt]
    amax = np.max(np.abs(x.reshape(16, 16, 32)), axis=-1)
    m, _ = np.frexp(s)
    assert np.all(m == 0.5)                                       # powers of two
    lo, hi = (2.0 ** -9, 2.0 ** 8) if fmt == "nvfp4" else (2.0 ** -126, np.inf)
    free = (s > lo) & (s < hi)
    assert free.mean() > 0.5
    assert np.all(amax[free] <= s[free] * fmax) and np.all(amax[free] > s[free] / 2 * fmax)
    assert np.all(s >= lo) and np.all(s <= hi)


def test_packed_fp8_codes_are_torchs_cast():
    x = _wide(4, 32, 1024, 128)
    codes, scales = oracle.quantize_cache_packed(x, "fp8", 128)
    s = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 128, axis=1)
    want = torch.from_numpy((x / s).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, want)


def test_packed_hand_block():
    """amax 6 gives s = 1 (E8M0 127, E4M3 0x38): 6.0 -> code 7 and -0.5 -> code 9
    share byte 0 (even channel low); -0.0 -> code 0; -0.1 rounds to a signed
    zero, code 8, which decodes to +0.0.  fp8: amax 6 -> s = 2^-6 (byte 121)."""
    x = np.zeros((1, 16))
    x[0, :4] = [6.0, -0.5, -0.0, -0.1]
    for fmt, sbyte in (("mxfp4", 127), ("nvfp4", 0x38)):
        codes, scales = oracle.quantize_cache_packed(x, fmt, 16)
        assert codes[0, 0] == 0x97 and codes[0, 1] == 0x80 and np.all(codes[0, 2:] == 0) and scales[0, 0] == sbyte
        back = oracle.dequantize_cache_packed(codes, scales, fmt, 16, "f32")
        assert back[0, 3] == 0 and not np.signbit(oracle.from_dtype_bits(back, "f32")[0, 3])
    codes, scales = oracle.quantize_cache_packed(x, "fp8", 16)
    # x / 2^-6: 384 = 1.5 * 2^8 (0x7C), -32 = -2^5 (0xE0), -0.0 (0x80), -6.4 -> -6.5 = -1.625 * 2^2 (0xCD)
    assert scales[0, 0] == 121 and list(codes[0, :4]) == [0x7C, 0xE0, 0x80, 0xCD]


def test_packed_bad_arguments():
    with pytest.raises(ValueError):
        oracle.quantize_cache_packed(np.zeros((2, 40)), "fp8", 32)     # partial group
    with pytest.raises(ValueError):
        oracle.quantize_cache_packed(np.zeros((2, 42)), "mxfp4", 7)    # odd fp4 group
    with pytest.raises(ValueError):
        oracle.quantize_cache_packed(np.zeros((2, 32)), "int4", 32)
