"""Pins for oracle/nvfp4.py (two-level NVFP4, "NVIDIA Model Optimizer: from
mtq.quantize to a 4.95-bit DeepSeek-R1", section "NVFP4 in the code: two
scales and a nibble"): the E4M3 encode/decode against PyTorch's
float8_e4m3fn, the two facts the page states about the scales (the block
holding the tensor's maximum gets exactly 448; block maxima land between about
5.6 and 6.4 times the divisor), an exact round trip on representable values,
the zero-scale rule, power-of-two scale invariance and the error bound."""

import numpy as np
import pytest
import torch

import oracle
from oracle.nvfp4 import NVFP4_BLOCK

F8 = getattr(torch, "float8_e4m3fn", None)
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def rand_tensor(seed, shape, outliers=0.0):
    g = np.random.default_rng(seed)
    scale = np.exp2(g.integers(-6, 7, size=shape[:-1] + (shape[-1] // 16,)))
    x = g.standard_normal(shape) * np.repeat(scale, 16, axis=-1)
    if outliers:
        m = g.random(shape) < outliers
        x[m] *= 40.0
    return x.astype(np.float32).astype(np.float64)


@pytest.mark.skipif(F8 is None, reason="torch without float8_e4m3fn")
def test_e4m3_codec_matches_torch():
    bits = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(bits).view(F8).to(torch.float32).numpy().astype(np.float64)
    got = oracle.e4m3_decode(bits)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    pos = bits[(bits < 0x7F)]
    assert np.array_equal(oracle.e4m3_bits(oracle.e4m3_decode(pos)), pos)


@pytest.mark.skipif(F8 is None, reason="torch without float8_e4m3fn")
def test_e4m3_cast_of_block_ratios_matches_torch():
    """The scale cast: fp32 ratios in [2^-9, 448], nearest-even, subnormals included."""
    g = np.random.default_rng(3)
    r = np.exp2(g.uniform(-9, np.log2(448.0), 200000)).astype(np.float32)
    grid = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)       # every rounding tie, exactly
    r = np.concatenate([r, mids[mids >= 2.0 ** -9], np.float32([2.0 ** -9, 448.0])])
    want = torch.from_numpy(r).to(F8).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_bits(oracle.formats.e4m3_round(r.astype(np.float64))), want)


def test_block_holding_the_maximum_gets_448():
    for seed in range(20):
        x = rand_tensor(seed, (7, 96), outliers=0.01)
        packed, sb, g = oracle.quantize_nvfp4(x)
        r, b = np.unravel_index(np.argmax(np.abs(x)), x.shape)
        assert sb[r, b // NVFP4_BLOCK] == 0x7E                     # 448 = 1.75 * 2^8
        assert oracle.e4m3_decode(sb).max() == 448.0


def test_block_maxima_land_between_5_6_and_6_4():
    """A block's largest |x| over its divisor s_b g is within the E4M3
    rounding of the scale from 6: [6 / (1 + 1/16), 6 / (1 - 1/16)] (page:
    about 5.6 to 6.4, from the scale's 3 mantissa bits), for every block whose
    ratio is in E4M3's normal range (below 2^-6 the subnormal spacing is
    coarser, and below 2^-9 the clamp binds)."""
    x = rand_tensor(11, (64, 256), outliers=0.005)
    packed, sb, g = oracle.quantize_nvfp4(x)
    s = oracle.e4m3_decode(sb)
    d = (s.astype(np.float32) * g).astype(np.float32).astype(np.float64)
    amax_b = np.max(np.abs(x.reshape(64, -1, 16)), axis=-1)
    ratio = amax_b / (6.0 * float(g))
    free = ratio >= 2.0 ** -6
    assert free.mean() > 0.5
    t = amax_b[free] / d[free]
    assert t.min() >= 6 / (1 + 1 / 16) - 1e-5 and t.max() <= 6 / (1 - 1 / 16) + 1e-5
    assert t.min() < 5.8 and t.max() > 6.2                         # both ends are reached


def test_round_trip_of_representable_values_is_exact():
    """g = 2^t exactly when the tensor max is 6 * 448 * 2^t; blocks whose
    values are e2m1 grid values times 448 * 2^t or 2^(j+t) (j in -9..8) have
    exact scales and divisors, so they come back bit for bit."""
    g = np.random.default_rng(5)
    for t in (-20, 0, 13):
        rows, nb = 6, 10
        x = np.zeros((rows, nb * 16))
        for r in range(rows):
            for b in range(nb):
                vals = GRID[g.integers(0, 8, 16)] * np.where(g.random(16) < 0.5, -1.0, 1.0)
                vals[g.integers(0, 16)] = 6.0                       # each block reaches 6 * its scale
                scale = 448.0 if (r, b) == (0, 0) else 2.0 ** int(g.integers(-9, 8))
                x[r, 16 * b:16 * b + 16] = vals * scale * 2.0 ** t
        packed, sb, gs = oracle.quantize_nvfp4(x)
        assert gs == np.float32(2.0 ** t)
        assert np.array_equal(oracle.dequantize_nvfp4_values(packed, sb, gs), x)


def test_zero_scale_rule_and_zero_tensor():
    x = rand_tensor(2, (3, 64))
    x[1, 16:32] = 0.0                                              # one all-zero block
    packed, sb, g = oracle.quantize_nvfp4(x)
    assert sb[1, 1] == 0x38                                        # zero scale -> 1.0
    assert np.all(packed[1, 8:16] == 0)
    # the all-zero tensor: g = 0, every scale 1.0, every code 0 (reading)
    packed, sb, g = oracle.quantize_nvfp4(np.zeros((2, 32)))
    assert g == 0 and np.all(sb == 0x38) and np.all(packed == 0)
    assert np.all(oracle.dequantize_nvfp4_values(packed, sb, g) == 0)


def test_power_of_two_scaling_moves_only_the_global_scale():
    x = rand_tensor(8, (5, 128), outliers=0.01)
    p0, s0, g0 = oracle.quantize_nvfp4(x)
    for t in (-30, -1, 7, 40):
        p1, s1, g1 = oracle.quantize_nvfp4(x * 2.0 ** t)
        assert g1 == np.float32(g0 * 2.0 ** t)
        assert np.array_equal(p1, p0) and np.array_equal(s1, s0)


def test_error_bound():
    """Within a block an element moves by at most half the widest grid gap
    (2 -> 1) times the divisor d = s_b g while |x| / d <= 6, and by its
    overshoot past 6 beyond that (the cast saturates): at most
    d * max(1, amax_b / d - 6).  With a normal-range scale the overshoot is
    below 0.4, so the bound is d."""
    x = rand_tensor(9, (32, 512), outliers=0.01)
    packed, sb, g = oracle.quantize_nvfp4(x)
    v = oracle.dequantize_nvfp4_values(packed, sb, g)
    d = (oracle.e4m3_decode(sb).astype(np.float32) * g).astype(np.float32).astype(np.float64)
    amax_b = np.max(np.abs(x.reshape(32, -1, 16)), axis=-1)
    bound = d * np.maximum(1.0, amax_b / d - 6.0)
    err = np.abs(v - x).reshape(32, -1, 16)
    assert np.all(err <= bound[..., None] * (1 + 1e-6))
    normal = amax_b / (6.0 * float(g)) >= 2.0 ** -6
    assert np.all(err[normal] <= d[normal][..., None] * (1 + 1e-6))


def test_nibble_order_and_shapes():
    x = np.zeros((1, 16))
    x[0, 0], x[0, 1] = 6.0, -0.5 * 6.0 / 6.0       # codes 7 (6.0) and 9 (-0.5)
    packed, sb, g = oracle.quantize_nvfp4(x)
    assert packed.shape == (1, 8) and sb.shape == (1, 1)
    assert packed[0, 0] == (7 | (9 << 4))
    with pytest.raises(ValueError):
        oracle.quantize_nvfp4(np.zeros((1, 24)))


# ---- MSE block-scale rule ("Where the scales come from", NVFP4's own rules)

E4M3_POS = oracle.e4m3_decode(np.arange(1, 0x7F, dtype=np.uint8))     # the 126 candidates


def _exact_errors(block, g):
    """Squared error (fp64) of one 16-block under each of the 126 candidates,
    rounding x / d to the nearest e2m1 value (ties to the even code) in fp64:
    an implementation independent of the oracle's fp32 steps."""
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    out = []
    for s in E4M3_POS:
        d = float(np.float32(np.float32(s) * np.float32(g)))
        q = np.abs(block) / d
        dist = np.abs(q[:, None] - grid[None, :])
        best = dist.min(axis=1, keepdims=True)
        cand = np.where(dist == best, np.arange(8)[None, :], 99)
        even = np.where(cand % 2 == 0, cand, 99).min(axis=1)      # ties: the even code
        idx = np.where(np.sum(dist == best, axis=1) > 1, even, cand.min(axis=1))
        xhat = np.sign(block) * grid[idx] * d
        out.append(float(np.sum((block - xhat) ** 2)))
    return np.array(out)


def test_mse_scale_is_the_least_error_candidate_by_brute_force():
    x = rand_tensor(21, (4, 256), outliers=0.01)
    packed, sb, g = oracle.quantize_nvfp4_mse(x)
    blocks = x.reshape(4, 16, 16)
    for r in range(4):
        for b in range(16):
            errs = _exact_errors(blocks[r, b], g)
            chosen = errs[int(sb[r, b]) - 1]
            assert chosen <= errs.min() * (1 + 1e-5) + 1e-300, (r, b, int(sb[r, b]), int(np.argmin(errs)) + 1)


def test_mse_never_worse_than_the_max_rule():
    """The max rule's scale is one of the 126 candidates, so the chosen
    block's fp32 error is at most the max rule's, block by block; the sweep
    also changes most blocks' scales and lowers the total error."""
    x = rand_tensor(22, (32, 512), outliers=0.005)
    p_m, s_m, g = oracle.quantize_nvfp4_mse(x)
    p_x, s_x, g_x = oracle.quantize_nvfp4(x)
    assert g == g_x
    blocks = x.astype(np.float32).reshape(32, 32, 16)
    e_m, _ = oracle.nvfp4_block_sq_errors(blocks, g, oracle.e4m3_decode(s_m))
    e_x, _ = oracle.nvfp4_block_sq_errors(blocks, g, oracle.e4m3_decode(s_x))
    assert np.all(e_m <= e_x)
    nz = e_x > 0
    assert (s_m != s_x).mean() > 0.3 and e_m.sum() < e_x.sum() and np.median(e_m[nz] / e_x[nz]) < 0.9
    # the stored codes are the two-level encoding under the chosen scales
    v = oracle.dequantize_nvfp4_values(p_m, s_m, g)
    assert np.allclose(((v - x) ** 2).reshape(32, 32, 16).sum(-1), e_m, rtol=1e-5, atol=0)


def test_mse_exact_blocks_come_back_exactly_with_the_first_exact_scale():
    """Blocks of e2m1 grid values times an E4M3 value s and g = 2^t are
    quantized without error; the scale kept is the smallest code that is
    exact (a smaller scale that also represents the block wins)."""
    g0 = np.random.default_rng(23)
    t = -4
    rows = []
    rows.append(np.concatenate([[6.0 * 448.0], np.zeros(15)]) * 2.0 ** t)       # sets g = 2^t
    for code in (0x01, 0x05, 0x21, 0x38, 0x4B, 0x7E):
        s = float(oracle.e4m3_decode(np.uint8(code)))
        vals = GRID[g0.integers(0, 8, 16)] * np.where(g0.random(16) < 0.5, -1.0, 1.0)
        rows.append(vals * s * 2.0 ** t)
    x = np.stack(rows)
    packed, sb, g = oracle.quantize_nvfp4_mse(x)
    assert g == np.float32(2.0 ** t)
    assert np.array_equal(oracle.dequantize_nvfp4_values(packed, sb, g), x)
    for r in range(x.shape[0]):
        errs = _exact_errors(x[r], g)
        assert errs[int(sb[r, 0]) - 1] == 0 and np.all(errs[: int(sb[r, 0]) - 1] > 0)


def test_mse_zero_block_zero_tensor_and_subnormal_scales():
    x = rand_tensor(24, (2, 64))
    x[0, 16:32] = 0.0
    gx = np.float32(np.abs(x).max()) / np.float32(2688.0)
    x[1, 0:16] *= 6.0 * float(gx) * 2.0 ** -8 / np.abs(x[1, 0:16]).max()   # block ratio 2^-8: an E4M3 subnormal scale
    x = x.astype(np.float32).astype(np.float64)
    packed, sb, g = oracle.quantize_nvfp4_mse(x)
    assert sb[0, 1] == 0x01 and np.all(packed[0, 8:16] == 0)        # every candidate is exact: the first
    assert sb[1, 0] < 0x08                                          # subnormal candidates are in the sweep
    errs = _exact_errors(x[1, :16], g)
    assert errs[int(sb[1, 0]) - 1] <= errs.min() * (1 + 1e-5)
    packed, sb, g = oracle.quantize_nvfp4_mse(np.zeros((2, 32)))
    assert g == 0 and np.all(sb == 0x38) and np.all(packed == 0)


def test_mse_power_of_two_scaling_moves_only_the_global_scale():
    x = rand_tensor(25, (6, 128), outliers=0.01)
    p0, s0, g0 = oracle.quantize_nvfp4_mse(x)
    for t in (-20, -3, 5, 30):
        p1, s1, g1 = oracle.quantize_nvfp4_mse(x * 2.0 ** t)
        assert g1 == np.float32(g0 * 2.0 ** t)
        assert np.array_equal(s1, s0) and np.array_equal(p1, p0)


def test_mse_fused_residual_is_exact_in_float64():
    """The oracle forms the fused residual x - e2m1 * d in float64 and rounds
    it once to fp32; that equals the fused multiply-add only if the float64
    difference is exact.  Checked with exact rationals over every candidate
    of blocks whose quotients saturate (small scales) or round to zero."""
    from fractions import Fraction
    x = rand_tensor(26, (2, 64), outliers=0.05)
    g = oracle.nvfp4_global_scale(x)
    blocks = x.astype(np.float32).reshape(2, 4, 16)
    for code in range(1, 0x7F):
        s = np.full((2, 4), oracle.e4m3_decode(np.uint8(code)))
        d = (s.astype(np.float32) * np.float32(g)).astype(np.float32)
        codes = oracle.nvfp4._codes_for_scales(blocks, g, s)
        vd = oracle.E2M1_TABLE[codes.astype(np.int64)] * d.astype(np.float64)[..., None]
        diff = blocks.astype(np.float64) - vd
        for xi, vi, di, df in zip(blocks.reshape(-1), oracle.E2M1_TABLE[codes.astype(np.int64)].reshape(-1),
                                  np.repeat(d.reshape(-1), 16), diff.reshape(-1)):
            assert Fraction(float(xi)) - Fraction(float(vi)) * Fraction(float(di)) == Fraction(float(df))
