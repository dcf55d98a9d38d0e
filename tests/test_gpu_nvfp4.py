"""GPU parity of two-level NVFP4 (quantize_nvfp4, dequantize_nvfp4) against the
CPU oracle, bit for bit: the global scale, the E4M3 block scales, the codes and
the dequantized values on random tensors of every dtype (outliers, zero
blocks, wide binade spreads that hit the scale clamp), exact e2m1 ties, the
all-zero tensor, misaligned buffers (the general path), every code byte under
every finite scale byte, and the bf16 [65536, 7168] stream on sampled rows."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import nvfp4_quantization_grouped_amd as mxq
from tests.gpu_util import DTYPES, assert_bits_equal, bits_of, dev, from_gpu_bits, to_gpu_bits
from tests.test_gpu_codec import random_blocks

pytestmark = pytest.mark.gpu

_DT = {"f32": 0, "bf16": 1, "f16": 2}


def f32_bits(v):
    return int(np.float32(v).view(np.uint32))


def normal_blocks(seed, rows, k, dtype, outliers=0.002):
    g = np.random.default_rng(seed)
    scale = np.exp2(g.integers(-6, 7, size=(rows, k // 16)))
    v = g.standard_normal((rows, k)) * np.repeat(scale, 16, axis=1)
    m = g.random((rows, k)) < outliers
    v[m] *= 50.0
    v[g.random((rows, k // 16)).repeat(16, axis=1) < 0.01] = 0.0      # zero blocks
    if dtype == "f16":
        v = np.clip(v, -6e4, 6e4)
    return bits_of(v.astype(np.float32), dtype)


def check_all(xb, dtype, what, gpu_x=None):
    x = oracle.from_dtype_bits(xb, dtype)
    wp, ws, wg = oracle.quantize_nvfp4(x)
    p, s, g = mxq.quantize_nvfp4(to_gpu_bits(xb, dtype) if gpu_x is None else gpu_x)
    assert f32_bits(g.item()) == f32_bits(wg), f"{what}: global scale {g.item()!r} vs {wg!r}"
    assert_bits_equal(from_gpu_bits(p), wp, f"{what} packed")
    assert_bits_equal(from_gpu_bits(s.view(torch.uint8)), ws, f"{what} block scales")
    for od in ("f32", "bf16", "f16"):
        back = mxq.dequantize_nvfp4(p, s, g, DTYPES[od])
        assert_bits_equal(from_gpu_bits(back), oracle.dequantize_nvfp4(wp, ws, wg, od), f"{what} dequant {od}")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("rows,k", [(1, 16), (7, 48), (33, 1024), (5, 7168), (300, 512)])
def test_random_tensors_bit_exact(dtype, rows, k):
    check_all(normal_blocks(rows * k + len(dtype), rows, k, dtype), dtype, f"{dtype} [{rows},{k}]")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_wide_binade_spread_hits_the_clamp(dtype):
    """Blocks spread over the whole exponent range of the dtype: most block
    ratios fall below 2^-9 (clamped) or into E4M3's subnormals."""
    g = np.random.default_rng(4)
    xb = random_blocks(g, 4096, 16, dtype).reshape(256, 256)
    check_all(xb, dtype, f"{dtype} wide spread")


def test_exact_ties_and_zero_tensor():
    """g = 2^t when the tensor max is 6 * 448 * 2^t; blocks with max 6 * 2^j get
    s_b = 2^j and a power-of-two divisor, so x = m * d for each e2m1 midpoint m
    is an exact tie (0.25, 1.25, 2.5, 5 stay down; 0.75, 1.75, 3.5 move up)."""
    t = -3
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    rows = []
    rows.append(np.concatenate([[6.0 * 448.0 * 2.0 ** t], np.zeros(15)]))
    for j in range(-9, 9):
        blk = np.concatenate([[6.0], mids, -mids, [0.0]]) * 2.0 ** (j + t)
        rows.append(blk)
    x = np.stack(rows)
    for dtype in ("f32", "bf16"):
        check_all(bits_of(x.astype(np.float32), dtype), dtype, f"ties {dtype}")
    zb = bits_of(np.zeros((4, 64), np.float32), "bf16")
    check_all(zb, "bf16", "all-zero tensor")
    p, s, g = mxq.quantize_nvfp4(to_gpu_bits(zb, "bf16"))
    assert g.item() == 0.0 and torch.all(s.view(torch.uint8) == 0x38) and torch.all(p == 0)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_tensor_max_sharing_a_factor_with_2688(dtype):
    """A tensor max of 91 * 2^-4 (odd part 7 * 13; 2688 = 2^7 * 3 * 7) puts
    many quotients x / d exactly on e2m1 midpoints: in bf16 about 3% of the
    chunks hold one, beside elements the reciprocal bracket decides, so
    chunks mix both kinds (the block pass divides only where the bracket
    straddles).  Whole [1024, 2048] tensor."""
    g = np.random.default_rng(91)
    v = np.clip(g.standard_normal((1024, 2048)), -5.5, 5.5) * 2.0 ** (g.integers(-3, 1, size=(1024, 1)))
    v[17, 5] = 91.0 / 16.0
    check_all(bits_of(v.astype(np.float32), dtype), dtype, f"max 91/16 {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_misaligned_buffers_take_the_general_path(dtype):
    rows, k = 37, 96
    xb = normal_blocks(77, rows, k, dtype)
    x = oracle.from_dtype_bits(xb, dtype)
    wp, ws, wg = oracle.quantize_nvfp4(x)
    esz = 4 if dtype == "f32" else 2
    big = to_gpu_bits(np.concatenate([np.zeros(1, xb.dtype), xb.reshape(-1)]), dtype)   # x one element in
    pk = torch.zeros(rows * k // 2 + 3, dtype=torch.uint8, device=dev())
    sc = torch.zeros(rows * k // 16 + 1, dtype=torch.uint8, device=dev())
    gs = torch.zeros(2, dtype=torch.float32, device=dev())
    L = mxq.lib()
    st = torch.cuda.current_stream().cuda_stream
    assert L.quantize_nvfp4(big.data_ptr() + esz, _DT[dtype], rows, k, pk.data_ptr() + 1, sc.data_ptr() + 1,
                            gs.data_ptr() + 4, st) == 0
    assert f32_bits(gs[1].item()) == f32_bits(wg)
    assert_bits_equal(from_gpu_bits(pk[1:1 + rows * k // 2]).reshape(rows, -1), wp, "general packed")
    assert_bits_equal(from_gpu_bits(sc[1:]).reshape(rows, -1), ws, "general scales")
    out = torch.zeros(rows * k + 1, dtype=DTYPES[dtype], device=dev())
    assert L.dequantize_nvfp4(pk.data_ptr() + 1, sc.data_ptr() + 1, gs.data_ptr() + 4, rows, k,
                              out.data_ptr() + esz, _DT[dtype], st) == 0
    assert_bits_equal(from_gpu_bits(out[1:]).reshape(rows, k), oracle.dequantize_nvfp4(wp, ws, wg, dtype),
                      "general dequant")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_dequantize_every_code_byte_under_every_scale_byte(dtype):
    """254 finite E4M3 scale bytes (both signs) x all 256 code bytes, g = 0.0371;
    the two NaN scale bytes give NaN."""
    sbytes = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
    rows, k = len(sbytes), 512
    packed = np.tile(np.arange(256, dtype=np.uint8), (rows, 1))
    scales = np.repeat(sbytes[:, None], k // 16, axis=1)
    g = np.float32(0.0371)
    out = mxq.dequantize_nvfp4(torch.from_numpy(packed).to(dev()), torch.from_numpy(scales).to(dev()),
                               torch.tensor(g, device=dev()), DTYPES[dtype])
    assert_bits_equal(from_gpu_bits(out), oracle.dequantize_nvfp4(packed, scales, g, dtype), f"dequant {dtype}")
    nan_s = np.full((2, k // 16), 0x7F, np.uint8)
    nan_s[1] = 0xFF
    out = mxq.dequantize_nvfp4(torch.from_numpy(packed[:2]).to(dev()), torch.from_numpy(nan_s).to(dev()),
                               torch.tensor(g, device=dev()), torch.float32)
    assert torch.all(torch.isnan(out))


def test_mid_size_tensor_bf16():
    """bf16 [8192, 4096] (64 MB, the medium access mode) in full."""
    xb = normal_blocks(5, 8192, 4096, "bf16")
    check_all(xb, "bf16", "bf16 [8192,4096]")


@pytest.mark.timeout(900)
def test_bulk_stream_sampled_rows():
    """bf16 [65536, 7168] (the large access mode): the global scale against the
    oracle's over the whole tensor, 256 sampled rows' codes, scales and
    dequantized values against the oracle's encoding with that scale."""
    d = synth.bulk_stream(seed=0, with_weights=False)
    xb = d["x"]
    p, s, g = mxq.quantize_nvfp4(to_gpu_bits(xb, "bf16"))
    amax = oracle.from_dtype_bits(np.array([np.max(xb & np.uint16(0x7FFF))], np.uint16), "bf16")
    wg = oracle.nvfp4_global_scale(amax)
    assert f32_bits(g.item()) == f32_bits(wg)
    rows = np.sort(np.random.default_rng(3).choice(xb.shape[0], 256, replace=False))
    ri = torch.from_numpy(rows).to(dev())
    wp, ws = oracle.nvfp4_encode(oracle.from_dtype_bits(xb[rows], "bf16"), wg)
    assert_bits_equal(from_gpu_bits(p[ri]), wp, "bulk packed")
    assert_bits_equal(from_gpu_bits(s.view(torch.uint8)[ri]), ws, "bulk scales")
    back = mxq.dequantize_nvfp4(p, s, g, torch.bfloat16)
    assert_bits_equal(from_gpu_bits(back[ri]), oracle.dequantize_nvfp4(wp, ws, wg, "bf16"), "bulk dequant")
