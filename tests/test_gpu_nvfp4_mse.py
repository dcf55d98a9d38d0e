"""GPU parity of the NVFP4 MSE block-scale sweep (quantize_nvfp4_mse) against
the CPU oracle, bit for bit: global scale, chosen E4M3 block scales and codes
for fp32/bf16/f16 tensors with outliers and zero blocks, binade spreads that
reach E4M3's subnormal scales, exact e2m1 ties under power-of-two candidates,
the all-zero tensor, misaligned buffers, dequantization through
dequantize_nvfp4, and the bf16 [4096, 7168] weight on sampled rows."""

import numpy as np
import pytest
import torch

import oracle
import synth
import nvfp4_quantization_grouped_amd as mxq
from tests.gpu_util import DTYPES, assert_bits_equal, dev, from_gpu_bits, to_gpu_bits
from tests.test_gpu_codec import random_blocks
from tests.test_gpu_nvfp4 import f32_bits, normal_blocks

pytestmark = pytest.mark.gpu

_DT = {"f32": 0, "bf16": 1, "f16": 2}


def check(xb, dtype, what):
    x = oracle.from_dtype_bits(xb, dtype)
    wp, ws, wg = oracle.quantize_nvfp4_mse(x)
    p, s, g = mxq.quantize_nvfp4_mse(to_gpu_bits(xb, dtype))
    assert f32_bits(g.item()) == f32_bits(wg), f"{what}: global scale"
    assert_bits_equal(from_gpu_bits(s.view(torch.uint8)), ws, f"{what} block scales")
    assert_bits_equal(from_gpu_bits(p), wp, f"{what} packed")
    back = mxq.dequantize_nvfp4(p, s, g, DTYPES[dtype])
    assert_bits_equal(from_gpu_bits(back), oracle.dequantize_nvfp4(wp, ws, wg, dtype), f"{what} dequant")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("rows,k", [(1, 16), (7, 48), (33, 1024), (3, 7168)])
def test_random_tensors_bit_exact(dtype, rows, k):
    check(normal_blocks(rows * k + 3 * len(dtype), rows, k, dtype), dtype, f"mse {dtype} [{rows},{k}]")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_wide_binade_spread(dtype):
    """Blocks spread over the dtype's exponent range: most ratios fall in or
    below E4M3's subnormal scales, where the small candidates matter."""
    g = np.random.default_rng(41)
    check(random_blocks(g, 1024, 16, dtype).reshape(64, 256), dtype, f"mse {dtype} wide spread")


def test_exact_ties_zero_blocks_and_zero_tensor():
    """g = 2^t; blocks of e2m1 midpoints times 2^(j+t) put candidates' quotients
    exactly on midpoints (the tie path), and zero blocks take code 0x01."""
    t = -3
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    rows = [np.concatenate([[6.0 * 448.0 * 2.0 ** t], np.zeros(15)]), np.zeros(16)]
    for j in range(-9, 9):
        rows.append(np.concatenate([[6.0], mids, -mids, [0.0]]) * 2.0 ** (j + t))
    x = np.stack(rows).astype(np.float32)
    for dtype in ("f32", "bf16"):
        xb = x.view(np.uint32) if dtype == "f32" else (x.view(np.uint32) >> 16).astype(np.uint16)
        check(xb, dtype, f"mse ties {dtype}")
    zb = np.zeros((4, 64), np.uint16)
    check(zb, "bf16", "mse all-zero tensor")


def test_overflowing_errors_and_repeated_maxima():
    """Blocks whose squared errors overflow fp32 under most candidates (the
    sweep then ties at infinity and keeps the first code), blocks whose
    largest magnitude appears more than once with both signs, blocks of one
    repeated value, and single-value blocks that many candidates represent
    exactly (zero-error ties)."""
    g = np.random.default_rng(77)
    big = (g.uniform(-1.0, 1.0, (8, 64)) * 3.0e38).astype(np.float32)
    big[1, :16] = 3.0e38
    big[1, 16:32] = -3.0e38
    big[2] = (g.uniform(-1.0, 1.0, 64) * 1.0e20).astype(np.float32)
    big[3, 32:48] = 0.0
    big[3, 40] = 6.0 * 2.0 ** 100
    check(big.view(np.uint32), "f32", "mse overflowing errors")
    x = g.standard_normal((16, 64)).astype(np.float32)
    for b in range(x.size // 16):
        blk = x.reshape(-1, 16)[b]
        m = np.float32(1.5) * np.abs(blk).max()
        blk[b % 16] = m
        blk[(b + 5) % 16] = -m
        if b % 7 == 0:
            blk[:] = m
        if b % 11 == 0:
            blk[:] = 0.0
            blk[b % 16] = np.float32(3.0 * 2.0 ** (b % 5 - 2))
    for dtype in ("f32", "bf16"):
        xb = x.view(np.uint32) if dtype == "f32" else (x.view(np.uint32) >> 16).astype(np.uint16)
        check(xb, dtype, f"mse repeated maxima {dtype}")


def test_misaligned_input():
    rows, k = 21, 96
    xb = normal_blocks(43, rows, k, "bf16")
    x = oracle.from_dtype_bits(xb, "bf16")
    wp, ws, wg = oracle.quantize_nvfp4_mse(x)
    big = to_gpu_bits(np.concatenate([np.zeros(1, xb.dtype), xb.reshape(-1)]), "bf16")
    pk = torch.zeros(rows * k // 2 + 1, dtype=torch.uint8, device=dev())
    sc = torch.zeros(rows * k // 16 + 1, dtype=torch.uint8, device=dev())
    gs = torch.zeros(2, dtype=torch.float32, device=dev())
    st = torch.cuda.current_stream().cuda_stream
    assert mxq.lib().quantize_nvfp4_mse(big.data_ptr() + 2, 1, rows, k, pk.data_ptr() + 1, sc.data_ptr() + 1,
                                        gs.data_ptr() + 4, st) == 0
    assert f32_bits(gs[1].item()) == f32_bits(wg)
    assert_bits_equal(from_gpu_bits(pk[1:]).reshape(rows, -1), wp, "misaligned packed")
    assert_bits_equal(from_gpu_bits(sc[1:]).reshape(rows, -1), ws, "misaligned scales")


def test_weight_workload_sampled_rows():
    """bf16 [4096, 7168]: the global scale over the whole weight, 48 sampled
    rows' scales and codes against the oracle's sweep with that g; the total
    squared error is below the max rule's."""
    wb = synth.nvfp4_weight(seed=0)["w"]
    t = to_gpu_bits(wb, "bf16")
    p, s, g = mxq.quantize_nvfp4_mse(t)
    amax = oracle.from_dtype_bits(np.array([np.max(wb & np.uint16(0x7FFF))], np.uint16), "bf16")
    wg = oracle.nvfp4_global_scale(amax)
    assert f32_bits(g.item()) == f32_bits(wg)
    rows = np.sort(np.random.default_rng(7).choice(wb.shape[0], 48, replace=False))
    ri = torch.from_numpy(rows).to(dev())
    xr = oracle.from_dtype_bits(wb[rows], "bf16")
    ws = oracle.nvfp4_mse_block_scales(xr, wg)
    assert_bits_equal(from_gpu_bits(s.view(torch.uint8)[ri]), ws, "weight scales")
    pm, sm, gm = mxq.quantize_nvfp4(t)
    w = t.float()
    err_mse = ((mxq.dequantize_nvfp4(p, s, g, torch.float32) - w) ** 2).sum().item()
    err_max = ((mxq.dequantize_nvfp4(pm, sm, gm, torch.float32) - w) ** 2).sum().item()
    assert err_mse < err_max
    # the sampled rows' codes: the two-level encoding under the chosen scales
    blocks = xr.astype(np.float32).reshape(len(rows), -1, 16)
    codes = oracle.e2m1_encode(
        (blocks / (oracle.e4m3_decode(ws).astype(np.float32) * np.float32(wg)).astype(np.float32)[..., None])
        .astype(np.float32).astype(np.float64)).reshape(len(rows), -1)
    want = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    assert_bits_equal(from_gpu_bits(p[ri]), want, "weight codes")
