"""GPU parity of the codec kernels (quantize_mxfp4, dequantize_mxfp4,
quantize_cache, straight-through backward) against the CPU oracle: bit-exact
on seeded inputs, exhaustive byte x scale grids, hand-worked blocks, ragged
and misaligned shapes, and the full-size workloads (sampled rows)."""

import json
import os
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
import nvfp4_quantization_grouped_amd as mxq
from tests.gpu_util import DTYPES, assert_bits_equal, bits_of, dev, from_gpu_bits, to_gpu_bits

pytestmark = pytest.mark.gpu

HAND = os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")


def nan_of(dtype):
    if dtype == "f32":
        return lambda b: np.isnan(b.view(np.float32))
    return lambda b: np.isnan(oracle.from_dtype_bits(b, dtype))


def random_blocks(g, nblocks, block, dtype):
    """Blocks whose elements share a random binade (so every code and tie
    occurs), including zeros, negative zeros and subnormals."""
    lo = {"f32": -148, "bf16": -132, "f16": -24}[dtype]
    hi = {"f32": 126, "bf16": 126, "f16": 15}[dtype]
    j = g.integers(lo, hi, size=(nblocks, 1))
    d = g.integers(0, 5, size=(nblocks, block))
    mant = g.integers(0, 1 << 10, size=(nblocks, block)) / 1024.0 + 1.0
    v = np.ldexp(mant, j - d) * np.where(g.integers(0, 2, size=(nblocks, block)) == 1, -1.0, 1.0)
    special = g.integers(0, 40, size=(nblocks, block))
    v = np.where(special == 0, 0.0, v)
    v = np.where(special == 1, -0.0, v)
    v = np.clip(v, -6e4, 6e4) if dtype == "f16" else v
    bits = bits_of(v.astype(np.float32), dtype)
    return bits


# ------------------------------------------------------------------ dequantize
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_dequantize_all_bytes_times_all_scales(dtype):
    packed = np.tile(np.arange(256, dtype=np.uint8), (256, 1)).view(np.int8)      # [256, 256] -> K = 512
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 16, axis=1)
    want = oracle.dequantize_mxfp4(packed, scales, dtype)
    nan = np.isnan(oracle.mxfp4.dequantize_mxfp4_values(packed, scales))
    got = mxq.dequantize_mxfp4(torch.from_numpy(packed).to(dev()), torch.from_numpy(scales).to(dev()), DTYPES[dtype])
    torch.cuda.synchronize()
    assert_bits_equal(from_gpu_bits(got), want, f"dequant {dtype}", nan, nan_of(dtype))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_dequantize_misaligned_general_path(dtype):
    g = np.random.default_rng(1)
    rows, K = 19, 96
    packed = g.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    scales = g.integers(100, 150, size=(rows, K // 32), dtype=np.uint8)
    want = oracle.dequantize_mxfp4(packed.view(np.int8), scales, dtype)
    # packed and out both start one element past an aligned address
    pbuf = torch.empty(rows * K // 2 + 1, dtype=torch.uint8, device=dev())[1:]
    pbuf.copy_(torch.from_numpy(packed.reshape(-1)).to(dev()))
    ts = torch.from_numpy(scales).to(dev())
    out = torch.empty(rows * K + 1, dtype=DTYPES[dtype], device=dev())[1:]
    st = mxq.lib().dequantize_mxfp4(pbuf.data_ptr(), ts.data_ptr(), rows, K, out.data_ptr(),
                                    {"f32": 0, "bf16": 1, "f16": 2}[dtype], None)
    assert st == 0
    torch.cuda.synchronize()
    assert_bits_equal(from_gpu_bits(out).reshape(rows, K), want, "dequant misaligned")
    got = mxq.dequantize_mxfp4(torch.from_numpy(packed).to(dev()).view(torch.int8), ts, DTYPES[dtype])
    assert_bits_equal(from_gpu_bits(got), want, "dequant aligned")


def test_dequantize_weight_tensor_sampled():
    """2^30-parameter expert weight [64, 4096, 4096] -> bf16; sampled rows."""
    d = synth.bulk_stream(seed=0, rows=8, cols=64, with_weights=True)
    p, s = d["w_packed"], d["w_scales"]
    got = mxq.dequantize_mxfp4(torch.from_numpy(p).to(dev()), torch.from_numpy(s).to(dev()), torch.bfloat16)
    g = np.random.default_rng(2)
    e = g.integers(0, 64, 16)
    n = g.integers(0, 4096, 16)
    gb = from_gpu_bits(got[torch.from_numpy(e).to(dev()), torch.from_numpy(n).to(dev())])
    want = oracle.dequantize_mxfp4(p[e, n], s[e, n], "bf16")
    assert_bits_equal(gb, want, "weight dequant")


# ------------------------------------------------------------- quantize_mxfp4
with open(HAND) as _f:
    _HAND = json.load(_f)


def _num(v):
    return float.fromhex(v) if isinstance(v, str) else float(v)


def _block(nonzero, n):
    b = np.zeros(n)
    for k, v in nonzero.items():
        b[int(k)] = _num(v)
    return b


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_hand_worked_blocks(dtype):
    blocks = np.stack([_block(c["nonzero"], 32) for c in _HAND["floor_rule"]])
    x = to_gpu_bits(bits_of(blocks.astype(np.float32), dtype), dtype)
    p, s = mxq.quantize_mxfp4(x)
    deq = mxq.dequantize_mxfp4(p, s, torch.float32)
    pb, sb, db = from_gpu_bits(p), from_gpu_bits(s), from_gpu_bits(deq).view(np.float32)
    for i, c in enumerate(_HAND["floor_rule"]):
        assert sb[i].tolist() == [c["scale_byte"]], c["name"]
        assert pb[i].view(np.uint8).tobytes().hex() == c["packed_hex"], c["name"]
        want = _block(c["dequant_nonzero"], 32)
        assert np.array_equal(db[i].astype(np.float64), want), c["name"]
        assert not np.any(np.signbit(db[i][want == 0])), c["name"]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_quantize_random_blocks_bit_exact(dtype):
    g = np.random.default_rng({"f32": 10, "bf16": 11, "f16": 12}[dtype])
    bits = random_blocks(g, 1 << 16, 32, dtype).reshape(1024, 2048)
    x = oracle.from_dtype_bits(bits, dtype)
    wp, ws = oracle.quantize_mxfp4(x)
    p, s = mxq.quantize_mxfp4(to_gpu_bits(bits, dtype))
    assert_bits_equal(from_gpu_bits(s), ws, f"scales {dtype}")
    assert_bits_equal(from_gpu_bits(p).view(np.uint8), wp.view(np.uint8), f"packed {dtype}")
    back = mxq.dequantize_mxfp4(p, s, DTYPES[dtype])
    assert_bits_equal(from_gpu_bits(back), oracle.dequantize_mxfp4(wp, ws, dtype), f"round trip {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_quantize_ragged_and_misaligned(dtype):
    g = np.random.default_rng(13)
    for rows, K in [(1, 32), (37, 96), (5, 1056)]:
        bits = random_blocks(g, rows * K // 32, 32, dtype).reshape(rows, K)
        x = oracle.from_dtype_bits(bits, dtype)
        wp, ws = oracle.quantize_mxfp4(x)
        t = to_gpu_bits(bits, dtype)
        p, s = mxq.quantize_mxfp4(t)
        assert_bits_equal(from_gpu_bits(p).view(np.uint8), wp.view(np.uint8), f"packed {rows}x{K}")
        assert_bits_equal(from_gpu_bits(s), ws, f"scales {rows}x{K}")
        # misaligned source (general kernel): shift the data by one element
        big = torch.empty(rows * K + 1, dtype=DTYPES[dtype], device=dev())
        big[1:] = t.reshape(-1)
        mis = big[1:].view(rows, K)
        assert mis.data_ptr() % 16 != 0
        pk = torch.empty(rows, K // 2, dtype=torch.int8, device=dev())
        sc = torch.empty(rows, K // 32, dtype=torch.uint8, device=dev())
        st = mxq.lib().quantize_mxfp4(mis.data_ptr(), {"f32": 0, "bf16": 1, "f16": 2}[dtype], rows, K,
                                      pk.data_ptr(), sc.data_ptr(), None)
        assert st == 0
        torch.cuda.synchronize()
        assert_bits_equal(from_gpu_bits(pk).view(np.uint8), wp.view(np.uint8), "packed misaligned")
        assert_bits_equal(from_gpu_bits(sc), ws, "scales misaligned")


def test_roundtrip_workload_f32():
    """fp32 [256, 1024] with per-block 2^k scaling, 1% zero blocks, 1% +-1000 outliers."""
    d = synth.roundtrip_f32(seed=0)
    x = d["x"]
    wp, ws = oracle.quantize_mxfp4(x.astype(np.float64))
    p, s = mxq.quantize_mxfp4(torch.from_numpy(x).to(dev()))
    assert_bits_equal(from_gpu_bits(p).view(np.uint8), wp.view(np.uint8), "packed")
    assert_bits_equal(from_gpu_bits(s), ws, "scales")
    back = mxq.dequantize_mxfp4(p, s, torch.float32)
    assert_bits_equal(from_gpu_bits(back), oracle.dequantize_mxfp4(wp, ws, "f32"), "dequant fp32")


def test_bulk_stream_mxfp4_sampled_rows():
    """bf16 [65536, 7168] quantize + dequantize; 256 sampled rows vs the oracle."""
    d = synth.bulk_stream(seed=0, with_weights=False)
    xb = d["x"]
    t = to_gpu_bits(xb, "bf16")
    p, s = mxq.quantize_mxfp4(t)
    back = mxq.dequantize_mxfp4(p, s, torch.bfloat16)
    rows = np.sort(np.random.default_rng(3).choice(xb.shape[0], 256, replace=False))
    ri = torch.from_numpy(rows).to(dev())
    x = oracle.from_dtype_bits(xb[rows], "bf16")
    wp, ws = oracle.quantize_mxfp4(x)
    assert_bits_equal(from_gpu_bits(p[ri]).view(np.uint8), wp.view(np.uint8), "packed")
    assert_bits_equal(from_gpu_bits(s[ri]), ws, "scales")
    assert_bits_equal(from_gpu_bits(back[ri]), oracle.dequantize_mxfp4(wp, ws, "bf16"), "dequant")
    for fmt, block in [("mxfp4", 32), ("nvfp4", 16), ("fp8", 128)]:
        out = mxq.quantize_cache(t, fmt, block)
        assert_bits_equal(from_gpu_bits(out[ri]), oracle.quantize_cache(x, fmt, block, "bf16"), f"cache {fmt}")


@pytest.mark.parametrize("dtype,rows,cols", [("bf16", 8192, 4096), ("f32", 4096, 2048), ("f16", 2048, 8192)])
def test_mid_size_inputs_sampled_rows(dtype, rows, cols):
    """33-67 MB inputs (between the tiny and the large-input access modes):
    quantize_mxfp4 + dequantize and quantize_cache in three formats, 64 sampled
    rows against the oracle."""
    g = np.random.default_rng(rows + cols)
    x32 = (g.standard_normal((rows, cols)) * np.exp2(g.integers(-4, 5, (rows, 1)))).astype(np.float32)
    bits = bits_of(x32, dtype)
    t = to_gpu_bits(bits, dtype)
    sel = np.sort(g.choice(rows, 64, replace=False))
    ri = torch.from_numpy(sel).to(dev())
    x = oracle.from_dtype_bits(bits[sel], dtype)
    p, s = mxq.quantize_mxfp4(t)
    wp, ws = oracle.quantize_mxfp4(x)
    assert_bits_equal(from_gpu_bits(p[ri]).view(np.uint8), wp.view(np.uint8), f"packed {dtype}")
    assert_bits_equal(from_gpu_bits(s[ri]), ws, f"scales {dtype}")
    back = mxq.dequantize_mxfp4(p, s, t.dtype)
    assert_bits_equal(from_gpu_bits(back[ri]), oracle.dequantize_mxfp4(wp, ws, dtype), f"dequant {dtype}")
    for fmt, block in [("fp8", 128), ("mxfp4", 32), ("nvfp4", 16)]:
        out = mxq.quantize_cache(t, fmt, block)
        assert_bits_equal(from_gpu_bits(out[ri]), oracle.quantize_cache(x, fmt, block, dtype), f"cache {fmt} {dtype}")


# ------------------------------------------------------------- quantize_cache
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "nvfp4"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("block,channels", [(8, 64), (16, 64), (32, 96), (64, 128), (128, 256), (256, 512),
                                            (512, 1024), (24, 96), (32, 100), (16, 7), (128, 200)])
def test_quantize_cache_bit_exact(fmt, dtype, block, channels):
    g = np.random.default_rng(zlib.crc32(f"{fmt}/{dtype}/{block}/{channels}".encode()))
    rows = 67
    nb = -(-channels // block)
    bits = random_blocks(g, rows * nb, block, dtype)[:, :].reshape(rows, nb * block)[:, :channels].copy()
    x = oracle.from_dtype_bits(bits, dtype)
    want = oracle.quantize_cache(x, fmt, block, dtype)
    t = to_gpu_bits(bits, dtype)
    got = mxq.quantize_cache(t, fmt, block)
    assert got.dtype == t.dtype and got.shape == t.shape and got.data_ptr() != t.data_ptr()
    assert_bits_equal(from_gpu_bits(got), want, f"{fmt} {dtype} B={block} C={channels}")
    assert_bits_equal(from_gpu_bits(t), bits, "input unchanged")


@pytest.mark.parametrize("case", _HAND["ceil_rule"], ids=lambda c: c["name"])
def test_quantize_cache_hand_worked(case):
    x = _block(case["nonzero"], case["block"])[None, :]
    for dtype in ("f32", "bf16"):
        t = to_gpu_bits(bits_of(x.astype(np.float32), dtype), dtype)
        out = oracle.from_dtype_bits(from_gpu_bits(mxq.quantize_cache(t, case["format"], case["block"])), dtype)
        assert np.array_equal(out[0], _block(case["out_nonzero"], case["block"])), (case["name"], dtype)


def test_kv_cache_workload_three_formats_and_ste():
    """bf16 [4, 8192, 512], normal(0, 0.5) with 0.1% +-U(20, 200) outliers."""
    d = synth.kv_cache(seed=0)
    xb, gb = d["x"], d["grad"]
    x = oracle.from_dtype_bits(xb, "bf16")
    t = to_gpu_bits(xb, "bf16").requires_grad_(True)
    for fmt, block in [("fp8", 128), ("mxfp4", 32), ("nvfp4", 16)]:
        y = mxq.quantize_cache(t, fmt, block)
        assert_bits_equal(from_gpu_bits(y), oracle.quantize_cache(x, fmt, block, "bf16"), f"kv {fmt}")
        gt = to_gpu_bits(gb, "bf16")
        t.grad = None
        y.backward(gt)
        assert_bits_equal(from_gpu_bits(t.grad), gb, f"straight-through grad {fmt}")
    # the ABI copy form of the backward
    gt = to_gpu_bits(gb, "bf16")
    gi = mxq.quantize_cache_bwd(gt)
    assert gi.data_ptr() != gt.data_ptr()
    assert_bits_equal(from_gpu_bits(gi), gb, "quantize_cache_bwd copy")
    assert mxq.lib().quantize_cache_bwd(gt.data_ptr(), gt.data_ptr(), 1, gt.numel(), None) == 0


def test_empty_inputs():
    z = torch.empty(0, 64, dtype=torch.bfloat16, device=dev())
    p, s = mxq.quantize_mxfp4(z)
    assert p.shape == (0, 32) and s.shape == (0, 2)
    assert mxq.dequantize_mxfp4(p, s, torch.float32).shape == (0, 64)
    assert mxq.quantize_cache(z, "nvfp4", 16).shape == (0, 64)
    for fmt, bs, cw in (("fp8", 32, 64), ("mxfp4", 32, 32), ("nvfp4", 16, 32)):
        c, sc = mxq.quantize_cache_packed(z, fmt, bs)
        assert c.shape == (0, cw) and sc.shape == (0, 64 // bs)
        assert mxq.dequantize_cache_packed(c, sc, fmt, bs, torch.bfloat16).shape == (0, 64)
    # two-level NVFP4 of an empty tensor: no launch (the library leaves g alone; the binding starts it at 0)
    for q in (mxq.quantize_nvfp4, mxq.quantize_nvfp4_mse):
        p2, s2, g2 = q(z)
        assert p2.shape == (0, 32) and s2.shape == (0, 4) and g2.item() == 0.0
        assert mxq.dequantize_nvfp4(p2, s2, g2, torch.bfloat16).shape == (0, 64)
