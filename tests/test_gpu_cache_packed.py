"""GPU parity of packed KV-cache storage (quantize_cache_packed,
dequantize_cache_packed) against the CPU oracle, bit for bit: codes, scale
bytes and dequantized values on seeded blocks of every binade (zeros, signed
zeros, subnormals) for every format, dtype and fast-path block size plus
general-path block sizes, misaligned buffers, every code byte under every
scale byte the format can store, and the bf16 [4, 8192, 512] KV cache in full.
The dequantized tensor must also equal the GPU fake-quant (quantize_cache)."""

import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
import nvfp4_quantization_grouped_amd as mxq
from tests.gpu_util import DTYPES, assert_bits_equal, dev, from_gpu_bits, to_gpu_bits
from tests.test_gpu_codec import nan_of, random_blocks

pytestmark = pytest.mark.gpu

_DT = {"f32": 0, "bf16": 1, "f16": 2}
_FMT = {"fp8": 0, "mxfp4": 1, "nvfp4": 2}


def check(bits, dtype, fmt, block, what):
    x = oracle.from_dtype_bits(bits, dtype)
    wc, ws = oracle.quantize_cache_packed(x, fmt, block)
    t = to_gpu_bits(bits, dtype)
    c, s = mxq.quantize_cache_packed(t, fmt, block)
    assert_bits_equal(from_gpu_bits(c), wc, f"{what} codes")
    assert_bits_equal(from_gpu_bits(s), ws, f"{what} scales")
    for od in ("f32", "bf16", "f16") if dtype == "f32" else (dtype,):
        back = mxq.dequantize_cache_packed(c, s, fmt, block, DTYPES[od])
        assert_bits_equal(from_gpu_bits(back), oracle.dequantize_cache_packed(wc, ws, fmt, block, od),
                          f"{what} dequant {od}")
    fq = mxq.quantize_cache_forward(t, fmt, block)
    assert_bits_equal(from_gpu_bits(mxq.dequantize_cache_packed(c, s, fmt, block, t.dtype)), from_gpu_bits(fq),
                      f"{what} packed round trip vs quantize_cache")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "nvfp4"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("block", [8, 16, 32, 64, 128, 256, 512, 6, 24, 48])
def test_bit_exact(fmt, dtype, block):
    g = np.random.default_rng(zlib.crc32(f"packed/{fmt}/{dtype}/{block}".encode()))
    rows, nb = 37, max(1, 2048 // block)
    bits = random_blocks(g, rows * nb, block, dtype).reshape(rows, nb * block)
    check(bits, dtype, fmt, block, f"{fmt} {dtype} B={block}")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "nvfp4"])
def test_misaligned_buffers_take_the_general_path(fmt):
    dtype, rows, C, block = "bf16", 19, 256, 32
    g = np.random.default_rng(5)
    bits = random_blocks(g, rows * C // block, block, dtype).reshape(rows, C)
    x = oracle.from_dtype_bits(bits, dtype)
    wc, ws = oracle.quantize_cache_packed(x, fmt, block)
    nc = rows * C // (1 if fmt == "fp8" else 2)
    big = to_gpu_bits(np.concatenate([np.zeros(1, bits.dtype), bits.reshape(-1)]), dtype)
    codes = torch.zeros(nc + 1, dtype=torch.uint8, device=dev())
    scales = torch.zeros(rows * C // block + 1, dtype=torch.uint8, device=dev())
    L = mxq.lib()
    st = torch.cuda.current_stream().cuda_stream
    assert L.quantize_cache_packed(big.data_ptr() + 2, _DT[dtype], rows, C, _FMT[fmt], block, codes.data_ptr() + 1,
                                   scales.data_ptr() + 1, st) == 0
    assert_bits_equal(from_gpu_bits(codes[1:]).reshape(wc.shape), wc, "general codes")
    assert_bits_equal(from_gpu_bits(scales[1:]).reshape(ws.shape), ws, "general scales")
    out = torch.zeros(rows * C + 1, dtype=torch.bfloat16, device=dev())
    assert L.dequantize_cache_packed(codes.data_ptr() + 1, scales.data_ptr() + 1, rows, C, _FMT[fmt], block,
                                     out.data_ptr() + 2, _DT[dtype], st) == 0
    assert_bits_equal(from_gpu_bits(out[1:]).reshape(rows, C), oracle.dequantize_cache_packed(wc, ws, fmt, block, dtype),
                      "general dequant")


def _scale_bytes(fmt):
    if fmt == "nvfp4":
        return np.array([b for b in range(0x7F)], np.uint8)      # every finite non-negative E4M3 scale
    if fmt == "mxfp4":
        return np.arange(255, dtype=np.uint8)                    # every finite E8M0 scale
    return np.arange(1, 248, dtype=np.uint8)                     # fp8: 2^-126 .. 2^120, what the quantizer stores


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "nvfp4"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("block", [32, 10])
def test_dequantize_every_code_byte_under_every_scale_byte(fmt, dtype, block):
    sb = _scale_bytes(fmt)
    if fmt == "fp8":
        codes = np.tile(np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8), (len(sb), 1))
        codes = codes[:, : (codes.shape[1] // block) * block]
        C = codes.shape[1]
    else:
        codes = np.tile(np.arange(256, dtype=np.uint8), (len(sb), 1))[:, : (256 // (block // 2)) * (block // 2)]
        C = codes.shape[1] * 2
    scales = np.repeat(sb[:, None], C // block, axis=1)
    want = oracle.dequantize_cache_packed(codes, scales, fmt, block, dtype)
    got = mxq.dequantize_cache_packed(torch.from_numpy(codes).to(dev()), torch.from_numpy(scales).to(dev()), fmt,
                                      block, DTYPES[dtype])
    nan = np.isnan(oracle.from_dtype_bits(want, dtype)) if dtype != "f32" else np.isnan(want.view(np.float32))
    assert_bits_equal(from_gpu_bits(got), want, f"{fmt} {dtype} B={block}", nan, nan_of(dtype))


def test_kv_cache_workload_three_formats():
    """bf16 [4, 8192, 512], normal(0, 0.5) with 0.1% +-U(20, 200) outliers, in full."""
    xb = synth.kv_cache(seed=0)["x"]
    x = oracle.from_dtype_bits(xb, "bf16")
    t = to_gpu_bits(xb, "bf16")
    for fmt, block in [("fp8", 128), ("mxfp4", 32), ("nvfp4", 16)]:
        wc, ws = oracle.quantize_cache_packed(x, fmt, block)
        c, s = mxq.quantize_cache_packed(t, fmt, block)
        assert c.shape == wc.shape and s.shape == ws.shape
        assert_bits_equal(from_gpu_bits(c), wc, f"kv {fmt} codes")
        assert_bits_equal(from_gpu_bits(s), ws, f"kv {fmt} scales")
        back = mxq.dequantize_cache_packed(c, s, fmt, block, torch.bfloat16)
        assert_bits_equal(from_gpu_bits(back), oracle.quantize_cache(x, fmt, block, "bf16"), f"kv {fmt} dequant")


def test_empty_and_bad_shapes():
    z = torch.empty(0, 64, dtype=torch.bfloat16, device=dev())
    c, s = mxq.quantize_cache_packed(z, "mxfp4", 32)
    assert c.shape == (0, 32) and s.shape == (0, 2)
    assert mxq.dequantize_cache_packed(c, s, "mxfp4", 32, torch.float32).shape == (0, 64)
    with pytest.raises(ValueError):
        mxq.quantize_cache_packed(torch.zeros(2, 40, dtype=torch.bfloat16, device=dev()), "fp8", 32)
    with pytest.raises(ValueError):
        mxq.quantize_cache_packed(torch.zeros(2, 42, dtype=torch.bfloat16, device=dev()), "nvfp4", 7)


def test_typed_scale_views():
    """nvfp4 scale bytes viewed as float8_e4m3fn, and mxfp4 / fp8 scale bytes
    viewed as float8_e8m0fnu, decode as the raw bytes do; a view that names
    the other encoding is refused."""
    e4m3, e8m0 = getattr(torch, "float8_e4m3fn", None), getattr(torch, "float8_e8m0fnu", None)
    g = np.random.default_rng(11)
    bits = random_blocks(g, 24 * 4, 32, "bf16").reshape(24, 128)
    x = oracle.from_dtype_bits(bits, "bf16")
    t = to_gpu_bits(bits, "bf16")
    for fmt, block, view in [("nvfp4", 16, e4m3), ("mxfp4", 32, e8m0), ("fp8", 32, e8m0)]:
        if view is None:
            continue
        wc, ws = oracle.quantize_cache_packed(x, fmt, block)
        c, s = mxq.quantize_cache_packed(t, fmt, block)
        back = mxq.dequantize_cache_packed(c, s.view(view), fmt, block, torch.bfloat16)
        assert_bits_equal(from_gpu_bits(back), oracle.dequantize_cache_packed(wc, ws, fmt, block, "bf16"),
                          f"{fmt} typed scales")
        other = e8m0 if view is e4m3 else e4m3
        if other is not None:
            with pytest.raises(TypeError):
                mxq.dequantize_cache_packed(c, s.view(other), fmt, block, torch.bfloat16)
