"""The C-ABI library loads, exports every entry point include/mxq.h declares,
and rejects bad arguments on the host before any HIP call (no GPU needed)."""

import ctypes
import os
import re

import pytest

import nvfp4_quantization_grouped_amd as mxq
from nvfp4_quantization_grouped_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxq.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmxq.so is not built (python -m nvfp4_quantization_grouped_amd.build)")
    return mxq.lib()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name
        assert isinstance(getattr(L, name), ctypes._CFuncPtr)


def test_status_strings(L):
    for s in range(0, -10, -1):
        msg = L.mxq_status_string(s)
        assert msg and msg != b"unknown status"
    assert L.mxq_status_string(12345) == b"unknown status"


# Host-side validation: every call below must fail before touching the GPU.
FAKE = 0x10000            # a non-null, 16-byte aligned address that is never dereferenced


def test_quantize_mxfp4_validation(L):
    assert L.quantize_mxfp4(FAKE, 1, 4, 48, FAKE * 2, FAKE * 3, None) == -2      # k % 32
    assert L.quantize_mxfp4(FAKE, 1, -1, 32, FAKE * 2, FAKE * 3, None) == -2     # rows < 0
    assert L.quantize_mxfp4(FAKE, 7, 4, 32, FAKE * 2, FAKE * 3, None) == -3      # dtype
    assert L.quantize_mxfp4(None, 1, 4, 32, FAKE * 2, FAKE * 3, None) == -1      # null
    assert L.quantize_mxfp4(FAKE, 1, 4, 32, FAKE + 8, FAKE * 3, None) == -7      # packed inside x
    assert L.quantize_mxfp4(FAKE, 1, 0, 32, None, None, None) == 0               # empty: no launch


def test_dequantize_validation(L):
    assert L.dequantize_mxfp4(FAKE, FAKE * 2, 4, 40, FAKE * 3, 1, None) == -2
    assert L.dequantize_mxfp4(FAKE, FAKE * 2, 4, 32, FAKE * 3, 5, None) == -3
    assert L.dequantize_mxfp4(FAKE, None, 4, 32, FAKE * 3, 1, None) == -1
    assert L.dequantize_mxfp4(FAKE, FAKE * 2, 4, 32, FAKE, 1, None) == -7
    assert L.dequantize_mxfp4(None, None, 4, 0, None, 1, None) == 0


def test_quantize_cache_validation(L):
    assert L.quantize_cache(FAKE, FAKE * 4, 1, 2, 64, 3, 32, None) == -4         # format
    assert L.quantize_cache(FAKE, FAKE * 4, 1, 2, 64, 1, 0, None) == -5          # block
    assert L.quantize_cache(FAKE, FAKE * 4, 9, 2, 64, 1, 32, None) == -3         # dtype
    assert L.quantize_cache(FAKE, FAKE + 64, 1, 2, 64, 1, 32, None) == -7        # out overlaps x
    assert L.quantize_cache(FAKE, None, 1, 2, 64, 1, 32, None) == -1
    assert L.quantize_cache(FAKE, FAKE * 4, 1, -2, 64, 1, 32, None) == -2
    assert L.quantize_cache(None, None, 1, 0, 64, 2, 16, None) == 0


def test_quantize_cache_bwd_validation(L):
    assert L.quantize_cache_bwd(FAKE, FAKE, 1, 100, None) == 0                   # aliased: identity
    assert L.quantize_cache_bwd(FAKE, FAKE + 2, 1, 100, None) == -7              # partial overlap
    assert L.quantize_cache_bwd(None, FAKE, 1, 100, None) == -1
    assert L.quantize_cache_bwd(FAKE, FAKE * 8, 4, 100, None) == -3


def test_grouped_mm_validation(L):
    f = L.mxfp4_grouped_mm_fwd
    assert f(FAKE, 16, 48, FAKE * 2, FAKE * 3, 2, 64, FAKE * 4, FAKE * 5, None) == -2    # k % 32
    assert f(FAKE, 16, 64, FAKE * 2, FAKE * 3, 2, 60, FAKE * 4, FAKE * 5, None) == -2    # n % 8
    assert f(FAKE, 16, 64, None, FAKE * 3, 2, 64, FAKE * 4, FAKE * 5, None) == -1
    assert f(FAKE + 2, 16, 64, FAKE * 2, FAKE * 3, 2, 64, FAKE * 4, FAKE * 5, None) == -6  # alignment
    assert f(FAKE, 16, 64, FAKE * 2, FAKE * 3, 2, 64, FAKE * 4, FAKE * 5 + 8, None) == -6  # output alignment
    assert f(FAKE, 16, 64, FAKE * 2, FAKE * 3, 2, 64, FAKE * 4, FAKE + 64, None) == -7   # y overlaps x
    assert f(FAKE, 0, 64, FAKE * 2, FAKE * 3, 2, 64, FAKE * 4, FAKE * 5, None) == 0      # no tokens
    b = L.mxfp4_grouped_mm_bwd_x
    assert b(FAKE, 16, 64, FAKE * 2, FAKE * 3, 2, 40, FAKE * 4, FAKE * 5, None) == -2    # k % 32
    assert b(FAKE, 16, 64, FAKE * 2, FAKE * 3, -1, 64, FAKE * 4, FAKE * 5, None) == -2
    # 32-bit addressing limits of the backward: n <= 2^22 and n * k / 2 < 2^31
    assert b(FAKE, 1, (1 << 22) + 8, FAKE * 2, FAKE * 3, 2, 64, FAKE * 4, FAKE << 12, None) == -2
    assert b(FAKE, 1, 1 << 16, FAKE * 2, FAKE * 3, 2, 1 << 16, FAKE * 4, FAKE * 5, None) == -2


def test_nvfp4_validation(L):
    q = L.quantize_nvfp4
    # (x, dtype, rows, k, packed, block_scales, global_scale, stream)
    assert q(FAKE, 1, 4, 24, FAKE * 2, FAKE * 3, FAKE * 4, None) == -2     # k % 16
    assert q(FAKE, 1, -1, 32, FAKE * 2, FAKE * 3, FAKE * 4, None) == -2
    assert q(FAKE, 7, 4, 32, FAKE * 2, FAKE * 3, FAKE * 4, None) == -3     # dtype
    assert q(FAKE, 1, 4, 32, FAKE * 2, FAKE * 3, None, None) == -1
    assert q(FAKE, 1, 4, 32, FAKE * 2, FAKE * 3, FAKE * 4 + 2, None) == -6   # global scale 4-byte aligned
    assert q(FAKE, 1, 4, 32, FAKE + 8, FAKE * 3, FAKE * 4, None) == -7       # packed inside x
    assert q(FAKE, 1, 4, 32, FAKE * 2, FAKE * 3, FAKE * 2 + 4, None) == -7   # global scale inside packed
    assert q(FAKE, 1, 0, 32, FAKE * 2, FAKE * 3, FAKE * 4, None) == 0        # nothing to do
    d = L.dequantize_nvfp4
    # (packed, block_scales, global_scale, rows, k, out, dtype, stream)
    assert d(FAKE, FAKE * 2, FAKE * 3, 4, 40, FAKE * 4, 1, None) == -2
    assert d(FAKE, FAKE * 2, FAKE * 3, 4, 32, FAKE * 4, 9, None) == -3
    assert d(FAKE, None, FAKE * 3, 4, 32, FAKE * 4, 1, None) == -1
    assert d(FAKE, FAKE * 2, FAKE * 3 + 1, 4, 32, FAKE * 4, 1, None) == -6
    assert d(FAKE, FAKE * 2, FAKE * 3, 4, 32, FAKE - 16, 1, None) == -7      # out over packed
    assert d(FAKE, FAKE * 2, FAKE * 3, 0, 32, FAKE * 4, 1, None) == 0


def test_grouped_mm_w4a4_validation(L):
    f = L.mxfp4_grouped_mm_fwd_w4a4
    # (xq, xs, tokens, k, packed, scales, experts, n, offs, y, stream)
    ok = (FAKE, FAKE * 2, 16, 512, FAKE * 3, FAKE * 4, 2, 64, FAKE * 5, FAKE * 6, None)
    def call(**kw):
        names = ("xq", "xs", "tokens", "k", "packed", "scales", "experts", "n", "offs", "y", "stream")
        args = dict(zip(names, ok))
        args.update(kw)
        return f(*[args[n] for n in names])
    assert call(k=256) == -2                      # whole 512-k scale chunks
    assert call(k=544) == -2
    assert call(n=60) == -2                       # n % 8
    assert call(tokens=-1) == -2
    assert call(k=1 << 22) == -2                  # 32-bit offsets
    assert call(k=1 << 16, n=1 << 16) == -2       # one expert's packed weights reach 2 GiB
    assert call(xq=None) == -1
    assert call(scales=None) == -1
    assert call(xs=FAKE * 2 + 4) == -6            # every operand 16-byte aligned
    assert call(scales=FAKE * 4 + 8) == -6
    assert call(y=FAKE * 6 + 2) == -6
    assert call(y=FAKE + 16) == -7                # y overlaps xq
    assert call(tokens=0) == 0                    # nothing to do
    assert call(n=0) == 0


def test_ops_reject_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        mxq.quantize_mxfp4(torch.zeros(2, 32))
    with pytest.raises(ValueError):
        mxq.quantize_cache(torch.zeros(2, 32, dtype=torch.bfloat16), "fp8", 32)


def test_cache_packed_validation(L):
    q = L.quantize_cache_packed
    # (x, dtype, rows, channels, fmt, block, codes, scales, stream)
    assert q(FAKE, 1, 4, 40, 1, 32, FAKE * 2, FAKE * 3, None) == -2        # partial group
    assert q(FAKE, 1, -1, 64, 1, 32, FAKE * 2, FAKE * 3, None) == -2
    assert q(FAKE, 5, 4, 64, 1, 32, FAKE * 2, FAKE * 3, None) == -3        # dtype
    assert q(FAKE, 1, 4, 64, 3, 32, FAKE * 2, FAKE * 3, None) == -4        # format
    assert q(FAKE, 1, 4, 63, 1, 7, FAKE * 2, FAKE * 3, None) == -5         # odd fp4 group
    assert q(FAKE, 1, 4, 63, 0, 7, None, FAKE * 3, None) == -1             # an odd fp8 group passes the block check
    assert q(FAKE, 1, 4, 64, 1, 0, FAKE * 2, FAKE * 3, None) == -5
    assert q(FAKE, 1, 4, 64, 2, 16, None, FAKE * 3, None) == -1
    assert q(FAKE, 1, 4, 64, 0, 16, FAKE + 64, FAKE * 3, None) == -7       # codes inside x
    assert q(FAKE, 1, 4, 64, 0, 16, FAKE * 2, FAKE * 2 + 255, None) == -7  # scales inside the fp8 codes
    assert q(FAKE, 1, 0, 64, 1, 32, FAKE * 2, FAKE * 3, None) == 0         # nothing to do
    d = L.dequantize_cache_packed
    # (codes, scales, rows, channels, fmt, block, out, dtype, stream)
    assert d(FAKE, FAKE * 2, 4, 40, 1, 32, FAKE * 3, 1, None) == -2
    assert d(FAKE, FAKE * 2, 4, 64, 1, 32, FAKE * 3, 4, None) == -3
    assert d(FAKE, FAKE * 2, 4, 64, -1, 32, FAKE * 3, 1, None) == -4
    assert d(FAKE, FAKE * 2, 4, 66, 2, 11, FAKE * 3, 1, None) == -5
    assert d(FAKE, None, 4, 64, 1, 32, FAKE * 3, 1, None) == -1
    assert d(FAKE, FAKE * 2, 4, 64, 1, 32, FAKE - 100, 1, None) == -7      # out over the codes
    assert d(FAKE, FAKE * 2, 0, 64, 1, 32, FAKE * 3, 1, None) == 0


def test_nvfp4_mse_validation(L):
    q = L.quantize_nvfp4_mse
    # (x, dtype, rows, k, packed, block_scales, global_scale, stream): quantize_nvfp4's checks
    assert q(FAKE, 1, 4, 24, FAKE * 2, FAKE * 3, FAKE * 4, None) == -2
    assert q(FAKE, 3, 4, 32, FAKE * 2, FAKE * 3, FAKE * 4, None) == -3
    assert q(FAKE, 1, 4, 32, None, FAKE * 3, FAKE * 4, None) == -1
    assert q(FAKE, 1, 4, 32, FAKE * 2, FAKE * 3, FAKE * 4 + 1, None) == -6
    assert q(FAKE, 1, 4, 32, FAKE * 2, FAKE * 2 + 8, FAKE * 4, None) == -7   # scales inside packed
    assert q(FAKE, 1, 4, 0, FAKE * 2, FAKE * 3, FAKE * 4, None) == 0



def test_grouped_mm_w4a8_validation(L):
    f = L.mxfp4_grouped_mm_fwd_w4a8
    # (xq, xs, tokens, k, packed, scales, experts, n, offs, y, stream)
    ok = (FAKE, FAKE * 2, 16, 512, FAKE * 3, FAKE * 4, 2, 64, FAKE * 5, FAKE * 6, None)
    names = ("xq", "xs", "tokens", "k", "packed", "scales", "experts", "n", "offs", "y", "stream")

    def call(**kw):
        args = dict(zip(names, ok))
        args.update(kw)
        return f(*[args[n] for n in names])
    assert call(k=256) == -2                      # whole 512-k scale chunks
    assert call(k=544) == -2
    assert call(n=60) == -2                       # n % 8
    assert call(experts=-1) == -2
    assert call(k=1 << 22) == -2                  # 32-bit offsets
    assert call(k=1 << 16, n=1 << 16) == -2       # one expert's packed weights reach 2 GiB
    assert call(xq=None) == -1
    assert call(offs=None) == -1
    assert call(xq=FAKE + 4) == -6                # every operand 16-byte aligned
    assert call(packed=FAKE * 3 + 8) == -6
    assert call(y=FAKE * 6 + 2) == -6
    assert call(y=FAKE + 4096) == -7              # y overlaps xq (16 rows x 512 bytes)
    assert call(y=FAKE * 2 + 16) == -7            # y overlaps xs
    assert call(tokens=0) == 0                    # nothing to do
    assert call(n=0) == 0


def test_validate_offs_validation(L):
    """mxq_validate_offs answers bad arguments and the empty case on the host
    (the check itself copies offs from the device: GPU test)."""
    bad = ctypes.c_int64(7)
    f = L.mxq_validate_offs
    assert f(FAKE, -1, 16, ctypes.byref(bad), None) == -2 and bad.value == -1
    assert f(FAKE, 4, -1, ctypes.byref(bad), None) == -2
    assert f(FAKE, (1 << 26) + 1, 16, ctypes.byref(bad), None) == -2
    assert f(None, 4, 16, ctypes.byref(bad), None) == -1
    bad.value = 7
    assert f(None, 0, 16, ctypes.byref(bad), None) == 0 and bad.value == -1   # no experts: holds, no HIP call
    assert f(None, 0, 16, None, None) == 0                                      # first_bad may be NULL
