"""PyTorch-facing binding of libmxq.

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI (``include/mxq.h``).  Tensors must be CUDA (ROCm) tensors on one device;
the call is enqueued on the current stream, outputs are allocated with
PyTorch's caching allocator.  There is no CPU path.

Names and signatures follow the pages:
* "nemo_automodel.components.quantization.mxfp4": ``quantize_mxfp4``,
  ``dequantize_mxfp4``, ``MXFP4GroupedMM``, ``MXFP4_BLOCK_SIZE``.
* "nemo_automodel.components.models.deepseek_v41.quantization":
  ``quantize_cache`` and ``_CacheQuantization``.
* "NVIDIA Model Optimizer: from mtq.quantize to a 4.95-bit DeepSeek-R1":
  ``quantize_nvfp4`` / ``dequantize_nvfp4`` (two-level NVFP4) and the W4A4
  and W4A8 forwards ``mxfp4_grouped_mm_fwd_w4a4`` / ``mxfp4_grouped_mm_fwd_w4a8``.
"""

import ctypes

import torch

from . import _lib

MXFP4_BLOCK_SIZE = 32

_DT = {torch.float32: _lib.MXQ_F32, torch.bfloat16: _lib.MXQ_BF16, torch.float16: _lib.MXQ_F16}
_FMT = {"fp8": _lib.MXQ_FMT_FP8, "mxfp4": _lib.MXQ_FMT_MXFP4, "nvfp4": _lib.MXQ_FMT_NVFP4}
_E8M0 = getattr(torch, "float8_e8m0fnu", None)


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t):
    return t.data_ptr() if t.numel() else None


def _need_cuda(*ts):
    dev = None
    for t in ts:
        if not t.is_cuda:
            raise ValueError("libmxq ops take GPU tensors only (there is no CPU implementation)")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return dev


def _as_u8(scales):
    if _E8M0 is not None and scales.dtype == _E8M0:
        return scales.view(torch.uint8)
    if scales.dtype != torch.uint8:
        raise TypeError("scales must be float8_e8m0fnu or uint8 E8M0 bytes")
    return scales


def quantize_mxfp4(weight):
    """[..., K] float tensor (K % 32 == 0) -> (int8 packed [..., K/2],
    float8_e8m0fnu scales [..., K/32])."""
    _need_cuda(weight)
    if weight.dtype not in _DT:
        raise TypeError(f"quantize_mxfp4: unsupported dtype {weight.dtype}")
    K = weight.shape[-1]
    if K % MXFP4_BLOCK_SIZE:
        raise ValueError("quantize_mxfp4: K must be divisible by 32")
    x = weight.contiguous()
    rows = x.numel() // K if K else 0
    packed = torch.empty(*x.shape[:-1], K // 2, dtype=torch.int8, device=x.device)
    scales = torch.empty(*x.shape[:-1], K // 32, dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        st = _lib.lib().quantize_mxfp4(_ptr(x), _DT[x.dtype], rows, K, _ptr(packed), _ptr(scales), _stream(x.device))
    _lib.check(st, "quantize_mxfp4")
    return packed, (scales.view(_E8M0) if _E8M0 is not None else scales)


def dequantize_mxfp4(packed, scales, dtype):
    """int8 packed [..., K/2] + E8M0 scales [..., K/32] -> [..., K] in ``dtype``."""
    _need_cuda(packed, scales)
    if dtype not in _DT:
        raise TypeError(f"dequantize_mxfp4: unsupported dtype {dtype}")
    s = _as_u8(scales).contiguous()
    p = packed.contiguous()
    K = p.shape[-1] * 2
    if tuple(s.shape) != tuple(p.shape[:-1]) + (K // 32,):
        raise ValueError("dequantize_mxfp4: scales must be [..., K/32] for packed [..., K/2]")
    rows = p.numel() * 2 // K if K else 0
    out = torch.empty(*p.shape[:-1], K, dtype=dtype, device=p.device)
    with torch.cuda.device(p.device):
        st = _lib.lib().dequantize_mxfp4(_ptr(p), _ptr(s), rows, K, _ptr(out), _DT[dtype], _stream(p.device))
    _lib.check(st, "dequantize_mxfp4")
    return out


_E4M3 = getattr(torch, "float8_e4m3fn", None)


def _quantize_nvfp4(x, name):
    _need_cuda(x)
    if x.dtype not in _DT:
        raise TypeError(f"{name}: unsupported dtype {x.dtype}")
    K = x.shape[-1] if x.dim() else 0
    if K % 16:
        raise ValueError(f"{name}: K must be divisible by 16")
    x = x.contiguous()
    rows = x.numel() // K if K else 0
    packed = torch.empty(*x.shape[:-1], K // 2, dtype=torch.uint8, device=x.device)
    scales = torch.empty(*x.shape[:-1], K // 16, dtype=torch.uint8, device=x.device)
    g = torch.zeros((), dtype=torch.float32, device=x.device)
    with torch.cuda.device(x.device):
        st = getattr(_lib.lib(), name)(_ptr(x), _DT[x.dtype], rows, K, _ptr(packed), _ptr(scales), g.data_ptr(),
                                       _stream(x.device))
    _lib.check(st, name)
    return packed, (scales.view(_E4M3) if _E4M3 is not None else scales), g


def quantize_nvfp4(x):
    """Two-level NVFP4 ("NVIDIA Model Optimizer: from mtq.quantize to a
    4.95-bit DeepSeek-R1", section "NVFP4 in the code: two scales and a
    nibble"): [..., K] float tensor (K % 16 == 0) -> (uint8 packed [..., K/2],
    float8_e4m3fn block scales [..., K/16], float32 global scale g [] on the
    device), the four-tensor checkpoint layout's weight, weight_scale and
    weight_scale_2."""
    return _quantize_nvfp4(x, "quantize_nvfp4")


def quantize_nvfp4_mse(x):
    """Two-level NVFP4 with each block scale searched over the 126 positive
    finite E4M3 values for the least squared error (same page, section "Where
    the scales come from"); outputs as ``quantize_nvfp4``."""
    return _quantize_nvfp4(x, "quantize_nvfp4_mse")


def dequantize_nvfp4(packed, block_scales, global_scale, dtype):
    """uint8 packed [..., K/2] + E4M3 block scales [..., K/16] + float32 global
    scale (a device scalar) -> [..., K] in ``dtype``."""
    _need_cuda(packed, block_scales, global_scale)
    if dtype not in _DT:
        raise TypeError(f"dequantize_nvfp4: unsupported dtype {dtype}")
    s = block_scales.view(torch.uint8) if block_scales.dtype != torch.uint8 else block_scales
    s = s.contiguous()
    p = packed.contiguous()
    g = global_scale.to(torch.float32).contiguous()
    if g.numel() != 1:
        raise ValueError("dequantize_nvfp4: global_scale must hold one value")
    K = p.shape[-1] * 2
    if tuple(s.shape) != tuple(p.shape[:-1]) + (K // 16,):
        raise ValueError("dequantize_nvfp4: block scales must be [..., K/16] for packed [..., K/2]")
    rows = p.numel() * 2 // K if K else 0
    out = torch.empty(*p.shape[:-1], K, dtype=dtype, device=p.device)
    with torch.cuda.device(p.device):
        st = _lib.lib().dequantize_nvfp4(_ptr(p), _ptr(s), g.data_ptr(), rows, K, _ptr(out), _DT[dtype],
                                         _stream(p.device))
    _lib.check(st, "dequantize_nvfp4")
    return out


def quantize_cache_forward(values, format, block_size):
    """Fake-quantized copy of ``values`` [..., channels] (no autograd)."""
    _need_cuda(values)
    if values.dtype not in _DT:
        raise TypeError(f"quantize_cache: unsupported dtype {values.dtype}")
    if format not in _FMT:
        raise ValueError("quantize_cache: format must be 'fp8', 'mxfp4' or 'nvfp4'")
    x = values.contiguous()
    C = x.shape[-1] if x.dim() else 1
    rows = x.numel() // C if C else 0
    out = torch.empty_like(x)
    with torch.cuda.device(x.device):
        st = _lib.lib().quantize_cache(_ptr(x), _ptr(out), _DT[x.dtype], rows, C, _FMT[format], int(block_size),
                                       _stream(x.device))
    _lib.check(st, "quantize_cache")
    return out


def quantize_cache_bwd(grad_out, grad_in=None):
    """Straight-through backward through the C ABI: grad_in = grad_out
    (a copy into ``grad_in`` or a new tensor; nothing to do if they alias)."""
    _need_cuda(grad_out)
    g = grad_out.contiguous()
    out = torch.empty_like(g) if grad_in is None else grad_in
    _need_cuda(out)
    if out.dtype != g.dtype or out.numel() != g.numel() or not out.is_contiguous():
        raise ValueError("quantize_cache_bwd: grad_in must be a contiguous tensor like grad_out")
    with torch.cuda.device(g.device):
        st = _lib.lib().quantize_cache_bwd(_ptr(g), _ptr(out), _DT[g.dtype], g.numel(), _stream(g.device))
    _lib.check(st, "quantize_cache_bwd")
    return out


def quantize_cache_packed(values, format, block_size):
    """Packed KV-cache storage of ``values`` [..., channels] (whole groups):
    returns (codes uint8 [..., channels/2] for mxfp4/nvfp4 or [..., channels]
    for fp8, scales uint8 [..., channels/block_size]); the stored form of
    quantize_cache's round trip."""
    _need_cuda(values)
    if values.dtype not in _DT:
        raise TypeError(f"quantize_cache_packed: unsupported dtype {values.dtype}")
    if format not in _FMT:
        raise ValueError("quantize_cache_packed: format must be 'fp8', 'mxfp4' or 'nvfp4'")
    x = values.contiguous()
    if x.dim() == 0:
        raise ValueError("quantize_cache_packed: needs at least one dimension")
    C, B = x.shape[-1], int(block_size)
    if B <= 0 or C % B or (format != "fp8" and B % 2):
        raise ValueError("quantize_cache_packed: channels must be whole groups (an even block for the fp4 formats)")
    rows = x.numel() // C if C else 0
    codes = torch.empty(x.shape[:-1] + (C if format == "fp8" else C // 2,), dtype=torch.uint8, device=x.device)
    scales = torch.empty(x.shape[:-1] + (C // B,), dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        st = _lib.lib().quantize_cache_packed(_ptr(x), _DT[x.dtype], rows, C, _FMT[format], B, _ptr(codes),
                                              _ptr(scales), _stream(x.device))
    _lib.check(st, "quantize_cache_packed")
    return codes, scales


def dequantize_cache_packed(codes, scales, format, block_size, dtype):
    """Dequant-on-read of the packed form into a new ``dtype`` tensor [..., channels]."""
    _need_cuda(codes, scales)
    if dtype not in _DT:
        raise TypeError(f"dequantize_cache_packed: unsupported dtype {dtype}")
    if format not in _FMT:
        raise ValueError("dequantize_cache_packed: format must be 'fp8', 'mxfp4' or 'nvfp4'")
    c = codes.contiguous()
    # a typed view of the scale bytes must name the encoding the format stores:
    # E4M3 bits for nvfp4, E8M0 bytes for mxfp4 and fp8 (raw uint8 is taken as is)
    if _E4M3 is not None and scales.dtype == _E4M3:
        if format != "nvfp4":
            raise TypeError(f"dequantize_cache_packed: float8_e4m3fn scales are nvfp4's; {format} stores E8M0 bytes")
        s = scales.view(torch.uint8)
    elif _E8M0 is not None and scales.dtype == _E8M0:
        if format == "nvfp4":
            raise TypeError("dequantize_cache_packed: nvfp4 stores E4M3 scale bits, not float8_e8m0fnu")
        s = scales.view(torch.uint8)
    elif scales.dtype == torch.uint8:
        s = scales
    else:
        raise TypeError("dequantize_cache_packed: scales must be uint8, float8_e8m0fnu (mxfp4, fp8) "
                        "or float8_e4m3fn (nvfp4)")
    s = s.contiguous()
    if c.dtype != torch.uint8 or c.dim() == 0:
        raise TypeError("dequantize_cache_packed: codes must be a uint8 tensor")
    C = c.shape[-1] * (1 if format == "fp8" else 2)
    B = int(block_size)
    if B <= 0 or C % B or s.shape != c.shape[:-1] + (C // B,):
        raise ValueError("dequantize_cache_packed: scales must be [..., channels / block_size]")
    rows = c.numel() // c.shape[-1] if c.shape[-1] else 0
    out = torch.empty(c.shape[:-1] + (C,), dtype=dtype, device=c.device)
    with torch.cuda.device(c.device):
        st = _lib.lib().dequantize_cache_packed(_ptr(c), _ptr(s), rows, C, _FMT[format], B, _ptr(out), _DT[dtype],
                                                _stream(c.device))
    _lib.check(st, "dequantize_cache_packed")
    return out


class CacheQuantization(torch.autograd.Function):
    """``_CacheQuantization``: quantize/dequantize in forward, pass the
    gradient through unchanged in backward (no gradient for block_size and
    format)."""

    @staticmethod
    def forward(ctx, values, block_size, format):
        return quantize_cache_forward(values, format, block_size)

    @staticmethod
    def backward(ctx, gradient):
        return gradient, None, None


def quantize_cache(values, format, block_size):
    """``quantize_cache(values, format, block_size)``: the cache
    quantize/dequantize round trip with a straight-through gradient."""
    return CacheQuantization.apply(values, block_size, format)


def _gemm_args(a, packed, scales, offs):
    _need_cuda(a, packed, scales, offs)
    if a.dtype != torch.bfloat16:
        raise TypeError("MXFP4GroupedMM: activations must be bfloat16")
    if offs.dtype != torch.int32:
        raise TypeError("MXFP4GroupedMM: offs must be int32")
    s = _as_u8(scales)
    if packed.dim() != 3 or s.dim() != 3 or offs.dim() != 1:
        raise ValueError("MXFP4GroupedMM: packed [E, N, K/2], scales [E, N, K/32], offs [E]")
    E, N, K2 = packed.shape
    if tuple(s.shape) != (E, N, K2 * 2 // 32) or offs.shape[0] != E:
        raise ValueError("MXFP4GroupedMM: inconsistent packed / scales / offs shapes")
    return a.contiguous(), packed.contiguous(), s.contiguous(), offs.contiguous(), E, N, K2 * 2


def validate_offs(offs, tokens):
    """Debug check of the grouped GEMM's offs precondition (non-decreasing,
    within [0, tokens]); synchronizes the current stream.  Returns -1 when it
    holds, else the first expert index that breaks it."""
    _need_cuda(offs)
    if offs.dtype != torch.int32 or offs.dim() != 1:
        raise TypeError("validate_offs: offs must be a 1-D int32 tensor")
    o = offs.contiguous()
    bad = ctypes.c_int64(-1)
    with torch.cuda.device(o.device):
        st = _lib.lib().mxq_validate_offs(_ptr(o), o.shape[0], int(tokens), ctypes.byref(bad), _stream(o.device))
    if st == _lib.MXQ_ERR_OFFS:
        return int(bad.value)
    _lib.check(st, "mxq_validate_offs")
    return -1


def mxfp4_grouped_mm_fwd(x, packed, scales, offs):
    """y [T, N] = x[rows_e] @ W_e^T per expert segment (bf16 in/out)."""
    x, p, s, o, E, N, K = _gemm_args(x, packed, scales, offs)
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError("mxfp4_grouped_mm_fwd: x must be [tokens, K]")
    T = x.shape[0]
    y = torch.empty(T, N, dtype=torch.bfloat16, device=x.device)
    with torch.cuda.device(x.device):
        st = _lib.lib().mxfp4_grouped_mm_fwd(_ptr(x), T, K, _ptr(p), _ptr(s), E, N, _ptr(o), _ptr(y),
                                             _stream(x.device))
    _lib.check(st, "mxfp4_grouped_mm_fwd")
    return y


def mxfp4_grouped_mm_bwd_x(grad_out, packed, scales, offs):
    """grad_x [T, K] = grad_out[rows_e] @ W_e per expert segment (bf16)."""
    g, p, s, o, E, N, K = _gemm_args(grad_out, packed, scales, offs)
    if g.dim() != 2 or g.shape[1] != N:
        raise ValueError("mxfp4_grouped_mm_bwd_x: grad_out must be [tokens, N]")
    T = g.shape[0]
    gx = torch.empty(T, K, dtype=torch.bfloat16, device=g.device)
    with torch.cuda.device(g.device):
        st = _lib.lib().mxfp4_grouped_mm_bwd_x(_ptr(g), T, N, _ptr(p), _ptr(s), E, K, _ptr(o), _ptr(gx),
                                               _stream(g.device))
    _lib.check(st, "mxfp4_grouped_mm_bwd_x")
    return gx


def mxfp4_grouped_mm_fwd_w4a4_quantized(xq, xs, packed, scales, offs):
    """y [T, N] = dq(xq)[rows_e] @ dq(W_e)^T per expert segment, activations
    already in MXFP4 (int8 [T, K/2] and E8M0 [T, K/32] as quantize_mxfp4
    returns them); K % 512 == 0.  bf16 output."""
    _need_cuda(xq, xs, packed, scales, offs)
    xs8, s = _as_u8(xs), _as_u8(scales)
    if offs.dtype != torch.int32:
        raise TypeError("mxfp4_grouped_mm_fwd_w4a4: offs must be int32")
    if packed.dim() != 3 or s.dim() != 3 or offs.dim() != 1 or xq.dim() != 2 or xs8.dim() != 2:
        raise ValueError("mxfp4_grouped_mm_fwd_w4a4: xq [T, K/2], xs [T, K/32], packed [E, N, K/2], "
                         "scales [E, N, K/32], offs [E]")
    E, N, K2 = packed.shape
    T = xq.shape[0]
    if (tuple(s.shape) != (E, N, K2 * 2 // 32) or offs.shape[0] != E or xq.shape[1] != K2
            or tuple(xs8.shape) != (T, K2 * 2 // 32)):
        raise ValueError("mxfp4_grouped_mm_fwd_w4a4: inconsistent shapes")
    xq, xs8, p, s, o = xq.contiguous(), xs8.contiguous(), packed.contiguous(), s.contiguous(), offs.contiguous()
    y = torch.empty(T, N, dtype=torch.bfloat16, device=xq.device)
    with torch.cuda.device(xq.device):
        st = _lib.lib().mxfp4_grouped_mm_fwd_w4a4(_ptr(xq), _ptr(xs8), T, K2 * 2, _ptr(p), _ptr(s), E, N, _ptr(o),
                                                  _ptr(y), _stream(xq.device))
    _lib.check(st, "mxfp4_grouped_mm_fwd_w4a4")
    return y


def mxfp4_grouped_mm_fwd_w4a4(x, packed, scales, offs):
    """W4A4 forward: quantize_mxfp4(x) (bf16 x [T, K], per 32-block E8M0
    scales by the floor rule), then the grouped GEMM of the two MXFP4
    operands on the block-scaled fp4 MFMA.  K % 512 == 0."""
    _need_cuda(x)
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise TypeError("mxfp4_grouped_mm_fwd_w4a4: x must be bfloat16 [tokens, K]")
    xq, xs = quantize_mxfp4(x)
    return mxfp4_grouped_mm_fwd_w4a4_quantized(xq, xs, packed, scales, offs)


def mxfp4_grouped_mm_fwd_w4a8_quantized(xq, xs, packed, scales, offs):
    """y [T, N] = dq(xq)[rows_e] @ dq(W_e)^T per expert segment, activations
    already in fp8 (uint8 E4M3 codes [T, K] and E8M0 scale bytes [T, K/32], as
    ``quantize_cache_packed(x, "fp8", 32)`` returns them); K % 512 == 0.  bf16
    output."""
    _need_cuda(xq, xs, packed, scales, offs)
    xs8, s = _as_u8(xs), _as_u8(scales)
    if xq.dtype != torch.uint8:
        raise TypeError("mxfp4_grouped_mm_fwd_w4a8: xq must be uint8 E4M3 codes")
    if offs.dtype != torch.int32:
        raise TypeError("mxfp4_grouped_mm_fwd_w4a8: offs must be int32")
    if packed.dim() != 3 or s.dim() != 3 or offs.dim() != 1 or xq.dim() != 2 or xs8.dim() != 2:
        raise ValueError("mxfp4_grouped_mm_fwd_w4a8: xq [T, K], xs [T, K/32], packed [E, N, K/2], "
                         "scales [E, N, K/32], offs [E]")
    E, N, K2 = packed.shape
    T, K = xq.shape
    if (K != 2 * K2 or tuple(s.shape) != (E, N, K // 32) or offs.shape[0] != E
            or tuple(xs8.shape) != (T, K // 32)):
        raise ValueError("mxfp4_grouped_mm_fwd_w4a8: inconsistent shapes")
    xq, xs8, p, s, o = xq.contiguous(), xs8.contiguous(), packed.contiguous(), s.contiguous(), offs.contiguous()
    y = torch.empty(T, N, dtype=torch.bfloat16, device=xq.device)
    with torch.cuda.device(xq.device):
        st = _lib.lib().mxfp4_grouped_mm_fwd_w4a8(_ptr(xq), _ptr(xs8), T, K, _ptr(p), _ptr(s), E, N, _ptr(o),
                                                  _ptr(y), _stream(xq.device))
    _lib.check(st, "mxfp4_grouped_mm_fwd_w4a8")
    return y


def mxfp4_grouped_mm_fwd_w4a8(x, packed, scales, offs):
    """W4A8 forward: the activations quantized to fp8 (E4M3 codes, one E8M0
    power-of-two scale per 32 columns: ``quantize_cache_packed(x, "fp8",
    32)``), then the grouped GEMM of fp8 activations and MXFP4 weights on the
    block-scaled MFMA.  bf16 x [T, K], K % 512 == 0."""
    _need_cuda(x)
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise TypeError("mxfp4_grouped_mm_fwd_w4a8: x must be bfloat16 [tokens, K]")
    xq, xs = quantize_cache_packed(x, "fp8", 32)
    return mxfp4_grouped_mm_fwd_w4a8_quantized(xq, xs, packed, scales, offs)


class MXFP4GroupedMM(torch.autograd.Function):
    """Grouped GEMM over mxfp4-packed frozen expert weights.  Saves only the
    packed weights, scales and offsets; the backward dequantizes again inside
    its kernel and returns (grad_x, None, None, None)."""

    @staticmethod
    def forward(ctx, x, packed, scales, offs):
        ctx.save_for_backward(packed, scales, offs)
        return mxfp4_grouped_mm_fwd(x, packed, scales, offs)

    @staticmethod
    def backward(ctx, grad_out):
        packed, scales, offs = ctx.saved_tensors
        return mxfp4_grouped_mm_bwd_x(grad_out.to(torch.bfloat16), packed, scales, offs), None, None, None
