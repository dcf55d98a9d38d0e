"""Helpers for the GPU parity tests: move seeded NumPy inputs (bit patterns)
to the device and results back, and compare against the oracle."""

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def to_gpu_bits(bits, dtype):
    """uint16/uint32 bit patterns (or float32 array) -> CUDA tensor of `dtype`."""
    a = np.ascontiguousarray(bits)
    if dtype == "f32":
        t = torch.from_numpy(a.view(np.float32))
    else:
        t = torch.from_numpy(a.view(np.int16)).view(DTYPES[dtype])
    return t.to(dev())


def from_gpu_bits(t):
    """CUDA tensor -> NumPy raw bit patterns."""
    c = t.detach().cpu().contiguous()
    if c.dtype == torch.float32:
        return c.view(torch.int32).numpy().view(np.uint32)
    if c.dtype in (torch.bfloat16, torch.float16):
        return c.view(torch.int16).numpy().view(np.uint16)
    if c.dtype == torch.int8:
        return c.numpy()
    if c.dtype == torch.uint8:
        return c.numpy()
    if c.dtype == getattr(torch, "float8_e8m0fnu", None):
        return c.view(torch.uint8).numpy()
    raise TypeError(c.dtype)


def bits_of(values_f32, dtype):
    """float32 array -> bit patterns of `dtype` using PyTorch's nearest-even cast
    (used only to build inputs)."""
    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32)).to(DTYPES[dtype])
    if dtype == "f32":
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.view(torch.int16).numpy().view(np.uint16)


def assert_bits_equal(got, want, what, nan_mask=None, is_nan=None):
    """Bit-exact comparison.  Where ``nan_mask`` is set the expected value is a
    NaN: there ``is_nan(got)`` must hold (any payload) instead of equal bits."""
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = got != want
    if nan_mask is not None:
        bad &= ~nan_mask
        nan_bad = nan_mask & ~is_nan(got)
        assert not nan_bad.any(), f"{what}: {int(nan_bad.sum())} expected NaNs are not NaN"
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(int(v) for v in i), hex(int(got[tuple(i)])), hex(int(want[tuple(i)]))) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} differ; first {detail}")


def rel_frobenius(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    return np.linalg.norm(got - want) / (den if den > 0 else 1.0)
