"""GPU parity of the W4A8 grouped GEMM forward (activations quantized to fp8
E4M3 with E8M0 block-32 scales by quantize_cache_packed, weights MXFP4, both
on the block-scaled MFMA) against the float64 oracle: bit-exact on one-hot
weights, relative Frobenius error <= 5e-3 per expert segment and globally on
random data, ragged segments, empty experts, rows no expert owns, clamped
offsets, NaN scales, and the routed-expert workload on sampled rows."""

import numpy as np
import pytest
import torch

import oracle
import synth
import nvfp4_quantization_grouped_amd as mxq
from tests.gpu_util import assert_bits_equal, dev, from_gpu_bits, rel_frobenius, to_gpu_bits
from tests.test_gpu_grouped_mm import TOL, bf16_values, check_segments, gpu_weights, random_case

pytestmark = pytest.mark.gpu


def host_quantized(xb):
    """Activations (bf16 bits) encoded by the oracle, as GPU tensors."""
    c, s = oracle.quantize_cache_packed(oracle.from_dtype_bits(xb, "bf16"), "fp8", 32)
    return torch.from_numpy(np.ascontiguousarray(c)).to(dev()), torch.from_numpy(np.ascontiguousarray(s)).to(dev())


def test_w4a8_one_hot_weights_bit_exact():
    """W_e[n, (n+e) mod K] = 2^(s_e-127): every output is one fp8-quantized
    activation times a power of two, exact in bf16; through the full path
    (GPU encoder) and through the quantized entry fed by the oracle's encoder."""
    E, T, N, K = 3, 300, 384, 512
    codes = np.zeros((E, N, K), np.uint8)
    for e in range(E):
        codes[e, np.arange(N), (np.arange(N) + e) % K] = 2
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8).view(np.int8)
    sbyte = np.array([120, 127, 131], np.uint8)
    scales = np.repeat(np.repeat(sbyte[:, None, None], N, axis=1), K // 32, axis=2)
    offs = np.array([70, 70, 290], np.int32)           # expert 1 empty, 10 uncovered rows
    xb = synth.normal_bf16(np.random.default_rng(0), (T, K))
    pt, st = gpu_weights(packed, scales)
    ot = torch.from_numpy(offs).to(dev())
    want = oracle.to_dtype_bits(
        oracle.grouped_mm_fwd_w4a8(oracle.from_dtype_bits(xb, "bf16"), packed, scales, offs), "bf16")
    xq, xs = host_quantized(xb)
    y2 = mxq.mxfp4_grouped_mm_fwd_w4a8_quantized(xq, xs, pt, st, ot)
    assert_bits_equal(from_gpu_bits(y2), want, "w4a8 one-hot (oracle-encoded activations)")
    y = mxq.mxfp4_grouped_mm_fwd_w4a8(to_gpu_bits(xb, "bf16"), pt, st, ot)
    assert_bits_equal(from_gpu_bits(y), want, "w4a8 one-hot (GPU-encoded activations)")


@pytest.mark.parametrize("E,T,N,K,counts", [
    (1, 64, 256, 512, [64]),                          # single expert = dense GEMM
    (4, 777, 264, 1024, [100, 0, 377, 250]),          # empty expert, N % 256 != 0, 50 uncovered rows
    (8, 1500, 512, 2048, [1, 255, 256, 257, 0, 300, 200, 231]),
    (3, 600, 1032, 512, [300, 0, 300]),
    (2, 2048, 512, 7168, [1000, 1048]),               # the routed layer's K
])
def test_w4a8_random_segments(E, T, N, K, counts):
    offs = np.cumsum(counts).astype(np.int32)
    packed, scales, xb = random_case(E * 1000 + T + 3, E, T, N, K, offs)
    # activations spread over binades, so block scales differ along each row
    x = oracle.from_dtype_bits(xb, "bf16") * np.repeat(2.0 ** np.random.default_rng(T).integers(-8, 9, (T, K // 32)),
                                                       32, axis=1)
    xb = oracle.to_dtype_bits(x, "bf16")
    pt, st = gpu_weights(packed, scales)
    ot = torch.from_numpy(offs).to(dev())
    y = mxq.mxfp4_grouped_mm_fwd_w4a8(to_gpu_bits(xb, "bf16"), pt, st, ot)
    want = oracle.grouped_mm_fwd_w4a8(oracle.from_dtype_bits(xb, "bf16"), packed, scales, offs)
    check_segments(bf16_values(y), want, offs, what="w4a8 fwd")


@pytest.mark.parametrize("raw", [[300, 200, 900], [-5, 150, 40, 10_000]])
def test_w4a8_out_of_range_offsets_are_clamped(raw):
    E, T, N, K = len(raw), 500, 256, 512
    clamped = np.minimum(np.maximum.accumulate(np.maximum(np.array(raw), 0)), T).astype(np.int32)
    packed, scales, xb = random_case(23 + E, E, T, N, K, clamped)
    pt, st = gpu_weights(packed, scales)
    y = mxq.mxfp4_grouped_mm_fwd_w4a8(to_gpu_bits(xb, "bf16"), pt, st,
                                      torch.tensor(raw, dtype=torch.int32, device=dev()))
    want = oracle.grouped_mm_fwd_w4a8(oracle.from_dtype_bits(xb, "bf16"), packed, scales, clamped)
    check_segments(bf16_values(y), want, clamped, what="w4a8 clamped offs")


def test_w4a8_nan_scale_byte():
    """An activation scale byte 0xFF makes the products of its block NaN (and
    only the rows that use it)."""
    E, T, N, K = 1, 64, 256, 512
    offs = np.array([T], np.int32)
    packed, scales, xb = random_case(31, E, T, N, K, offs)
    xq, xs = host_quantized(xb)
    xs[5, 3] = 0xFF
    pt, st = gpu_weights(packed, scales)
    y = bf16_values(mxq.mxfp4_grouped_mm_fwd_w4a8_quantized(xq, xs, pt, st, torch.from_numpy(offs).to(dev())))
    assert np.all(np.isnan(y[5])) and not np.any(np.isnan(np.delete(y, 5, axis=0)))


def test_w4a8_many_experts_and_shapes_rejected():
    E, T, N, K = 96, 3000, 256, 512
    g = np.random.default_rng(96)
    counts = g.integers(0, 2 * T // E, E)
    counts[g.choice(E, 12, replace=False)] = 0
    offs = np.minimum(np.cumsum(counts), T - 20).astype(np.int32)
    packed, scales, xb = random_case(96, E, T, N, K, offs)
    pt, st = gpu_weights(packed, scales)
    y = mxq.mxfp4_grouped_mm_fwd_w4a8(to_gpu_bits(xb, "bf16"), pt, st, torch.from_numpy(offs).to(dev()))
    want = oracle.grouped_mm_fwd_w4a8(oracle.from_dtype_bits(xb, "bf16"), packed, scales, offs)
    check_segments(bf16_values(y), want, offs, what="w4a8 E=96")
    with pytest.raises(mxq.MxqError):       # K % 512 != 0
        p2, s2, x2 = random_case(1, 1, 8, 8, 256, np.array([8], np.int32))
        pt2, st2 = gpu_weights(p2, s2)
        mxq.mxfp4_grouped_mm_fwd_w4a8(to_gpu_bits(x2, "bf16"), pt2, st2, torch.tensor([8], dtype=torch.int32,
                                                                                     device=dev()))


@pytest.mark.timeout(900)
def test_w4a8_moe_layer_workload_sampled_rows():
    """The routed-expert layer's gate/up and down forwards as W4A8, checked on
    8 sampled rows of every non-empty expert."""
    d = synth.moe_layer(seed=0)
    offs = d["offs"]
    ot = torch.from_numpy(offs).to(dev())
    g = np.random.default_rng(6)
    rows, start = [], 0
    for end in offs.tolist():
        if end > start:
            rows.append(np.sort(g.choice(np.arange(start, end), size=min(8, end - start), replace=False)))
        start = end
    rows = np.concatenate(rows)
    ri = torch.from_numpy(rows).to(dev())
    x_routed = to_gpu_bits(d["tokens_x"], "bf16")[torch.from_numpy(d["row_token"]).to(dev())]
    for name, pk, sc, a_gpu, a_rows_bits in [
            ("gate/up", d["gu_packed"], d["gu_scales"], x_routed, d["tokens_x"][d["row_token"][rows]]),
            ("down", d["dn_packed"], d["dn_scales"], to_gpu_bits(d["h"], "bf16"), d["h"][rows])]:
        pt, st = gpu_weights(pk, sc)
        y = mxq.mxfp4_grouped_mm_fwd_w4a8(a_gpu, pt, st, ot)
        q = oracle.w4a8_activations(oracle.from_dtype_bits(a_rows_bits, "bf16"))
        want, _ = oracle.grouped_mm_rows(rows, pk, sc, offs, x_rows=q)
        err = rel_frobenius(bf16_values(y[ri]), want)
        print(f"w4a8 {name}: sampled rel Frobenius {err:.2e}")
        assert err <= TOL, f"w4a8 {name}: {err:.3e}"
        del y
