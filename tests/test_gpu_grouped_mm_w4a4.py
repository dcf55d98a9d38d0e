"""GPU parity of the W4A4 grouped GEMM forward (activations quantized to MXFP4
by quantize_mxfp4, both operands on the block-scaled fp4 MFMA) against the
float64 oracle: bit-exact on one-hot weights, relative Frobenius error
<= 5e-3 per expert segment and globally on random data, ragged segments,
empty experts, rows no expert owns, clamped offsets, NaN scales, and the
full-size workloads."""

import numpy as np
import pytest
import torch

import oracle
import synth
import nvfp4_quantization_grouped_amd as mxq
from tests.gpu_util import dev, from_gpu_bits, rel_frobenius, to_gpu_bits
from tests.test_gpu_grouped_mm import TOL, bf16_values, check_segments, gpu_weights, random_case

pytestmark = pytest.mark.gpu


def host_quantized(xb):
    """Activations (bf16 bits) quantized by the oracle, as GPU tensors."""
    xq, xs = oracle.quantize_mxfp4(oracle.from_dtype_bits(xb, "bf16"))
    return torch.from_numpy(np.ascontiguousarray(xq)).to(dev()), torch.from_numpy(np.ascontiguousarray(xs)).to(dev())


def test_w4a4_one_hot_weights_bit_exact():
    """W_e[n, (n+e) mod K] = 2^(s_e-127): every output is one quantized
    activation times a power of two, exact in bf16; both through the full
    path (GPU quantizer) and through the quantized entry fed by the oracle's
    quantizer."""
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
        oracle.grouped_mm_fwd_w4a4(oracle.from_dtype_bits(xb, "bf16"), packed, scales, offs), "bf16")
    y = mxq.mxfp4_grouped_mm_fwd_w4a4(to_gpu_bits(xb, "bf16"), pt, st, ot)
    assert np.array_equal(from_gpu_bits(y), want)
    xq, xs = host_quantized(xb)
    y2 = mxq.mxfp4_grouped_mm_fwd_w4a4_quantized(xq, xs, pt, st, ot)
    assert np.array_equal(from_gpu_bits(y2), want)


@pytest.mark.parametrize("E,T,N,K,counts", [
    (1, 64, 256, 512, [64]),                          # single expert = dense GEMM
    (4, 777, 264, 1024, [100, 0, 377, 250]),          # empty expert, N % 256 != 0, 50 uncovered rows
    (8, 1500, 512, 2048, [1, 255, 256, 257, 0, 300, 200, 231]),
    (3, 600, 1032, 512, [300, 0, 300]),
    (2, 2048, 512, 7168, [1000, 1048]),               # the routed layer's K
])
def test_w4a4_random_segments(E, T, N, K, counts):
    offs = np.cumsum(counts).astype(np.int32)
    packed, scales, xb = random_case(21 + E, E, T, N, K, offs)
    pt, st = gpu_weights(packed, scales)
    ot = torch.from_numpy(offs).to(dev())
    want = oracle.grouped_mm_fwd_w4a4(oracle.from_dtype_bits(xb, "bf16"), packed, scales, offs)
    y = mxq.mxfp4_grouped_mm_fwd_w4a4(to_gpu_bits(xb, "bf16"), pt, st, ot)
    errs = check_segments(bf16_values(y), want, offs, what=f"w4a4 E={E} T={T} N={N} K={K}")
    print("w4a4 rel Frobenius", {k: f"{v:.2e}" for k, v in errs.items()})
    # the quantized entry on the oracle's quantization gives the same bits
    xq, xs = host_quantized(xb)
    assert torch.equal(mxq.mxfp4_grouped_mm_fwd_w4a4_quantized(xq, xs, pt, st, ot), y)


@pytest.mark.parametrize("raw", [[300, 200, 900], [-5, 150, 40, 10000]])
def test_w4a4_out_of_range_offsets_are_clamped(raw):
    E, T, N, K = len(raw), 500, 256, 512
    clamped = np.minimum(np.maximum.accumulate(np.maximum(np.array(raw), 0)), T).astype(np.int32)
    packed, scales, xb = random_case(31 + E, E, T, N, K, clamped)
    pt, st = gpu_weights(packed, scales)
    ot = torch.tensor(raw, dtype=torch.int32, device=dev())
    y = mxq.mxfp4_grouped_mm_fwd_w4a4(to_gpu_bits(xb, "bf16"), pt, st, ot)
    want = oracle.grouped_mm_fwd_w4a4(oracle.from_dtype_bits(xb, "bf16"), packed, scales, clamped)
    check_segments(bf16_values(y), want, clamped, what="w4a4 clamped offs")


def test_w4a4_nan_scale_propagates():
    """A weight scale byte 0xFF (E8M0 NaN) makes every output that block
    feeds NaN, as the oracle's exact dequantization does; the rest match."""
    E, T, N, K = 2, 300, 256, 1024
    offs = np.array([120, 300], np.int32)
    packed, scales, xb = random_case(41, E, T, N, K, offs)
    scales = scales.copy()
    scales[1, 17, 5] = 0xFF
    pt, st = gpu_weights(packed, scales)
    ot = torch.from_numpy(offs).to(dev())
    y = bf16_values(mxq.mxfp4_grouped_mm_fwd_w4a4(to_gpu_bits(xb, "bf16"), pt, st, ot))
    want = oracle.grouped_mm_fwd_w4a4(oracle.from_dtype_bits(xb, "bf16"), packed, scales, offs)
    nan = np.isnan(want)
    assert nan.any() and np.array_equal(np.isnan(y), nan)
    assert nan[120:, 17].all() and nan.sum() == 180
    y[nan] = 0.0
    want[nan] = 0.0
    check_segments(y, want, offs, what="w4a4 with a NaN scale")


def test_w4a4_e8_workload():
    """E=8, x bf16 [4096, 4096], weights [8, 2048, 4096] packed, multinomial counts."""
    d = synth.grouped_mm_e8(seed=0)
    pt, st = gpu_weights(d["packed"], d["scales"])
    ot = torch.from_numpy(d["offs"]).to(dev())
    y = mxq.mxfp4_grouped_mm_fwd_w4a4(to_gpu_bits(d["x"], "bf16"), pt, st, ot)
    want = oracle.grouped_mm_fwd_w4a4(oracle.from_dtype_bits(d["x"], "bf16"), d["packed"], d["scales"], d["offs"])
    errs = check_segments(bf16_values(y), want, d["offs"], what="w4a4 E=8")
    print("w4a4 E=8 rel Frobenius", {k: f"{v:.2e}" for k, v in errs.items()})


@pytest.mark.timeout(900)
def test_w4a4_moe_layer_workload_sampled_rows():
    """32 local experts, hidden 7168, intermediate 2048, 131072 routed rows:
    gate/up and down W4A4 forwards on 8 sampled rows of every non-empty
    expert."""
    d = synth.moe_layer(seed=0)
    offs = d["offs"]
    ot = torch.from_numpy(offs).to(dev())
    g = np.random.default_rng(9)
    rows, start = [], 0
    for end in offs.tolist():
        if end > start:
            rows.append(np.sort(g.choice(np.arange(start, end), size=min(8, end - start), replace=False)))
        start = end
    rows = np.concatenate(rows)
    ri = torch.from_numpy(rows).to(dev())
    x_routed = to_gpu_bits(d["tokens_x"], "bf16")[torch.from_numpy(d["row_token"]).to(dev())]
    layers = [
        ("gate/up", d["gu_packed"], d["gu_scales"], x_routed, d["tokens_x"][d["row_token"][rows]]),
        ("down", d["dn_packed"], d["dn_scales"], to_gpu_bits(d["h"], "bf16"), d["h"][rows]),
    ]
    for name, pk, sc, a_gpu, a_rows_bits in layers:
        pt, st = gpu_weights(pk, sc)
        y = mxq.mxfp4_grouped_mm_fwd_w4a4(a_gpu, pt, st, ot)
        want, _ = oracle.grouped_mm_rows(rows, pk, sc, offs,
                                         x_rows=oracle.w4a4_activations(oracle.from_dtype_bits(a_rows_bits, "bf16")))
        err = rel_frobenius(bf16_values(y[ri]), want)
        print(f"w4a4 {name}: sampled rel Frobenius {err:.2e}")
        assert err <= TOL, f"w4a4 {name}: {err:.3e}"
        del y
