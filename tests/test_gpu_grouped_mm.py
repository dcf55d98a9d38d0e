"""GPU parity of the MXFP4 grouped GEMM (forward and grad_x) against the
float64 oracle: bit-exact on one-hot weights, relative Frobenius error
<= 5e-3 per expert segment and globally on random data, ragged segments,
empty experts, rows no expert owns, tile tails, and the full-size workloads."""

import numpy as np
import pytest
import torch

import oracle
import synth
import nvfp4_quantization_grouped_amd as mxq
from tests.gpu_util import dev, from_gpu_bits, rel_frobenius, to_gpu_bits

pytestmark = pytest.mark.gpu

TOL = 5e-3   # relative Frobenius error against the fp64 oracle


def gpu_weights(packed, scales):
    return torch.from_numpy(packed).to(dev()), torch.from_numpy(scales).to(dev())


def bf16_values(t):
    return oracle.from_dtype_bits(from_gpu_bits(t), "bf16")


def check_segments(got, want, offs, rows=None, what=""):
    """Global and per-expert relative Frobenius error (only over `rows` if given)."""
    T = got.shape[0]
    sel = np.arange(T) if rows is None else rows
    errs = {"global": rel_frobenius(got[sel], want[sel])}
    start = 0
    for e, end in enumerate(np.asarray(offs).tolist()):
        r = sel[(sel >= start) & (sel < end)]
        if len(r):
            errs[e] = rel_frobenius(got[r], want[r])
        start = end
    worst = max(errs.values())
    assert worst <= TOL, f"{what}: rel Frobenius {worst:.3e} > {TOL} ({errs})"
    # rows no expert owns are exactly zero
    tail = sel[sel >= (offs[-1] if len(offs) else 0)]
    assert np.all(got[tail] == 0), f"{what}: uncovered rows are not zero"
    return errs


def random_case(seed, E, T, N, K, offs):
    d = synth.streams(seed, 3)
    packed, scales = synth.packed_weights(d[0], d[1], E, N, K)
    x = synth.normal_bf16(d[2], (T, K))
    return packed, scales, x


def test_one_hot_weights_bit_exact():
    """W_e[n, (n+e) mod K] = 2^(s_e-127): every output is one input times a
    power of two, so forward and backward must match the oracle bit for bit."""
    E, T, N, K = 3, 300, 384, 512
    codes = np.zeros((E, N, K), np.uint8)
    for e in range(E):
        codes[e, np.arange(N), (np.arange(N) + e) % K] = 2
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8).view(np.int8)
    sbyte = np.array([120, 127, 131], np.uint8)
    scales = np.repeat(np.repeat(sbyte[:, None, None], N, axis=1), K // 32, axis=2)
    offs = np.array([70, 70, 290], np.int32)           # expert 1 empty, 10 uncovered rows
    g = np.random.default_rng(0)
    xb = synth.f32_to_bf16_bits(g.standard_normal((T, K)).astype(np.float32))
    pt, st = gpu_weights(packed, scales)
    ot = torch.from_numpy(offs).to(dev())
    y = mxq.mxfp4_grouped_mm_fwd(to_gpu_bits(xb, "bf16"), pt, st, ot)
    want = oracle.grouped_mm_fwd(oracle.from_dtype_bits(xb, "bf16"), packed, scales, offs)
    assert np.array_equal(from_gpu_bits(y), oracle.to_dtype_bits(want, "bf16"))
    gb = synth.f32_to_bf16_bits(g.standard_normal((T, N)).astype(np.float32))
    gx = mxq.mxfp4_grouped_mm_bwd_x(to_gpu_bits(gb, "bf16"), pt, st, ot)
    want_b = oracle.grouped_mm_bwd_x(oracle.from_dtype_bits(gb, "bf16"), packed, scales, offs)
    # each grad_x entry is a sum of at most ceil(N/K) products of distinct columns: exact here (N < K)
    assert np.array_equal(from_gpu_bits(gx), oracle.to_dtype_bits(want_b, "bf16"))


@pytest.mark.parametrize("E,T,N,K,counts", [
    (1, 64, 256, 256, [64]),                          # single expert = dense GEMM
    (4, 777, 264, 96, [100, 0, 377, 250]),            # N, K tails; empty expert; 50 uncovered rows
    (8, 1500, 512, 1024, [300, 1, 255, 257, 0, 0, 400, 287]),
    (3, 600, 1024, 2048, [0, 600, 0]),
    (5, 2048, 2048, 512, [512, 512, 512, 256, 256]),
    # many tiles and a column tail (1032 = 4 x 256 + 8); K = 256 (per-step scale transfers)
    (4, 44000, 1032, 256, [11000, 0, 20999, 12001]),
    # the same with K = 1024 (8-step scale chunks) and a 150-row uncovered tail
    (4, 40000, 1032, 1024, [10000, 0, 19850, 10000]),
])
def test_random_segments(E, T, N, K, counts):
    offs = np.cumsum(counts).astype(np.int32)
    packed, scales, xb = random_case(E * 1000 + T, E, T, N, K, offs)
    pt, st = gpu_weights(packed, scales)
    ot = torch.from_numpy(offs).to(dev())
    x = oracle.from_dtype_bits(xb, "bf16")
    y = mxq.mxfp4_grouped_mm_fwd(to_gpu_bits(xb, "bf16"), pt, st, ot)
    want = oracle.grouped_mm_fwd(x, packed, scales, offs)
    check_segments(bf16_values(y), want, offs, what="fwd")
    gb = synth.normal_bf16(np.random.default_rng(T), (T, N), 0.1)
    gx = mxq.mxfp4_grouped_mm_bwd_x(to_gpu_bits(gb, "bf16"), pt, st, ot)
    want_b = oracle.grouped_mm_bwd_x(oracle.from_dtype_bits(gb, "bf16"), packed, scales, offs)
    check_segments(bf16_values(gx), want_b, offs, what="bwd_x")


@pytest.mark.parametrize("E,T,N,K,counts", [
    # two tiles of 64 reduction steps; 5 uncovered rows
    (2, 130, 256, 4096, [65, 60]),
    # 18 tiles x 32 steps, an empty expert
    (3, 1000, 512, 2048, [300, 0, 650]),
    # 18 steps (K % 512 != 0), a column tail (264 = 256 + 8)
    (2, 700, 264, 1152, [350, 300]),
])
def test_few_long_tiles(E, T, N, K, counts):
    """Few output tiles with long reductions (fewer tiles than workgroup
    slots): oracle parity, zeros past the last expert, and the same bits on a
    second call."""
    offs = np.cumsum(counts).astype(np.int32)
    packed, scales, xb = random_case(E * 7 + K, E, T, N, K, offs)
    pt, st = gpu_weights(packed, scales)
    ot = torch.from_numpy(offs).to(dev())
    xg = to_gpu_bits(xb, "bf16")
    y = mxq.mxfp4_grouped_mm_fwd(xg, pt, st, ot)
    want = oracle.grouped_mm_fwd(oracle.from_dtype_bits(xb, "bf16"), packed, scales, offs)
    check_segments(bf16_values(y), want, offs, what="few long tiles fwd")
    y2 = mxq.mxfp4_grouped_mm_fwd(xg, pt, st, ot)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("raw", [[300, 200, 900], [-5, 150, 40, 10_000]])
def test_out_of_range_offsets_are_clamped(raw):
    """Offsets that decrease, go negative or pass the row count are clamped
    into [previous clamped offset, tokens] by the kernels: no access leaves
    the buffers and the result is the oracle's on the clamped offsets."""
    E, T, N, K = len(raw), 500, 256, 512
    clamped = np.minimum(np.maximum.accumulate(np.maximum(np.array(raw), 0)), T).astype(np.int32)
    packed, scales, xb = random_case(11 + E, E, T, N, K, clamped)
    pt, st = gpu_weights(packed, scales)
    ot = torch.tensor(raw, dtype=torch.int32, device=dev())
    y = mxq.mxfp4_grouped_mm_fwd(to_gpu_bits(xb, "bf16"), pt, st, ot)
    want = oracle.grouped_mm_fwd(oracle.from_dtype_bits(xb, "bf16"), packed, scales, clamped)
    check_segments(bf16_values(y), want, clamped, what="fwd clamped offs")
    gb = synth.normal_bf16(np.random.default_rng(E), (T, N), 0.1)
    gx = mxq.mxfp4_grouped_mm_bwd_x(to_gpu_bits(gb, "bf16"), pt, st, ot)
    want_b = oracle.grouped_mm_bwd_x(oracle.from_dtype_bits(gb, "bf16"), packed, scales, clamped)
    check_segments(bf16_values(gx), want_b, clamped, what="bwd_x clamped offs")


def test_very_long_reduction():
    """K = 2^22: past the 32-bit buffer ranges of the DMA forward, so the
    forward takes the general kernel; grad_x (reduction over n = 16) covers
    16384 column tiles.  Parity with the oracle both ways."""
    E, T, N, K = 1, 3, 16, 1 << 22
    offs = np.array([T], np.int32)
    packed, scales, xb = random_case(99, E, T, N, K, offs)
    pt, st = gpu_weights(packed, scales)
    ot = torch.from_numpy(offs).to(dev())
    y = mxq.mxfp4_grouped_mm_fwd(to_gpu_bits(xb, "bf16"), pt, st, ot)
    want = oracle.grouped_mm_fwd(oracle.from_dtype_bits(xb, "bf16"), packed, scales, offs)
    check_segments(bf16_values(y), want, offs, what="K = 2^22 fwd")
    gb = synth.normal_bf16(np.random.default_rng(3), (T, N), 0.1)
    gx = mxq.mxfp4_grouped_mm_bwd_x(to_gpu_bits(gb, "bf16"), pt, st, ot)
    want_b = oracle.grouped_mm_bwd_x(oracle.from_dtype_bits(gb, "bf16"), packed, scales, offs)
    check_segments(bf16_values(gx), want_b, offs, what="K = 2^22 bwd_x")


def test_expert_segment_past_4gib():
    """One expert owning 2^24 + 16 rows: its activation segment (K = 128) and
    grad_out segment (N = 128) span 2^32 + 4096 bytes, past any 32-bit
    buffer range, and each row tile must still read its own 128 or 256 rows
    (a range taken over the whole segment would wrap to 4 KB and read zeros
    from row 16 on).  The rows repeat a seeded 4096-row block, so the oracle
    takes the sampled rows from the block: the first tiles, the middle and
    the last rows, both ways."""
    T = (1 << 24) + 16
    rows = np.concatenate([np.arange(0, 512), (1 << 23) + np.arange(0, 256), np.arange(T - 300, T)])
    offs = np.array([T], np.int32)
    ot = torch.from_numpy(offs).to(dev())
    d = synth.streams(41, 6)

    def tiled(block):
        t = to_gpu_bits(block, "bf16")
        return t.repeat(T // block.shape[0] + 1, 1)[:T].contiguous()

    # forward: x [T, 128] -> y [T, 8]
    K, N = 128, 8
    packed, scales = synth.packed_weights(d[0], d[1], 1, N, K)
    xb = synth.normal_bf16(d[2], (4096, K))
    pt, st = gpu_weights(packed, scales)
    x = tiled(xb)
    y = from_gpu_bits(mxq.mxfp4_grouped_mm_fwd(x, pt, st, ot)[torch.from_numpy(rows).to(dev())])
    del x
    want = oracle.grouped_mm_fwd(oracle.from_dtype_bits(xb[rows % 4096], "bf16"), packed, scales,
                                 np.array([len(rows)], np.int32))
    check_segments(oracle.from_dtype_bits(y, "bf16"), want, [len(rows)], what="2^24 + 16 rows fwd")

    # grad_x: grad_out [T, 128] -> grad_x [T, 32]
    N, K = 128, 32
    packed, scales = synth.packed_weights(d[3], d[4], 1, N, K)
    gb = synth.normal_bf16(d[5], (4096, N), 0.1)
    pt, st = gpu_weights(packed, scales)
    g = tiled(gb)
    gx = from_gpu_bits(mxq.mxfp4_grouped_mm_bwd_x(g, pt, st, ot)[torch.from_numpy(rows).to(dev())])
    del g
    want_b = oracle.grouped_mm_bwd_x(oracle.from_dtype_bits(gb[rows % 4096], "bf16"), packed, scales,
                                     np.array([len(rows)], np.int32))
    check_segments(oracle.from_dtype_bits(gx, "bf16"), want_b, [len(rows)], what="2^24 + 16 rows bwd_x")


def test_autograd_function():
    E, T, N, K = 4, 400, 256, 512
    offs = np.array([100, 200, 300, 400], np.int32)
    packed, scales, xb = random_case(7, E, T, N, K, offs)
    pt, st = gpu_weights(packed, scales)
    ot = torch.from_numpy(offs).to(dev())
    xt = to_gpu_bits(xb, "bf16").requires_grad_(True)
    y = mxq.MXFP4GroupedMM.apply(xt, pt, st, ot)
    gb = synth.normal_bf16(np.random.default_rng(8), (T, N), 0.1)
    y.backward(to_gpu_bits(gb, "bf16"))
    want = oracle.grouped_mm_bwd_x(oracle.from_dtype_bits(gb, "bf16"), packed, scales, offs)
    check_segments(bf16_values(xt.grad), want, offs, what="autograd grad_x")
    direct = mxq.mxfp4_grouped_mm_bwd_x(to_gpu_bits(gb, "bf16"), pt, st, ot)
    assert torch.equal(direct, xt.grad)


def test_grouped_mm_e8_workload():
    """E=8, x bf16 [4096, 4096], weights [8, 2048, 4096] packed, multinomial counts."""
    d = synth.grouped_mm_e8(seed=0)
    pt, st = gpu_weights(d["packed"], d["scales"])
    ot = torch.from_numpy(d["offs"]).to(dev())
    y = mxq.mxfp4_grouped_mm_fwd(to_gpu_bits(d["x"], "bf16"), pt, st, ot)
    want = oracle.grouped_mm_fwd(oracle.from_dtype_bits(d["x"], "bf16"), d["packed"], d["scales"], d["offs"])
    errs = check_segments(bf16_values(y), want, d["offs"], what="E=8 fwd")
    print("E=8 fwd rel Frobenius", {k: f"{v:.2e}" for k, v in errs.items()})


def test_one_round_height_order():
    """A forward grid of at most two workgroups per CU (328 slots of 128 x
    256 for 20 experts) takes its tiles in height order, the first one per CU
    XCD-major: segment tails of 1, 2, 3 and 4 row blocks, whole tiles, empty
    experts, a one-row expert and 77 uncovered rows all match the oracle, and
    a second call gives the same bits."""
    counts = [128, 31, 64, 65, 96, 97, 0, 127, 1, 256, 300, 0, 33, 200, 160, 129, 190, 250, 100, 300]
    E, N, K = len(counts), 2048, 512
    T = sum(counts) + 77
    offs = np.cumsum(counts).astype(np.int32)
    assert N // 256 * ((T + 127) // 128 + E) <= 512
    packed, scales, xb = random_case(4242, E, T, N, K, offs)
    pt, st = gpu_weights(packed, scales)
    ot = torch.from_numpy(offs).to(dev())
    xg = to_gpu_bits(xb, "bf16")
    y = mxq.mxfp4_grouped_mm_fwd(xg, pt, st, ot)
    want = oracle.grouped_mm_fwd(oracle.from_dtype_bits(xb, "bf16"), packed, scales, offs)
    check_segments(bf16_values(y), want, offs, what="one-round height order fwd")
    y2 = mxq.mxfp4_grouped_mm_fwd(xg, pt, st, ot)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.timeout(900)
def test_moe_layer_workload_sampled_rows():
    """32 local experts, hidden 7168, intermediate 2048, 131072 routed rows
    (Zipf-skewed, 4 idle experts): gate/up and down, forward and grad_x,
    checked on 8 sampled rows of every non-empty expert."""
    d = synth.moe_layer(seed=0)
    offs = d["offs"]
    ot = torch.from_numpy(offs).to(dev())
    assert (d["counts"] == 0).sum() >= 4
    g = np.random.default_rng(5)
    rows, start = [], 0
    for end in offs.tolist():
        if end > start:
            rows.append(np.sort(g.choice(np.arange(start, end), size=min(8, end - start), replace=False)))
        start = end
    rows = np.concatenate(rows)
    ri = torch.from_numpy(rows).to(dev())

    x_routed = to_gpu_bits(d["tokens_x"], "bf16")[torch.from_numpy(d["row_token"]).to(dev())]
    layers = [
        ("gate/up", d["gu_packed"], d["gu_scales"], x_routed, d["tokens_x"][d["row_token"][rows]], d["gu_grad"]),
        ("down", d["dn_packed"], d["dn_scales"], to_gpu_bits(d["h"], "bf16"), d["h"][rows], d["dn_grad"]),
    ]
    for name, pk, sc, a_gpu, a_rows_bits, grad_bits in layers:
        pt, st = gpu_weights(pk, sc)
        y = mxq.mxfp4_grouped_mm_fwd(a_gpu, pt, st, ot)
        gx = mxq.mxfp4_grouped_mm_bwd_x(to_gpu_bits(grad_bits, "bf16"), pt, st, ot)
        want_y, want_gx = oracle.grouped_mm_rows(
            rows, pk, sc, offs, x_rows=oracle.from_dtype_bits(a_rows_bits, "bf16"),
            g_rows=oracle.from_dtype_bits(grad_bits[rows], "bf16"))
        for what, got, want in [("fwd", bf16_values(y[ri]), want_y), ("bwd_x", bf16_values(gx[ri]), want_gx)]:
            err = rel_frobenius(got, want)
            print(f"{name} {what}: sampled rel Frobenius {err:.2e}")
            assert err <= TOL, f"{name} {what}: {err:.3e}"
        del y, gx


@pytest.mark.parametrize("E,clamp", [(96, False), (256, False), (96, True), (256, True)])
def test_many_experts(E, clamp):
    """More than 64 experts: the tile lookup scans the offsets 64 experts at a
    time.  Forward, grad_x and the W4A4 forward against the oracle, with empty
    experts, rows no expert owns and (clamp) offsets that go negative,
    decrease and pass the row count, which the kernels clamp into
    [previous clamped offset, tokens]."""
    T, N, K = 6000, 256, 512
    g = np.random.default_rng(E + clamp)
    counts = g.integers(0, 2 * T // E, E)
    counts[g.choice(E, E // 8, replace=False)] = 0
    raw = np.cumsum(counts)
    raw = (raw * (T - 37) // max(int(raw[-1]), 1)).astype(np.int64)      # 37+ uncovered rows
    if clamp:
        idx = g.choice(E, 12, replace=False)
        raw[idx[:4]] = -7
        raw[idx[4:8]] = raw[idx[4:8]] // 2
        raw[idx[8:]] = T + 1000
    raw = raw.astype(np.int32)
    offs = np.minimum(np.maximum.accumulate(np.maximum(raw, 0)), T).astype(np.int32)
    packed, scales, xb = random_case(E * 13 + clamp, E, T, N, K, offs)
    pt, st = gpu_weights(packed, scales)
    ot = torch.from_numpy(raw).to(dev())
    x = oracle.from_dtype_bits(xb, "bf16")
    y = mxq.mxfp4_grouped_mm_fwd(to_gpu_bits(xb, "bf16"), pt, st, ot)
    check_segments(bf16_values(y), oracle.grouped_mm_fwd(x, packed, scales, offs), offs, what=f"E={E} fwd")
    gb = synth.normal_bf16(np.random.default_rng(E), (T, N), 0.1)
    gx = mxq.mxfp4_grouped_mm_bwd_x(to_gpu_bits(gb, "bf16"), pt, st, ot)
    want_b = oracle.grouped_mm_bwd_x(oracle.from_dtype_bits(gb, "bf16"), packed, scales, offs)
    check_segments(bf16_values(gx), want_b, offs, what=f"E={E} bwd_x")
    y4 = mxq.mxfp4_grouped_mm_fwd_w4a4(to_gpu_bits(xb, "bf16"), pt, st, ot)
    check_segments(bf16_values(y4), oracle.grouped_mm_fwd_w4a4(x, packed, scales, offs), offs, what=f"E={E} w4a4")


@pytest.mark.gpu
def test_validate_offs():
    """The offs debug check: valid offsets (empty experts included) hold;
    a decrease, a negative first offset and an end past the tokens are
    reported at the first expert that breaks the precondition."""
    def check(raw, tokens):
        return mxq.validate_offs(torch.tensor(raw, dtype=torch.int32, device=dev()), tokens)
    assert check([0, 10, 10, 40], 40) == -1
    assert check([0, 0, 0], 0) == -1
    assert check([5, 9, 40], 64) == -1
    assert check([5, 4, 40], 64) == 1
    assert check([-1, 4, 40], 64) == 0
    assert check([5, 9, 65], 64) == 2
    assert check([5, 70, 60], 64) == 1
    assert check(list(range(0, 4000, 2)), 3998) == -1          # many experts
    assert check(list(range(0, 4000, 2)), 3996) == 1999


def test_degenerate_shapes_write_zeros():
    """Every grouped-GEMM entry point, through the C-ABI, on the shapes with
    nothing to reduce or no owning expert: zero experts, an empty reduction
    (k = 0 for the forwards, n = 0 for grad_x) and offsets that cover no row
    write an all-zero output; zero tokens launch nothing and succeed."""
    L = mxq.lib()
    st = torch.cuda.current_stream().cuda_stream
    T, N, K, E = 300, 288, 512, 3          # N is grad_x's output width: a multiple of 32
    g = np.random.default_rng(12)
    packed, scales = gpu_weights(*synth.packed_weights(*synth.streams(12, 2), E, N, K))
    packed_t, scales_t = gpu_weights(*synth.packed_weights(*synth.streams(13, 2), E, K, N))   # W_e [K, N] for grad_x
    x = to_gpu_bits(synth.normal_bf16(g, (T, K)), "bf16")
    go = to_gpu_bits(synth.normal_bf16(g, (T, K)), "bf16")
    xq = torch.from_numpy(g.integers(0, 256, (T, K // 2), dtype=np.uint8)).to(dev())
    x8 = torch.from_numpy(g.integers(0, 0x70, (T, K), dtype=np.uint8)).to(dev())
    xs = torch.from_numpy(g.integers(120, 130, (T, K // 32), dtype=np.uint8)).to(dev())
    none = torch.zeros(E, dtype=torch.int32, device=dev())
    some = torch.tensor([100, 200, 300], dtype=torch.int32, device=dev())

    def fresh(cols):
        return torch.full((T, cols), 7.0, dtype=torch.bfloat16, device=dev())

    def run(name, out, *args):
        assert getattr(L, name)(*args, st) == 0, name
        torch.cuda.synchronize()
        assert torch.all(out.float() == 0), f"{name}: output not all zero"

    for e, offs in ((0, some), (E, none)):
        y = fresh(N)
        run("mxfp4_grouped_mm_fwd", y, x.data_ptr(), T, K, packed.data_ptr(), scales.data_ptr(), e, N,
            offs.data_ptr(), y.data_ptr())
        y = fresh(N)
        run("mxfp4_grouped_mm_fwd_w4a4", y, xq.data_ptr(), xs.data_ptr(), T, K, packed.data_ptr(), scales.data_ptr(),
            e, N, offs.data_ptr(), y.data_ptr())
        y = fresh(N)
        run("mxfp4_grouped_mm_fwd_w4a8", y, x8.data_ptr(), xs.data_ptr(), T, K, packed.data_ptr(), scales.data_ptr(),
            e, N, offs.data_ptr(), y.data_ptr())
        gx = fresh(N)
        run("mxfp4_grouped_mm_bwd_x", gx, go.data_ptr(), T, K, packed_t.data_ptr(), scales_t.data_ptr(), e, N,
            offs.data_ptr(), gx.data_ptr())
    # an empty reduction
    y = fresh(N)
    run("mxfp4_grouped_mm_fwd", y, x.data_ptr(), T, 0, packed.data_ptr(), scales.data_ptr(), E, N, some.data_ptr(),
        y.data_ptr())
    for name, a in (("mxfp4_grouped_mm_fwd_w4a4", xq), ("mxfp4_grouped_mm_fwd_w4a8", x8)):
        y = fresh(N)
        run(name, y, a.data_ptr(), xs.data_ptr(), T, 0, packed.data_ptr(), scales.data_ptr(), E, N, some.data_ptr(),
            y.data_ptr())
    gx = fresh(N)
    run("mxfp4_grouped_mm_bwd_x", gx, go.data_ptr(), T, 0, packed_t.data_ptr(), scales_t.data_ptr(), E, N,
        some.data_ptr(), gx.data_ptr())
    # zero tokens: nothing launched, the output untouched
    y = fresh(N)
    assert L.mxfp4_grouped_mm_fwd(x.data_ptr(), 0, K, packed.data_ptr(), scales.data_ptr(), E, N, some.data_ptr(),
                                  y.data_ptr(), st) == 0
    assert L.mxfp4_grouped_mm_bwd_x(go.data_ptr(), 0, K, packed_t.data_ptr(), scales_t.data_ptr(), E, N,
                                    some.data_ptr(), y.data_ptr(), st) == 0
    torch.cuda.synchronize()
    assert torch.all(y.float() == 7.0)
