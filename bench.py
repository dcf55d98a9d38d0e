"""Throughput of the block-scaled quantization / MXFP4 grouped-GEMM hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

One step runs every part of the path once, each on its own seeded synthetic
workload, all inputs already resident in HBM:

* grouped GEMM, one GPU's share of a routed-expert layer: 32 experts, hidden
  7168, intermediate 2048, 131072 routed rows (16384 tokens x top-8,
  Zipf(1.1)-skewed, 4 idle experts): gate/up and down forward, then down and
  gate/up grad_x (re-dequantizing the weights);
* grouped GEMM forward, 8 experts, x [4096, 4096], W [8, 2048, 4096];
* quantize_cache on a bf16 KV cache [4, 8192, 512]: fp8/128, mxfp4/32,
  nvfp4/16, and the straight-through backward copy; the packed storage form
  of each (codes + scale bytes) and its dequantize-on-read;
* bulk bf16 [65536, 7168]: quantize_mxfp4, dequantize_mxfp4, quantize_cache
  nvfp4/16, fp8/128 and mxfp4/32, two-level NVFP4 quantize and dequantize;
  the NVFP4 MSE block-scale sweep of a bf16 weight [4096, 7168] (reported
  as the rule's operation rate, 6 per element and candidate over all 126
  candidates: the kernel skips the candidates an exact bound rules out, so
  no roofline fraction applies); dequantization of a 2^30-parameter mxfp4 weight
  [64, 4096, 4096] to bf16;
* mxfp4 round trip of an fp32 [256, 1024] tensor (latency-bound).

Legs whose working set fits in the 256 MB Infinity Cache rotate over enough
buffer copies to exceed it.  Each leg is bracketed by HIP events recorded on
the stream its kernels run on; a leg of short calls repeats them over
rotating inputs (32 calls per step for the KV cache) so that the hand-over
from the previous leg is a small share of its time; `value` is the grouped-GEMM throughput of the
routed-expert layer (algorithmic flops 2 * rows * N * K summed over its four
GEMMs, divided by their event time); `hbm` aggregates the codec legs
(algorithmic bytes over event time).  Prints one JSON line.
"""

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
MFMA_FP4_PEAK_TFLOPS = 10100.0   # MI355X dense fp4 (MXFP4) MFMA
MFMA_FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
METRIC = "quant/dequant GB/s (% HBM peak); MXFP4 grouped-GEMM TFLOP/s (% MFMA peak)"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--legs", default="all", help="comma-separated leg-name prefixes to run (profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


class Leg:
    def __init__(self, name, kernel, kind, work, fn, reps=1, peak=None, rule_ops=None):
        self.name, self.kernel, self.kind, self.work, self.fn, self.reps = name, kernel, kind, work, fn, reps
        self.rule_ops = rule_ops   # fp32 operations per call of an exhaustive search rule (all candidates)
        # the roof this leg's rate is a fraction of (TFLOP/s or GB/s)
        self.peak = peak or (MFMA_BF16_PEAK_TFLOPS if kind == "flop" else HBM_PEAK_GBPS)
        self.ms = 0.0   # summed event time over the timed steps

    def run(self, step):
        for r in range(self.reps):
            self.fn(step * self.reps + r)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(the workloads are one GPU's share; see the sharding notes).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import synth
    import nvfp4_quantization_grouped_amd as mxq

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    L = mxq.lib()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream       # every leg runs on this stream; its events are recorded on it
    want = None if args.legs == "all" else [p.strip() for p in args.legs.split(",")]

    def wanted(name):   # a leg (or a group prefix of legs) asked for by --legs
        return want is None or any(name.startswith(p) or p.startswith(name) for p in want)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def check(st, what):
        if st != 0:
            raise RuntimeError(f"{what}: {L.mxq_status_string(st).decode()}")

    legs = []
    t_gen = time.perf_counter()

    # ---------------- routed-expert layer (gate/up + down, fwd + grad_x)
    moe = bulk = kv = None
    if wanted("moe") or wanted("w4a4") or wanted("w4a8"):
        moe = synth.moe_layer(seed=0)
        T = int(moe["offs"][-1])
        E, H, I2, I = 32, 7168, 4096, 2048
        offs = torch.from_numpy(moe["offs"]).to(dev)
        gu_p, gu_s = torch.from_numpy(moe["gu_packed"]).to(dev), torch.from_numpy(moe["gu_scales"]).to(dev)
        dn_p, dn_s = torch.from_numpy(moe["dn_packed"]).to(dev), torch.from_numpy(moe["dn_scales"]).to(dev)
        x_routed = bf16(moe["tokens_x"])[torch.from_numpy(moe["row_token"]).to(dev)].contiguous()
        h = bf16(moe["h"])
        gu_g, dn_g = bf16(moe["gu_grad"]), bf16(moe["dn_grad"])
        gu_y = torch.empty(T, I2, dtype=torch.bfloat16, device=dev)
        dn_y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        dn_gx = torch.empty(T, I, dtype=torch.bfloat16, device=dev)
        gu_gx = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        moe_rows = int(moe["counts"].sum())

        def fwd(a, p, s, n, k, y):
            return lambda i: check(L.mxfp4_grouped_mm_fwd(a.data_ptr(), T, k, p.data_ptr(), s.data_ptr(), E, n,
                                                          offs.data_ptr(), y.data_ptr(), sp), "fwd")

        def bwd(g, p, s, n, k, gx):
            return lambda i: check(L.mxfp4_grouped_mm_bwd_x(g.data_ptr(), T, n, p.data_ptr(), s.data_ptr(), E, k,
                                                            offs.data_ptr(), gx.data_ptr(), sp), "bwd_x")

        legs += [
            Leg("moe.gate_up.fwd", "k_grouped_mm_fwd_fl128", "flop", 2.0 * moe_rows * I2 * H, fwd(x_routed, gu_p, gu_s, I2, H, gu_y)),
            Leg("moe.down.fwd", "k_grouped_mm_fwd_fl128", "flop", 2.0 * moe_rows * H * I, fwd(h, dn_p, dn_s, H, I, dn_y)),
            Leg("moe.down.bwd_x", "k_grouped_mm_bwd", "flop", 2.0 * moe_rows * H * I, bwd(dn_g, dn_p, dn_s, H, I, dn_gx)),
            Leg("moe.gate_up.bwd_x", "k_grouped_mm_bwd", "flop", 2.0 * moe_rows * I2 * H, bwd(gu_g, gu_p, gu_s, I2, H, gu_gx)),
        ]

        # the same forwards as W4A4: the activations quantized to MXFP4
        # (quantize_mxfp4), then the block-scaled fp4 MFMA GEMM
        if wanted("w4a4"):
            gu_xq = torch.empty(T, H // 2, dtype=torch.int8, device=dev)
            gu_xs = torch.empty(T, H // 32, dtype=torch.uint8, device=dev)
            dn_xq = torch.empty(T, I // 2, dtype=torch.int8, device=dev)
            dn_xs = torch.empty(T, I // 32, dtype=torch.uint8, device=dev)

            def quant(a, k, xq, xs):
                return lambda i: check(L.quantize_mxfp4(a.data_ptr(), mxq._lib.MXQ_BF16, T, k, xq.data_ptr(),
                                                        xs.data_ptr(), sp), "quantize x")

            def w4(xq, xs, p, s, n, k, y):
                return lambda i: check(L.mxfp4_grouped_mm_fwd_w4a4(xq.data_ptr(), xs.data_ptr(), T, k, p.data_ptr(),
                                                                   s.data_ptr(), E, n, offs.data_ptr(), y.data_ptr(),
                                                                   sp), "w4a4 fwd")

            legs += [
                Leg("w4a4.gate_up.quantize_x", "k_quantize_mxfp4<bf16>", "byte", T * H * (2 + 0.5 + 1 / 32),
                    quant(x_routed, H, gu_xq, gu_xs)),
                Leg("w4a4.gate_up.fwd", "k_grouped_mm_fwd_w4a4_128", "flop", 2.0 * moe_rows * I2 * H,
                    w4(gu_xq, gu_xs, gu_p, gu_s, I2, H, gu_y), peak=MFMA_FP4_PEAK_TFLOPS),
                Leg("w4a4.down.quantize_x", "k_quantize_mxfp4<bf16>", "byte", T * I * (2 + 0.5 + 1 / 32),
                    quant(h, I, dn_xq, dn_xs)),
                Leg("w4a4.down.fwd", "k_grouped_mm_fwd_w4a4_128", "flop", 2.0 * moe_rows * H * I,
                    w4(dn_xq, dn_xs, dn_p, dn_s, H, I, dn_y), peak=MFMA_FP4_PEAK_TFLOPS),
            ]

        # the same forwards as W4A8: the activations encoded as E4M3 with E8M0
        # block-32 scales (quantize_cache_packed, fp8), then the fp8 x fp4 GEMM
        if wanted("w4a8"):
            gu_x8 = torch.empty(T, H, dtype=torch.uint8, device=dev)
            gu_s8 = torch.empty(T, H // 32, dtype=torch.uint8, device=dev)
            dn_x8 = torch.empty(T, I, dtype=torch.uint8, device=dev)
            dn_s8 = torch.empty(T, I // 32, dtype=torch.uint8, device=dev)

            def enc8(a, k, xq, xs):
                return lambda i: check(L.quantize_cache_packed(a.data_ptr(), mxq._lib.MXQ_BF16, T, k, mxq._lib.MXQ_FMT_FP8,
                                                               32, xq.data_ptr(), xs.data_ptr(), sp), "encode x fp8")

            def w8(xq, xs, p, s, n, k, y):
                return lambda i: check(L.mxfp4_grouped_mm_fwd_w4a8(xq.data_ptr(), xs.data_ptr(), T, k, p.data_ptr(),
                                                                   s.data_ptr(), E, n, offs.data_ptr(), y.data_ptr(),
                                                                   sp), "w4a8 fwd")

            legs += [
                Leg("w4a8.gate_up.quantize_x", "k_quantize_cache_packed<bf16,fp8,4>", "byte", T * H * (2 + 1 + 1 / 32),
                    enc8(x_routed, H, gu_x8, gu_s8)),
                Leg("w4a8.gate_up.fwd", "k_grouped_mm_fwd_w4a8", "flop", 2.0 * moe_rows * I2 * H,
                    w8(gu_x8, gu_s8, gu_p, gu_s, I2, H, gu_y), peak=MFMA_FP8_PEAK_TFLOPS),
                Leg("w4a8.down.quantize_x", "k_quantize_cache_packed<bf16,fp8,4>", "byte", T * I * (2 + 1 + 1 / 32),
                    enc8(h, I, dn_x8, dn_s8)),
                Leg("w4a8.down.fwd", "k_grouped_mm_fwd_w4a8", "flop", 2.0 * moe_rows * H * I,
                    w8(dn_x8, dn_s8, dn_p, dn_s, H, I, dn_y), peak=MFMA_FP8_PEAK_TFLOPS),
            ]

    # ---------------- 8-expert grouped GEMM forward (4 rotating buffer sets > 256 MB)
    if wanted("e8"):
        e8 = synth.grouped_mm_e8(seed=0)
        R8 = 4
        e8_x = [bf16(e8["x"]) for _ in range(R8)]
        e8_p = [torch.from_numpy(e8["packed"]).to(dev) for _ in range(R8)]
        e8_s = [torch.from_numpy(e8["scales"]).to(dev) for _ in range(R8)]
        e8_o = torch.from_numpy(e8["offs"]).to(dev)
        e8_y = [torch.empty(4096, 2048, dtype=torch.bfloat16, device=dev) for _ in range(R8)]

        def e8_fn(i):
            j = i % R8
            check(L.mxfp4_grouped_mm_fwd(e8_x[j].data_ptr(), 4096, 4096, e8_p[j].data_ptr(), e8_s[j].data_ptr(), 8,
                                         2048, e8_o.data_ptr(), e8_y[j].data_ptr(), sp), "e8 fwd")
        legs.append(Leg("e8.fwd", "k_grouped_mm_fwd_fl128_by_height", "flop", 2.0 * 4096 * 2048 * 4096, e8_fn, reps=R8))

    # ---------------- KV cache quantize_cache x3 + STE: 32 calls per step over 16 rotating sets of
    # 32 MiB in + 32 MiB out (537 MB of inputs per leg, twice the Infinity Cache), separate inputs per
    # leg, so no call reads what an earlier one left in the cache
    if wanted("kv"):
        kv = synth.kv_cache(seed=0)
        R, KV_REPS = 16, 32
        kv_xs = {fmt: [bf16(kv["x"]) for _ in range(R)] for fmt in ("fp8", "mxfp4", "nvfp4")}
        kv_o = [torch.empty_like(kv_xs["fp8"][0]) for _ in range(R)]
        kv_g = [bf16(kv["grad"]) for _ in range(R)]
        kv_gi = [torch.empty_like(kv_g[0]) for _ in range(R)]
        n_kv = kv_o[0].numel()
        rows_kv, C_kv = n_kv // 512, 512
        for fmt, code, block in [("fp8", 0, 128), ("mxfp4", 1, 32), ("nvfp4", 2, 16)]:
            def f(i, code=code, block=block, kv_x=kv_xs[fmt]):
                j = i % R
                check(L.quantize_cache(kv_x[j].data_ptr(), kv_o[j].data_ptr(), 1, rows_kv, C_kv, code, block, sp), "kv")
            legs.append(Leg(f"kv.quantize_cache.{fmt}", f"k_quantize_cache<bf16,{fmt},{block // 8}>", "byte",
                            4.0 * n_kv, f, reps=KV_REPS))

        def ste(i):
            j = i % R
            check(L.quantize_cache_bwd(kv_g[j].data_ptr(), kv_gi[j].data_ptr(), 1, n_kv, sp), "ste")
        legs.append(Leg("kv.ste_bwd", "k_copy16", "byte", 4.0 * n_kv, ste, reps=KV_REPS))

        # packed KV storage: store codes + scale bytes, dequantize on read (same rotating inputs)
        for fmt, code, block in [("fp8", 0, 128), ("mxfp4", 1, 32), ("nvfp4", 2, 16)]:
            cb = 1.0 if fmt == "fp8" else 0.5
            kv_c = [torch.empty(int(n_kv * cb), dtype=torch.uint8, device=dev) for _ in range(R)]
            kv_s = [torch.empty(n_kv // block, dtype=torch.uint8, device=dev) for _ in range(R)]

            def fq(i, code=code, block=block, kv_x=kv_xs[fmt], kv_c=kv_c, kv_s=kv_s):
                j = i % R
                check(L.quantize_cache_packed(kv_x[j].data_ptr(), 1, rows_kv, C_kv, code, block, kv_c[j].data_ptr(),
                                              kv_s[j].data_ptr(), sp), "kv.pack")

            def fd(i, code=code, block=block, kv_c=kv_c, kv_s=kv_s):
                j = i % R
                check(L.dequantize_cache_packed(kv_c[j].data_ptr(), kv_s[j].data_ptr(), rows_kv, C_kv, code, block,
                                                kv_o[j].data_ptr(), 1, sp), "kv.unpack")
            legs.append(Leg(f"kv.pack.{fmt}", f"k_quantize_cache_packed<bf16,{fmt},{block // 8}>", "byte",
                            n_kv * (2 + cb + 1 / block), fq, reps=KV_REPS))
            legs.append(Leg(f"kv.unpack.{fmt}", f"k_dequantize_cache_packed<bf16,{fmt},{block // 8}>", "byte",
                            n_kv * (cb + 1 / block + 2), fd, reps=KV_REPS))

    # ---------------- bulk bf16 [65536, 7168] + 2^30-parameter weight dequant
    if wanted("bulk"):
        bulk = synth.bulk_stream(seed=0)
        bx = bf16(bulk["x"])
        nb = bx.numel()
        br, bc = bx.shape
        bpk = torch.empty(br, bc // 2, dtype=torch.int8, device=dev)
        bsc = torch.empty(br, bc // 32, dtype=torch.uint8, device=dev)
        bdq = torch.empty_like(bx)
        bco = torch.empty_like(bx)
        wp, ws = torch.from_numpy(bulk["w_packed"]).to(dev), torch.from_numpy(bulk["w_scales"]).to(dev)
        wout = torch.empty(64, 4096, 4096, dtype=torch.bfloat16, device=dev)
        legs.append(Leg("bulk.quantize_mxfp4", "k_quantize_mxfp4<bf16>", "byte", nb * (2 + 0.5 + 1 / 32),
                        lambda i: check(L.quantize_mxfp4(bx.data_ptr(), 1, br, bc, bpk.data_ptr(), bsc.data_ptr(), sp), "q")))
        legs.append(Leg("bulk.dequantize_mxfp4", "k_dequantize_mxfp4<bf16>", "byte", nb * (0.5 + 1 / 32 + 2),
                        lambda i: check(L.dequantize_mxfp4(bpk.data_ptr(), bsc.data_ptr(), br, bc, bdq.data_ptr(), 1, sp), "dq")))
        for fmt, code, block in [("nvfp4", 2, 16), ("fp8", 0, 128), ("mxfp4", 1, 32)]:
            legs.append(Leg(f"bulk.quantize_cache.{fmt}", f"k_quantize_cache<bf16,{fmt},{block // 8}>", "byte", 4.0 * nb,
                            lambda i, code=code, block=block: check(
                                L.quantize_cache(bx.data_ptr(), bco.data_ptr(), 1, br, bc, code, block, sp), "qc")))
        # two-level NVFP4: the tensor max must be known before any block is
        # scaled, so the input is read twice (algorithmic bytes: 2 reads + outputs)
        npk = torch.empty(br, bc // 2, dtype=torch.uint8, device=dev)
        nsc = torch.empty(br, bc // 16, dtype=torch.uint8, device=dev)
        ng = torch.zeros(1, dtype=torch.float32, device=dev)
        legs.append(Leg("bulk.quantize_nvfp4", "k_nvfp4_amax+k_quantize_nvfp4<bf16>", "byte", nb * (2 * 2 + 0.5 + 1 / 16),
                        lambda i: check(L.quantize_nvfp4(bx.data_ptr(), 1, br, bc, npk.data_ptr(), nsc.data_ptr(),
                                                         ng.data_ptr(), sp), "qnv")))
        legs.append(Leg("bulk.dequantize_nvfp4", "k_dequantize_nvfp4<bf16>", "byte", nb * (0.5 + 1 / 16 + 2),
                        lambda i: check(L.dequantize_nvfp4(npk.data_ptr(), nsc.data_ptr(), ng.data_ptr(), br, bc,
                                                           bdq.data_ptr(), 1, sp), "dqnv")))
        # MSE block-scale sweep of one bf16 weight [4096, 7168]: 126 candidate scales per block of 16
        # (bytes: the amax read + the sweep read + outputs)
        nvw = bf16(synth.nvfp4_weight(seed=0)["w"])
        mr, mc = nvw.shape
        mpk = torch.empty(mr, mc // 2, dtype=torch.uint8, device=dev)
        msc = torch.empty(mr, mc // 16, dtype=torch.uint8, device=dev)
        mg = torch.zeros(1, dtype=torch.float32, device=dev)
        legs.append(Leg("bulk.quantize_nvfp4_mse", "k_nvfp4_amax+k_quantize_nvfp4_mse<bf16>", "byte",
                        nvw.numel() * (2 * 2 + 0.5 + 1 / 16),
                        lambda i: check(L.quantize_nvfp4_mse(nvw.data_ptr(), 1, mr, mc, mpk.data_ptr(), msc.data_ptr(),
                                                             mg.data_ptr(), sp), "qmse"), rule_ops=6.0 * 126 * nvw.numel()))
        nw = 64 * 4096 * 4096
        legs.append(Leg("bulk.weight_dequant", "k_dequantize_mxfp4<bf16>", "byte", nw * (0.5 + 1 / 32 + 2),
                        lambda i: check(L.dequantize_mxfp4(wp.data_ptr(), ws.data_ptr(), 64 * 4096, 4096,
                                                           wout.data_ptr(), 1, sp), "wdq")))

    # ---------------- fp32 [256, 1024] round trip (latency-bound; 64 rotating sets)
    if wanted("roundtrip"):
        rt = synth.roundtrip_f32(seed=0)
        RR = 64
        rx = [torch.from_numpy(rt["x"]).to(dev) for _ in range(RR)]
        rp = [torch.empty(256, 512, dtype=torch.int8, device=dev) for _ in range(RR)]
        rs = [torch.empty(256, 32, dtype=torch.uint8, device=dev) for _ in range(RR)]
        ro = [torch.empty(256, 1024, dtype=torch.float32, device=dev) for _ in range(RR)]

        def rt_fn(i):
            j = i % RR
            check(L.quantize_mxfp4(rx[j].data_ptr(), 0, 256, 1024, rp[j].data_ptr(), rs[j].data_ptr(), sp), "rt q")
            check(L.dequantize_mxfp4(rp[j].data_ptr(), rs[j].data_ptr(), 256, 1024, ro[j].data_ptr(), 0, sp), "rt dq")
        legs.append(Leg("roundtrip.f32", "k_quantize_mxfp4<f32>+k_dequantize_mxfp4<f32>", "byte",
                        2 * 262144 * (4 + 0.5 + 1 / 32), rt_fn, reps=8))

    legs = [l for l in legs if wanted(l.name)]
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen

    for s in range(args.warmup):
        for leg in legs:
            leg.run(s)
    torch.cuda.synchronize()

    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in legs]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for j, leg in enumerate(legs):
            evs[s][j][0].record(stream)
            leg.run(args.warmup + s)
            evs[s][j][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for s in range(args.steps):
        for j, leg in enumerate(legs):
            leg.ms += evs[s][j][0].elapsed_time(evs[s][j][1])

    K = args.steps
    out_legs = []
    for leg in legs:
        per_call_ms = leg.ms / (K * leg.reps)
        d = {"name": leg.name, "kernel": leg.kernel, "us": round(per_call_ms * 1e3, 2)}
        if leg.kind == "flop":
            rate = leg.work / (per_call_ms * 1e-3) / 1e12
            d.update({"tflop": round(leg.work / 1e12, 4), "TFLOP/s": round(rate, 1),
                      "frac_mfma": round(rate / leg.peak, 4)})
            if leg.peak != MFMA_BF16_PEAK_TFLOPS:
                d["peak_TFLOP/s"] = leg.peak
        else:
            rate = leg.work / (per_call_ms * 1e-3) / 1e9
            d.update({"GB": round(leg.work / 1e9, 4), "GB/s": round(rate, 1), "frac_hbm": round(rate / HBM_PEAK_GBPS, 4)})
        if leg.rule_ops:
            # the rule's work over the event time; the kernel skips candidates an exact lower bound
            # rules out, so this rate can pass the fp32 issue rate and has no roofline fraction
            d.update({"bound": "alu", "rule_Tops/s": round(leg.rule_ops / (per_call_ms * 1e-3) / 1e12, 2),
                      "rule_ops_per_call": leg.rule_ops})
            for k in ("GB/s", "frac_hbm"):
                d.pop(k, None)
        out_legs.append(d)

    moe_legs = [l for l in legs if l.name.startswith("moe.")]
    moe_rows = int(moe["counts"].sum()) if moe is not None else 0
    moe_flop = sum(l.work for l in moe_legs)
    moe_ms = sum(l.ms for l in moe_legs) / K
    value = moe_flop / (moe_ms * 1e-3) / 1e12 if moe_ms > 0 else None
    # HBM aggregates: the quantize/dequantize and fake-quant cache rows of the
    # path (mxfp4 codec, quantize_cache and its straight-through copy, weight
    # dequant), and separately the rows built beyond them (packed KV storage,
    # two-level NVFP4)
    def is_next(l):
        return l.name.startswith(("kv.pack", "kv.unpack")) or "nvfp4" in l.name.split(".")[1] and not \
            l.name.startswith(("kv.quantize_cache", "bulk.quantize_cache"))

    def aggregate(ls):
        b = sum(l.work * l.reps for l in ls)
        ms = sum(l.ms for l in ls) / K
        return b / (ms * 1e-3) / 1e9 if ms > 0 else None

    codec = [l for l in legs if l.kind == "byte" and not l.rule_ops and not l.name.startswith(("roundtrip", "w4a4.", "w4a8."))]
    hbm_gbps = aggregate([l for l in codec if not is_next(l)])
    hbm_next_gbps = aggregate([l for l in codec if is_next(l)])

    # dominant kernel: the instantiation with the largest total event time
    by_kernel = {}
    for l in legs:
        b = by_kernel.setdefault(l.kernel, {"ms": 0.0, "work": 0.0, "launches": 0, "kind": l.kind, "peak": l.peak})
        b["ms"] += l.ms / K
        b["work"] += l.work * l.reps
        b["launches"] += l.reps
    dom_name, dom = max(by_kernel.items(), key=lambda kv: kv[1]["ms"])
    avg_launch_ms = dom["ms"] / dom["launches"]
    work_per_launch = dom["work"] / dom["launches"]
    if dom["kind"] == "flop":
        achieved, peak, unit, bound = work_per_launch / (avg_launch_ms * 1e-3) / 1e12, dom["peak"], "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = work_per_launch / (avg_launch_ms * 1e-3) / 1e9, dom["peak"], "GB/s", "hbm"
    traffic = measured_traffic(dom_name)
    roofline = {"bound": bound, "kernel": dom_name, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "avg_launch_us": round(avg_launch_ms * 1e3, 1),
                "work_per_launch": work_per_launch,
                "traffic": traffic["bytes_per_launch"] if traffic else None, "traffic_detail": traffic}

    cpu = None
    if not args.no_cpu_baseline and moe is not None:
        cpu = cpu_baseline(moe)
        cpu["codecs"] = cpu_baseline_codecs(bulk_x=bulk["x"] if bulk is not None else None,
                                            kv_x=kv["x"] if kv is not None else None)

    line = {
        "metric": METRIC,
        "value": round(value, 1) if value else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; synth/)",
        "config": {
            "workload": "routed-expert layer share (32 experts, hidden 7168, intermediate 2048, 131072 routed rows, "
                        "fwd + grad_x) + 8-expert GEMM [4096x4096 -> 2048] + bf16 KV cache [4,8192,512] fake-quant "
                        "fp8/128, mxfp4/32, nvfp4/16 + STE + packed KV store/load + bulk bf16 [65536,7168] codecs (mxfp4, two-level nvfp4, "
                        "cache fake-quant) + NVFP4 MSE scale sweep of a bf16 [4096,7168] weight + [64,4096,4096] weight dequant + W4A4 and W4A8 routed-expert forwards",
            "value_is": "grouped-GEMM TFLOP/s of the routed-expert layer legs (event time)",
            "moe_rows": moe_rows,
        },
        "hbm": {"GB/s": round(hbm_gbps, 1) if hbm_gbps else None,
                "frac": round(hbm_gbps / HBM_PEAK_GBPS, 4) if hbm_gbps else None,
                "legs": "quantize_mxfp4 / dequantize_mxfp4 / quantize_cache (fp8, mxfp4, nvfp4) / STE copy / "
                        "weight dequant legs (kv + bulk)"},
        "hbm_next": {"GB/s": round(hbm_next_gbps, 1) if hbm_next_gbps else None,
                     "frac": round(hbm_next_gbps / HBM_PEAK_GBPS, 4) if hbm_next_gbps else None,
                     "legs": "packed KV store/load and two-level NVFP4 quantize/dequantize legs"},
        "mfma": {"TFLOP/s": round(value, 1) if value else None,
                 "frac": round(value / MFMA_BF16_PEAK_TFLOPS, 4) if value else None},
        "w4a4": low_bit_summary(legs, K, "w4a4", MFMA_FP4_PEAK_TFLOPS),
        "w4a8": low_bit_summary(legs, K, "w4a8", MFMA_FP8_PEAK_TFLOPS),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "legs": out_legs,
        "setup_s": round(t_gen, 1),
    }
    print(json.dumps(line), flush=True)


def low_bit_summary(legs, K, prefix, peak):
    """The routed-expert forwards as W4A4 or W4A8: GEMM rate against the fp4
    or fp8 peak, and the rate with the activation quantization counted in."""
    g = [l for l in legs if l.name.startswith(prefix + ".") and l.kind == "flop"]
    q = [l for l in legs if l.name.startswith(prefix + ".") and l.kind == "byte"]
    if not g:
        return None
    flop = sum(l.work for l in g)
    g_ms, q_ms = sum(l.ms for l in g) / K, sum(l.ms for l in q) / K
    bf = [l for l in legs if l.name in ("moe.gate_up.fwd", "moe.down.fwd")]
    bf_ms = sum(l.ms for l in bf) / K
    enc = "quantize_mxfp4" if prefix == "w4a4" else "quantize_cache_packed fp8/32"
    return {"gemm_TFLOP/s": round(flop / (g_ms * 1e-3) / 1e12, 1),
            "frac_peak": round(flop / (g_ms * 1e-3) / 1e12 / peak, 4), "peak_TFLOP/s": peak,
            "with_quantize_TFLOP/s": round(flop / ((g_ms + q_ms) * 1e-3) / 1e12, 1),
            "speedup_vs_bf16_fwd": round(bf_ms / (g_ms + q_ms), 3) if len(bf) == 2 else None,
            "legs": f"{prefix}.gate_up + {prefix}.down forwards ({enc} of the activations + block-scaled MFMA GEMM)"}


def source_code_hash(path):
    """sha256 of a C++/HIP source with its comments removed and whitespace
    collapsed: the code the counters were taken on, not its wording."""
    import hashlib
    import re
    with open(path, encoding="utf-8") as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return hashlib.sha256(" ".join(src.split()).encode()).hexdigest()


def measured_traffic(kernel):
    """Bytes per launch of `kernel` past L2 (to Infinity Cache / HBM) from the
    committed counter summary (rocprofv3 FETCH_SIZE and WRITE_SIZE, scaled by
    what they read for the copy kernel), averaged over the launches the bench
    makes, or None when there is none or the kernel code changed since."""
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(kernel)
    if not k:
        return None
    if source_code_hash(os.path.join(here, k["source"])) != k["source_code_sha256"]:
        return None
    return {"bytes_per_launch": k["bytes_per_launch"], "fetch_bytes": k["fetch_bytes"],
            "write_bytes": k["write_bytes"], "unit": "bytes",
            "fetch_factor": rec.get("calibration", {}).get("fetch_factor"), "from": "profiles/traffic.json"}


def cpu_baseline(moe):
    """The oracle (float64 NumPy, unmodified) on a bounded sample of the
    routed-expert layer: gate/up forward of 1024 rows in each of 6 experts."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                           default=1)
    except Exception:
        blas_threads = None
    offs = moe["offs"]
    starts = np.concatenate([[0], offs[:-1]])
    experts = [e for e in range(len(offs)) if offs[e] - starts[e] >= 1024][:6]
    rows = np.concatenate([np.arange(starts[e], starts[e] + 1024) for e in experts])
    x_rows = oracle.from_dtype_bits(moe["tokens_x"][moe["row_token"][rows]], "bf16")
    t0 = time.perf_counter()
    y, _ = oracle.grouped_mm_rows(rows, moe["gu_packed"], moe["gu_scales"], offs, x_rows=x_rows)
    dt = time.perf_counter() - t0
    flop = 2.0 * len(rows) * moe["gu_packed"].shape[1] * moe["gu_packed"].shape[2] * 2
    return {"value": round(flop / dt / 1e12, 4), "unit": "TFLOP/s", "cores": blas_threads,
            "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"gate/up forward, 1024 rows x {len(experts)} experts (float64 dequant + BLAS matmul), "
                      f"{flop / 1e9:.0f} GFLOP in {dt:.1f} s"}


def cpu_baseline_codecs(bulk_x=None, kv_x=None):
    """The oracle's quantize / dequantize / quantize_cache (NumPy, one thread,
    unmodified) on row samples of the bulk bf16 [65536, 7168] activation and
    the bf16 [4, 8192, 512] KV cache; GB/s counts the same algorithmic bytes
    as the GPU legs."""
    import numpy as np
    import oracle
    import synth
    out = []
    cores = 1   # NumPy elementwise code runs on one thread

    def timed(name, fn, nbytes, sample, min_s=0.5):
        reps, t = 0, 0.0
        t0 = time.perf_counter()
        while t < min_s:
            fn()
            reps += 1
            t = time.perf_counter() - t0
        out.append({"name": name, "GB/s": round(nbytes * reps / t / 1e9, 4), "s_per_call": round(t / reps, 3),
                    "cores": cores, "kind": "oracle", "sample": sample})

    if bulk_x is None:
        bulk_x = synth.bulk_stream(seed=0)["x"]
    rows = 128
    xb = np.ascontiguousarray(bulk_x[:rows])
    n = xb.size
    sample = f"rows 0..{rows - 1} of the bf16 [65536, 7168] activation ({n} elements)"
    xf = oracle.from_dtype_bits(xb, "bf16")
    packed, scales = oracle.quantize_mxfp4(xf)
    timed("bulk.quantize_mxfp4", lambda: oracle.quantize_mxfp4(oracle.from_dtype_bits(xb, "bf16")),
          n * (2 + 0.5 + 1 / 32), sample)
    timed("bulk.dequantize_mxfp4", lambda: oracle.dequantize_mxfp4(packed, scales, "bf16"), n * (0.5 + 1 / 32 + 2),
          sample)
    for fmt, block in [("nvfp4", 16), ("fp8", 128), ("mxfp4", 32)]:
        timed(f"bulk.quantize_cache.{fmt}",
              lambda fmt=fmt, block=block: oracle.quantize_cache(oracle.from_dtype_bits(xb, "bf16"), fmt, block,
                                                                 "bf16"), 4.0 * n, sample)
    kv = (kv_x if kv_x is not None else synth.kv_cache(seed=0)["x"]).reshape(-1, 512)
    kvs = np.ascontiguousarray(kv[:2048])
    nk = kvs.size
    ksample = f"rows 0..2047 (of 32768) of the bf16 [4, 8192, 512] KV cache ({nk} elements)"
    for fmt, block in [("fp8", 128), ("mxfp4", 32), ("nvfp4", 16)]:
        timed(f"kv.quantize_cache.{fmt}",
              lambda fmt=fmt, block=block: oracle.quantize_cache(oracle.from_dtype_bits(kvs, "bf16"), fmt, block,
                                                                 "bf16"), 4.0 * nk, ksample)
    return out


if __name__ == "__main__":
    main()
