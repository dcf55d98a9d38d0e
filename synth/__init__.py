"""Seeded synthetic inputs for the five workloads of the quantization / grouped-GEMM path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no scale rule, no rounding to e2m1/E4M3, no GEMM).  It is
the one piece of code both the CPU oracle and the HIP path are fed from.

All generators use NumPy ``Generator(PCG64)`` streams spawned from
``SeedSequence(seed)``, one stream per tensor, so every tensor is reproducible
on its own.  bf16 tensors are returned as uint16 bit patterns (NumPy has no
bfloat16), made by PyTorch's nearest-even float32 -> bfloat16 cast.

Workloads (the shapes of the KV caches and MoE expert weights on the pages):

* ``roundtrip_f32``   fp32 [256, 1024], normal(0,1) with each 32-column block
  scaled by 2^k, k uniform integer in [-8, 8]; 1% of the blocks zeroed and
  another, disjoint, 1% holding a single +-1000 outlier (mxfp4 round trip).
* ``kv_cache``        bf16 [4, 8192, 512], normal(0, 0.5), 0.1% of the entries
  replaced by +-uniform(20, 200); gradient bf16 normal(0, 1) (quantize_cache).
* ``grouped_mm_e8``   8 experts, packed [8, 2048, 2048] uniform bytes, scale
  bytes uniform in {117..123} (2^-10 .. 2^-4), x bf16 [4096, 4096] normal(0,1),
  counts multinomial(4096, uniform), cumulative int32 offsets.
* ``moe_layer``       32 local experts, hidden 7168, intermediate 2048: gate/up
  packed [32, 4096, 3584], down packed [32, 7168, 1024], same byte/scale
  distribution; 16384 tokens bf16 normal(0,1) routed top-8 (131072 grouped rows)
  with Zipf(1.1)-skewed expert popularity and 4 experts that receive no tokens;
  down-projection input bf16 normal(0,1) [131072, 2048]; output gradients
  normal(0, 0.1).
* ``bulk_stream``     bf16 [65536, 7168] normal(0,1) with per-row scale 2^k, k
  uniform integer in [-4, 4]; a 2^30-parameter packed weight [64, 4096, 2048]
  with scale bytes [64, 4096, 128] in {117..123}.
* ``nvfp4_weight``    bf16 [4096, 7168] (one expert's fused gate/up weight),
  normal(0, 0.02 * 2^k) with k in {-1, 0, 1} per row, 0.1% of the entries
  multiplied by uniform(4, 16) (NVFP4 MSE scale sweep).
"""

import numpy as np

SCALE_BYTE_LO, SCALE_BYTE_HI = 117, 123   # E8M0 bytes for 2^-10 .. 2^-4


def streams(seed, n):
    """n independent PCG64 generators spawned from SeedSequence(seed)."""
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def f32_to_bf16_bits(a):
    """float32 array -> bf16 bit patterns (uint16), PyTorch's nearest-even cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def normal_bf16(g, shape, std=1.0, chunk_rows=4096):
    """bf16 bits of normal(0, std) drawn in float32, in row chunks to bound memory."""
    shape = tuple(shape)
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(shape[0], -1) if len(shape) > 1 else out.reshape(1, -1)
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(r0 + chunk_rows, flat.shape[0])
        v = g.standard_normal((r1 - r0, flat.shape[1]), dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        flat[r0:r1] = f32_to_bf16_bits(v)
    return out


def packed_weights(g_bytes, g_scales, experts, n, k):
    """Uniform random packed e2m1 bytes [E, N, K/2] (int8) and scale bytes
    [E, N, K/32] (uint8) uniform in {117..123}."""
    packed = g_bytes.integers(0, 256, size=(experts, n, k // 2), dtype=np.uint8).view(np.int8)
    scales = g_scales.integers(SCALE_BYTE_LO, SCALE_BYTE_HI + 1, size=(experts, n, k // 32), dtype=np.uint8)
    return packed, scales


def roundtrip_f32(seed=0, rows=256, cols=1024, block=32, special_frac=0.01):
    g_val, g_pow, g_pick, g_sign, g_pos = streams(seed, 5)
    x = g_val.standard_normal((rows, cols)).astype(np.float32)
    nb = cols // block
    k = g_pow.integers(-8, 9, size=(rows, nb))
    x = (x.reshape(rows, nb, block) * np.ldexp(np.float32(1.0), k)[..., None].astype(np.float32)).astype(np.float32)
    n_special = int(round(special_frac * rows * nb))
    pick = g_pick.permutation(rows * nb)[: 2 * n_special]
    zero_blocks, outlier_blocks = pick[:n_special], pick[n_special:]
    xb = x.reshape(rows * nb, block)
    xb[zero_blocks] = 0.0
    signs = np.where(g_sign.integers(0, 2, size=n_special) == 1, 1.0, -1.0).astype(np.float32)
    pos = g_pos.integers(0, block, size=n_special)
    xb[outlier_blocks, pos] = signs * np.float32(1000.0)
    return {"x": xb.reshape(rows, cols).astype(np.float32),
            "zero_blocks": np.sort(zero_blocks), "outlier_blocks": np.sort(outlier_blocks)}


def kv_cache(seed=0, batch=4, seq=8192, channels=512, std=0.5, outlier_frac=0.001):
    g_val, g_pick, g_mag, g_sign, g_grad = streams(seed, 5)
    shape = (batch, seq, channels)
    v = g_val.standard_normal(shape, dtype=np.float32) * np.float32(std)
    n = v.size
    n_out = int(outlier_frac * n)
    idx = g_pick.choice(n, size=n_out, replace=False)
    mag = g_mag.uniform(20.0, 200.0, size=n_out).astype(np.float32)
    sgn = np.where(g_sign.integers(0, 2, size=n_out) == 1, 1.0, -1.0).astype(np.float32)
    v.reshape(-1)[idx] = sgn * mag
    return {"x": f32_to_bf16_bits(v), "grad": normal_bf16(g_grad, shape, 1.0)}


def offsets_from_counts(counts):
    return np.cumsum(np.asarray(counts, dtype=np.int64)).astype(np.int32)


def grouped_mm_e8(seed=0, experts=8, tokens=4096, n=2048, k=4096):
    g_b, g_s, g_x, g_c = streams(seed, 4)
    packed, scales = packed_weights(g_b, g_s, experts, n, k)
    x = normal_bf16(g_x, (tokens, k))
    counts = g_c.multinomial(tokens, [1.0 / experts] * experts)
    return {"x": x, "packed": packed, "scales": scales, "offs": offsets_from_counts(counts),
            "counts": counts}


def zipf_top8_routing(g_perm, g_zero, g_gumbel, tokens, experts, topk=8, zipf_s=1.1, n_idle=4):
    """Per-token top-k expert choice: expert popularity Zipf(s) over a seeded
    permutation, ``n_idle`` seeded experts with weight 0, each token drawing
    k distinct experts by Gumbel-top-k.  Returns (token index of each grouped
    row, sorted stably by expert; per-expert counts)."""
    rank = g_perm.permutation(experts)                    # popularity rank of each expert
    w = 1.0 / np.power(rank + 1.0, zipf_s)
    idle = g_zero.choice(experts, size=n_idle, replace=False)
    w[idle] = 0.0
    logw = np.where(w > 0, np.log(np.where(w > 0, w, 1.0)), -np.inf)
    choice = np.empty((tokens, topk), dtype=np.int64)
    for t0 in range(0, tokens, 4096):
        t1 = min(t0 + 4096, tokens)
        gum = g_gumbel.gumbel(size=(t1 - t0, experts))
        choice[t0:t1] = np.argsort(-(logw[None, :] + gum), axis=1, kind="stable")[:, :topk]
    flat_expert = choice.reshape(-1)
    flat_token = np.repeat(np.arange(tokens), topk)
    order = np.argsort(flat_expert, kind="stable")
    counts = np.bincount(flat_expert, minlength=experts)
    return flat_token[order], counts


def moe_layer(seed=0, experts=32, hidden=7168, inter=2048, tokens=16384, topk=8, with_activations=True):
    (g_gb, g_gs, g_db, g_ds, g_x, g_perm, g_zero, g_gum, g_h, g_go1, g_go2) = streams(seed, 11)
    gu_packed, gu_scales = packed_weights(g_gb, g_gs, experts, 2 * inter, hidden)
    dn_packed, dn_scales = packed_weights(g_db, g_ds, experts, hidden, inter)
    row_token, counts = zipf_top8_routing(g_perm, g_zero, g_gum, tokens, experts, topk)
    out = {"gu_packed": gu_packed, "gu_scales": gu_scales, "dn_packed": dn_packed,
           "dn_scales": dn_scales, "row_token": row_token, "counts": counts,
           "offs": offsets_from_counts(counts)}
    if with_activations:
        rows = tokens * topk
        out["tokens_x"] = normal_bf16(g_x, (tokens, hidden))
        out["h"] = normal_bf16(g_h, (rows, inter))
        out["gu_grad"] = normal_bf16(g_go1, (rows, 2 * inter), 0.1)
        out["dn_grad"] = normal_bf16(g_go2, (rows, hidden), 0.1)
    return out


def bulk_stream(seed=0, rows=65536, cols=7168, with_weights=True):
    g_x, g_k, g_b, g_s = streams(seed, 4)
    k = g_k.integers(-4, 5, size=rows)
    x = np.empty((rows, cols), dtype=np.uint16)
    for r0 in range(0, rows, 4096):
        r1 = min(r0 + 4096, rows)
        v = g_x.standard_normal((r1 - r0, cols), dtype=np.float32)
        v *= np.ldexp(np.float32(1.0), k[r0:r1])[:, None].astype(np.float32)
        x[r0:r1] = f32_to_bf16_bits(v)
    out = {"x": x, "row_pow": k}
    if with_weights:
        out["w_packed"], out["w_scales"] = packed_weights(g_b, g_s, 64, 4096, 4096)
    return out


def nvfp4_weight(seed=0, rows=4096, cols=7168, std=0.02, outlier_frac=0.001):
    """bf16 weight [rows, cols] (one routed expert's fused gate/up projection,
    2 x 2048 outputs over hidden 7168): normal(0, std * 2^k) with k in
    {-1, 0, 1} per output row, and outlier_frac of the entries multiplied by
    U(4, 16)."""
    g_x, g_k, g_pick, g_mag = streams(seed, 4)
    k = g_k.integers(-1, 2, size=rows)
    v = g_x.standard_normal((rows, cols), dtype=np.float32)
    v *= (np.float32(std) * np.ldexp(np.float32(1.0), k)[:, None]).astype(np.float32)
    n_out = int(outlier_frac * v.size)
    idx = g_pick.choice(v.size, size=n_out, replace=False)
    v.reshape(-1)[idx] *= g_mag.uniform(4.0, 16.0, size=n_out).astype(np.float32)
    return {"w": f32_to_bf16_bits(v), "row_pow": k}

