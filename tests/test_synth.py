"""The seeded generators produce the stated shapes and structure (small sizes)."""

import numpy as np

import synth


def test_roundtrip_structure():
    d = synth.roundtrip_f32(seed=0)
    x = d["x"]
    assert x.shape == (256, 1024) and x.dtype == np.float32
    blocks = x.reshape(-1, 32)
    assert len(d["zero_blocks"]) == 82 and len(d["outlier_blocks"]) == 82
    assert not set(d["zero_blocks"]) & set(d["outlier_blocks"])
    assert np.all(blocks[d["zero_blocks"]] == 0)
    assert np.all(np.max(np.abs(blocks[d["outlier_blocks"]]), axis=1) == 1000.0)
    again = synth.roundtrip_f32(seed=0)["x"]
    assert np.array_equal(x, again)


def test_kv_cache_small():
    d = synth.kv_cache(seed=0, batch=2, seq=64, channels=128)
    assert d["x"].shape == (2, 64, 128) and d["x"].dtype == np.uint16
    v = (d["x"].astype(np.uint32) << 16).view(np.float32)
    big = np.abs(v) >= 20
    assert big.sum() == int(0.001 * v.size)


def test_routing_structure():
    d = synth.moe_layer(seed=0, experts=32, hidden=64, inter=32, tokens=512, with_activations=False)
    counts = d["counts"]
    assert counts.sum() == 512 * 8
    assert (counts == 0).sum() >= 4
    assert counts.max() <= 512                     # distinct top-8: at most one row per token
    assert d["offs"][-1] == 512 * 8 and np.all(np.diff(d["offs"]) >= 0)
    rt = d["row_token"]
    for e in range(32):
        s = 0 if e == 0 else d["offs"][e - 1]
        seg = rt[s:d["offs"][e]]
        assert len(np.unique(seg)) == len(seg)


def test_grouped_e8_offsets():
    d = synth.grouped_mm_e8(seed=0, tokens=256, n=64, k=128)
    assert d["offs"].dtype == np.int32 and d["offs"][-1] == 256
    assert d["scales"].min() >= 117 and d["scales"].max() <= 123
