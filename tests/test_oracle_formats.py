"""Pins for oracle/formats.py: printed tables, the e2m1 format definition,
PyTorch's float8 casts, NumPy's float casts, and brute force."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "printed_facts.json")


@pytest.fixture(scope="module")
def facts():
    with open(GOLDEN) as f:
        return json.load(f)


def all_bf16_values():
    """Every finite bf16 value, as float64."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32).astype(np.float64)
    return v[np.isfinite(v)]


def test_printed_table_prefix(facts):
    pre = facts["e2m1_table_prefix"]["values"]
    assert np.array_equal(oracle.E2M1_TABLE[: len(pre)], np.array(pre))
    # entry 8 is printed as (positive) 0.0
    assert oracle.E2M1_TABLE[8] == 0.0 and not np.signbit(oracle.E2M1_TABLE[8])


def test_table_positive_half_is_printed_grid(facts):
    assert np.array_equal(oracle.E2M1_TABLE[:8], np.array(facts["e2m1_grid"]["values"]))


def test_printed_midpoints_and_block(facts):
    assert np.array_equal(oracle.E2M1_MIDPOINTS, np.array(facts["e2m1_midpoints"]["values"]))
    assert oracle.MXFP4_BLOCK_SIZE == facts["mxfp4_block_size"]["value"]
    assert oracle.E4M3_MAX == facts["e4m3_max"]["value"]


def test_midpoints_bisect_the_grid():
    g = oracle.E2M1_TABLE[:8]
    assert np.array_equal(oracle.E2M1_MIDPOINTS, (g[:-1] + g[1:]) / 2)


def e2m1_from_bitfields(code):
    """e2m1 by its bit fields: 1 sign, 2 exponent (bias 1), 1 mantissa bit;
    exponent 0 is subnormal (0 or 0.5)."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = (m * 0.5) if e == 0 else (2.0 ** (e - 1)) * (1 + m * 0.5)
    return -mag if s else mag


def test_table_matches_e2m1_bitfield_definition():
    for c in range(16):
        want = e2m1_from_bitfields(c)
        assert oracle.E2M1_TABLE[c] == want            # == ignores the sign of zero
    # the page's table decodes the negative-zero code as +0.0
    assert not np.signbit(oracle.E2M1_TABLE[8])


def brute_force_e2m1_magnitude(m):
    """Nearest grid value; ties to the even code (codes index the grid)."""
    grid = oracle.E2M1_TABLE[:8]
    out = np.empty(m.shape, dtype=np.int64)
    for i, v in enumerate(m):
        d = np.abs(grid - min(v, 6.0))
        best = np.flatnonzero(d == d.min())
        out[i] = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
    return out


def test_encode_vs_brute_force_all_bf16_magnitudes():
    v = all_bf16_values()
    v = v[(np.abs(v) <= 16.0)]
    got = oracle.e2m1_encode(v)
    want_mag = brute_force_e2m1_magnitude(np.abs(v))
    assert np.array_equal(got & 7, want_mag)
    assert np.array_equal((got >> 3) & 1, (v < 0).astype(np.uint8))


def test_encode_vs_generic_rounding_at_every_midpoint_and_neighbour():
    # e2m1 is the format (1 mantissa bit, smallest normal 2^0, max 6): nearest-even
    # rounding with saturation must land on the same grid value as the midpoint cast.
    mids = oracle.E2M1_MIDPOINTS
    pts = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 10),
                          np.nextafter(mids.astype(np.float32), np.float32(0)).astype(np.float64),
                          np.nextafter(mids.astype(np.float32), np.float32(10)).astype(np.float64),
                          np.linspace(0, 8, 4097)])
    got = oracle.E2M1_TABLE[oracle.e2m1_encode(pts)]
    want = np.minimum(F.round_to_format(pts, 1, 0, 6.0), 6.0)
    assert np.array_equal(got, want)


def test_tie_rule_printed(facts):
    for t in facts["ties_moved_up"]["values"]:
        lo = oracle.E2M1_TABLE[oracle.e2m1_encode(np.array([t - 1e-9]))[0]]
        hi = oracle.E2M1_TABLE[oracle.e2m1_encode(np.array([t]))[0]]
        assert hi > lo
    for t in (0.25, 1.25, 2.5, 5.0):    # the other midpoints keep ties down
        assert oracle.E2M1_TABLE[oracle.e2m1_encode(np.array([t]))[0]] < t


def test_byte_table_and_nibble_order():
    bt = oracle.e2m1_byte_table()
    assert bt.shape == (256, 2)
    codes = np.arange(16)
    for lo in codes:
        for hi in codes:
            b = lo | (hi << 4)
            assert bt[b, 0] == oracle.E2M1_TABLE[lo] and bt[b, 1] == oracle.E2M1_TABLE[hi]


def test_e8m0_decode_vs_torch():
    b = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = oracle.e8m0_decode(b)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.isnan(got[255])


def test_e4m3_round_vs_torch_all_bf16_in_range():
    v = all_bf16_values()
    v = v[np.abs(v) <= 448.0]
    got = oracle.e4m3_round(v)
    want = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_e4m3_round_vs_torch_random_f32():
    g = np.random.default_rng(1)
    v = (g.standard_normal(200000) * np.exp2(g.integers(-14, 9, 200000))).astype(np.float32)
    v = v[np.abs(v) <= 448]
    got = oracle.e4m3_round(v.astype(np.float64))
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(got, want)


def test_to_dtype_bits_vs_numpy_and_torch():
    g = np.random.default_rng(2)
    v = g.standard_normal(100000) * np.exp2(g.integers(-150, 130, 100000).astype(np.float64))
    v = np.concatenate([v, [0.0, -0.0, 65504.0, 65519.99, 65520.0, 2.0 ** -25, 3 * 2.0 ** -26,
                            float.fromhex("0x1.fep127"), float.fromhex("0x1.ffp127")]])
    f32 = F.to_dtype_bits(v, "f32")
    assert np.array_equal(f32, v.astype(np.float32).view(np.uint32))
    f16 = F.to_dtype_bits(v, "f16")
    assert np.array_equal(f16, v.astype(np.float16).view(np.uint16))
    # bf16: torch rounds float32 -> bfloat16 nearest-even; feed it values that
    # are exact in float32 so torch's own float64 -> float32 step is exact.
    v32 = v.astype(np.float32).astype(np.float64)
    bf = F.to_dtype_bits(v32, "bf16")
    want = torch.from_numpy(v32.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf, want)


def test_from_dtype_bits_roundtrip():
    bits16 = np.arange(1 << 16, dtype=np.uint16)
    for dt in ("bf16", "f16"):
        v = F.from_dtype_bits(bits16, dt)
        fin = np.isfinite(v)
        assert np.array_equal(F.to_dtype_bits(v[fin], dt), bits16[fin])
