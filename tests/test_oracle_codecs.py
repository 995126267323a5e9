"""Pins of the oracle's FP4 / E4M3 codecs and quantize-on-write.

The cache format is the one the course brief "DeepSeek-V4.1-Flash" gives in
"FP4 cache entries, and why they're safe": E2M1 elements, one E4M3 scale per
16 channels, no second-level scale, 256 + 32 = 288 bytes per 512-channel
entry, FP4-with-scale range 2,688 = 6 x 448.  Pins: the OCP format tables,
torch's own float8_e4m3fn cast (a library routine), hand-derived tie tables
and a worked group example, closed-form round trips and error bounds.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


def test_e2m1_decode_matches_ocp_table():
    for code, val in _read("e2m1_values.txt"):
        got = oracle.e2m1_value(int(code))
        assert got == float(val) and np.signbit(got) == np.signbit(float(val)), (code, got, val)


def test_e4m3_decode_matches_torch_float8_e4m3fn():
    bits = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = bits.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = np.array([oracle.e4m3_value(b) for b in range(256)])
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.all(np.isnan(got[nan]))
    assert np.array_equal(got[~nan], ref[~nan].astype(np.float64))
    # largest finite value times the largest E2M1 value = the pages' 2,688 range
    assert oracle.e4m3_value(0x7E) == 448.0 and 6.0 * oracle.e4m3_value(0x7E) == 2688.0


def _torch_e4m3(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_cast_on_midpoints_and_random():
    grid = np.array([oracle.e4m3_value(c) for c in range(0x7F)], dtype=np.float64)
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)  # midpoints are exact in fp32
    vals = [grid.astype(np.float32), mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))]
    rng = np.random.default_rng(0)
    vals.append(np.exp2(rng.uniform(-14, np.log2(448.0), 2_000_000)).astype(np.float32))
    bits = rng.integers(0, 0x43E00000, 2_000_000, dtype=np.uint32)  # every fp32 bit pattern in [0, 448)
    vals.append(bits.view(np.float32))
    v = np.concatenate(vals)
    v = v[v <= 448.0]
    assert np.array_equal(oracle.e4m3_encode(v), _torch_e4m3(v))


def test_e4m3_encode_ties_and_saturation_by_hand():
    cases = {
        2.0 ** -10: 0x00,  # midpoint of 0 and 2^-9 -> even code 0
        np.nextafter(np.float32(2.0 ** -10), np.float32(1)): 0x01,
        3 * 2.0 ** -10: 0x02,  # midpoint of 2^-9 (code 1) and 2^-8 (code 2)
        2.0 ** -6: 0x08,  # smallest normal
        2.5: 0x42,
        448.0: 0x7E,
        449.0: 0x7E,
        1e30: 0x7E,  # saturate (torch would give NaN above 464)
        0.0: 0x00,
    }
    for v, want in cases.items():
        assert int(oracle.e4m3_encode(np.array([v]))[0]) == want, (v, want)


def test_e2m1_encode_ties_table():
    for x, code in _read("e2m1_ties.txt"):
        assert int(oracle.e2m1_encode(np.array([float(x)]))[0]) == int(code), (x, code)


def test_e2m1_encode_thresholds_and_grid():
    grid = np.array([oracle.e2m1_value(c) for c in range(8)], dtype=np.float32)
    # every grid value (and its negation) encodes to itself
    for c in range(8):
        assert int(oracle.e2m1_encode(grid[c:c + 1])[0]) == c
        if c:
            assert int(oracle.e2m1_encode(-grid[c:c + 1])[0]) == c | 8
    # just inside each midpoint rounds towards that side
    mids = (grid[:-1] + grid[1:]) / 2
    below = oracle.e2m1_encode(np.nextafter(mids, np.float32(0)))
    above = oracle.e2m1_encode(np.nextafter(mids, np.float32(10)))
    assert list(below) == list(range(7)) and list(above) == list(range(1, 8))
    # monotone over a dense sweep, and decode(encode(x)) is the nearest grid value
    x = np.linspace(-8, 8, 400_001, dtype=np.float32)
    c = oracle.e2m1_encode(x)
    dec = np.array([oracle.e2m1_value(i) for i in range(16)])[c]
    dist = np.abs(np.abs(x)[:, None] - grid[None, :].astype(np.float64)).min(axis=1)
    assert np.all(np.abs(np.abs(dec) - np.abs(x)) == dist)
    mag = np.abs(dec)
    assert np.all(np.diff(mag[x >= 0]) >= 0) and np.all(np.diff(mag[x <= 0]) <= 0)


def test_quantize_worked_group_example():
    rows = {r[0]: r[1:] for r in _read("quant_group_example.txt")}
    x = np.tile(np.arange(16, dtype=np.float32), 32)[None]
    codes, scales = oracle.quantize(x)
    assert codes.shape == (1, 256) and scales.shape == (1, 32)  # 288 bytes per entry
    assert np.all(scales == int(rows["scale"][0], 16))
    assert list(codes[0, :8]) == [int(b, 16) for b in rows["bytes"]]
    nib = np.stack([codes[0, :8] & 15, codes[0, :8] >> 4], 1).reshape(-1)
    assert list(nib) == [int(c) for c in rows["codes"]]


def test_quantize_grid_values_round_trip_exactly():
    rng = np.random.default_rng(1)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    n = 64
    x = np.empty((n, 512))
    for r in range(n):
        for g in range(32):
            s = oracle.e4m3_value(int(rng.integers(8, 0x7F)))  # normal scales
            el = grid[rng.integers(0, 8, 16)] * rng.choice([-1, 1], 16)
            el[rng.integers(0, 16)] = 6.0 * rng.choice([-1, 1])  # amax = 6 s -> scale code exact
            x[r, g * 16:(g + 1) * 16] = el * s
    codes, scales = oracle.quantize(x.astype(np.float32))
    assert np.array_equal(oracle.dequant(codes, scales), x)
    # idempotent: quantizing the dequantized cache gives the same bytes
    c2, s2 = oracle.quantize(oracle.dequant(codes, scales).astype(np.float32))
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


def test_quantize_zero_and_tiny_groups():
    x = np.zeros((2, 512), dtype=np.float32)
    x[1, :16] = -1e-4  # amax/6 below 2^-10 -> scale code 0 -> every code 0 (not negative zero)
    x[1, 16] = 3.0
    codes, scales = oracle.quantize(x)
    assert np.all(codes[0] == 0) and np.all(scales[0] == 0)
    assert scales[1, 0] == 0 and np.all(codes[1, :8] == 0)
    assert scales[1, 1] == int(_torch_e4m3(np.array([0.5]))[0])


def test_quantize_scale_is_torch_e4m3_of_amax_over_6_and_error_bound():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((300, 512)).astype(np.float32)
    x[:, [3, 77, 300]] *= 20
    codes, scales = oracle.quantize(x)
    g = x.reshape(300, 32, 16)
    amax = np.abs(g).max(-1)
    assert np.array_equal(scales, _torch_e4m3((amax / np.float32(6)).astype(np.float32)).reshape(300, 32))
    s = np.array([oracle.e4m3_value(b) for b in range(256)])[scales][..., None]
    xh = oracle.dequant(codes, scales).reshape(300, 32, 16)
    # nearest-grid rounding of x/s: error at most half the local grid step (step <= 2 below 6)
    y = g / s
    step = np.where(np.abs(y) < 2, 0.5, np.where(np.abs(y) < 4, 1.0, 2.0))
    assert np.all(np.abs(xh / s - y) <= step / 2 + 1e-6)
    # the largest element of a group lands within a grid step of +-6
    assert np.all(np.abs(np.abs(xh).max(-1) / s[..., 0] - 6) <= 1.0 + 1e-6)
