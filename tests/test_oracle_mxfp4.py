"""Pins of the oracle's OCP MXFP4 indexer-key codec.

The course brief "DeepSeek-V4.1-Flash" ("FP4 cache entries, and why they're
safe") assumes indexer keys in OCP MXFP4: blocks of 32 values sharing one
8-bit power-of-two (E8M0) scale, E2M1 elements.  The pins hold the codec to
what that format fixes, without re-deriving its formula: the E8M0 value
table, the binade the scale puts every block maximum in, the nearest-value
choice of every element by brute force over the E2M1 grid, exact round trips
of representable blocks, and zero blocks.
"""
import numpy as np
import pytest

import oracle

E2M1 = np.array([oracle.e2m1_value(c) for c in range(16)])


def test_e8m0_table():
    assert oracle.e8m0_value(127) == 1.0
    assert oracle.e8m0_value(128) == 2.0 and oracle.e8m0_value(126) == 0.5
    assert oracle.e8m0_value(0) == 2.0 ** -127 and oracle.e8m0_value(254) == 2.0 ** 127
    assert np.isnan(oracle.e8m0_value(255))


def _blocks(seed, n=400):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 64)).astype(np.float32) * np.exp2(rng.uniform(-20, 20, (n, 1))).astype(np.float32)
    x[0] = 0.0
    x[1, :32] = 0.0           # one zero block
    x[2, 5] = 1e30            # one huge value
    x[3] = -x[3]
    return x


@pytest.mark.parametrize("seed", [0, 1])
def test_block_maximum_lands_in_the_top_binade(seed):
    x = _blocks(seed)
    codes, scales = oracle.mxfp4_quantize(x)
    X = np.array([[oracle.e8m0_value(int(s)) for s in row] for row in scales])
    amax = np.abs(x.reshape(len(x), 2, 32)).max(axis=2).astype(np.float64)
    nz = amax > 0
    ratio = amax[nz] / X[nz]
    assert np.all((ratio >= 4) & (ratio < 8))  # the largest element is at 4..6, or clamps to 6
    assert np.all(scales[~nz] == 0)


@pytest.mark.parametrize("seed", [2, 3])
def test_every_element_is_the_nearest_e2m1_value(seed):
    x = _blocks(seed)
    codes, scales = oracle.mxfp4_quantize(x)
    X = np.repeat(np.array([[oracle.e8m0_value(int(s)) for s in row] for row in scales]), 32, axis=1)
    q = (x / X.astype(np.float32)).astype(np.float64)  # fp32 division, as the format's conversion takes it
    c = np.empty(x.shape, np.uint8)
    c[:, 0::2] = codes & 15
    c[:, 1::2] = codes >> 4
    qc = np.clip(q, -6, 6)
    d = np.abs(qc[..., None] - E2M1[None, None, :])
    best = d.min(axis=2)
    assert np.array_equal(np.abs(qc - E2M1[c]), best)
    # ties go to the even code; the sign bit follows the value
    tie = (d == best[..., None]).sum(axis=2) > 1
    tie &= ~np.isin(np.abs(qc), [0.0])
    assert np.all(c[tie] % 2 == 0)
    assert np.all((c >> 3)[q < 0] == 1) and np.all((c >> 3)[q > 0] == 0)


def test_representable_blocks_round_trip_exactly():
    rng = np.random.default_rng(4)
    mags = E2M1[:8]
    for k in [-20, -3, 0, 1, 7, 30]:
        x = (rng.choice(mags, (50, 64)) * rng.choice([-1, 1], (50, 64))).astype(np.float64)
        x[:, 0] = 6.0   # block maxima of 6 or 4: the scale is exactly 2^k
        x[:, 32] = -4.0
        x = (x * 2.0 ** k).astype(np.float32)
        codes, scales = oracle.mxfp4_quantize(x)
        assert np.all(scales == 127 + k)
        assert np.array_equal(oracle.mxfp4_dequant(codes, scales), x)


def test_layout_low_nibble_is_the_even_channel():
    x = np.zeros((1, 64), np.float32)
    x[0, 0], x[0, 1], x[0, 33] = 6.0, -0.5, 1.0
    codes, scales = oracle.mxfp4_quantize(x)
    assert scales.tolist() == [[127, 125]]   # block maxima 6 (2^0) and 1 (2^-2)
    assert codes[0, 0] == (0x7 | (0x9 << 4))  # 6 -> code 7, -0.5 -> code 9
    assert codes[0, 16] == (0x0 | (0x6 << 4))  # channel 33: 1.0 / 2^-2 = 4 -> code 6, high nibble


def test_hand_worked_block():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_block_example.txt")
    rec = {l.split()[0]: l.split()[1:] for l in open(path) if l.strip() and not l.startswith("#")}
    x = np.zeros((1, 64), np.float32)
    x[0, :32] = np.arange(32) / 4.0
    codes, scales = oracle.mxfp4_quantize(x)
    assert scales[0].tolist() == [int(s) for s in rec["scales"]]
    assert codes[0].tolist() == [int(b, 16) for b in rec["codes"]]
