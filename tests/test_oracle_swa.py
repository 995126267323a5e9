"""Pins of the oracle's local sliding-window branch.

The window cache is FP8: one signed E4M3 byte per channel ("FP4 cache
entries, and why they're safe" in the course brief "DeepSeek-V4.1-Flash"
keeps the local cache in FP8).  Its encoder is pinned to PyTorch's own
float8_e4m3fn cast (a library routine, round to nearest even) and to a
brute-force nearest-value search; the joined attention is pinned to
textbook softmax attention over the concatenation of the selected Main KV
entries and the window entries ("The Paper" in the talk write-up
"DeepSeek V4.1 Flash: pushing the limits": the selection is joined to the
window's KV for one attention), and to the global-only oracle where the
window is empty or duplicates a selected entry.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

import oracle

GRID = np.array([oracle.e4m3_value(b) for b in range(256)])  # NaN at 0x7F and 0xFF


def _values(seed, n=200_000):
    rng = np.random.default_rng(seed)
    mag = np.exp2(rng.uniform(-12, 9, n))  # subnormals (< 2^-6) up to just past 448
    v = (mag * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    v[:4] = [0.0, -0.0, 448.0, -448.0]
    return v


def test_signed_e4m3_matches_torch_float8_cast():
    v = _values(0)
    v = v[np.abs(v) <= 448]
    got = oracle.e4m3_encode_signed(v)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_signed_e4m3_ties_to_even_code_at_every_midpoint():
    finite = [b for b in range(0x7F)]
    lo = np.array([GRID[b] for b in finite[:-1]])
    hi = np.array([GRID[b] for b in finite[1:]])
    mid = ((lo + hi) / 2).astype(np.float32)  # exact: neighbours differ by one ulp of the grid
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    for sign in (1.0, -1.0):
        got = oracle.e4m3_encode_signed(sign * mid)
        even = np.array([b if b % 2 == 0 else b + 1 for b in finite[:-1]], dtype=np.uint8)
        assert np.array_equal(got & 0x7F, even)
        assert np.all((got >> 7) == (1 if sign < 0 else 0))


def test_signed_e4m3_is_the_nearest_grid_value():
    v = _values(1, 20_000)
    got = oracle.e4m3_encode_signed(v)
    finite = np.array([b for b in range(256) if not np.isnan(GRID[b])])
    clipped = np.clip(v.astype(np.float64), -448, 448)
    d = np.abs(clipped[:, None] - GRID[finite][None, :])
    assert np.allclose(np.abs(clipped - GRID[got]), d.min(axis=1), rtol=0, atol=0)


def test_signed_e4m3_saturates_and_keeps_the_sign_of_zero():
    v = np.array([449.0, 464.0, 1e6, 3e38, -449.0, -1e6, -1e-9, 1e-9], np.float32)
    assert oracle.e4m3_encode_signed(v).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x80, 0x00]


def _setup(seed, R=3, Hq=16, n=300, K=40, W=140):
    rng = np.random.default_rng(seed)
    codes, scales = oracle.quantize(rng.standard_normal((n, 512)).astype(np.float32))
    q = rng.standard_normal((R, Hq, 512)).astype(np.float32)
    idx = rng.integers(-3, n + 20, (R, K)).astype(np.int32)  # some < 0, some >= visible
    visible = rng.integers(n // 2, n + 1, R).astype(np.int64)
    win_codes = oracle.e4m3_encode_signed(rng.standard_normal((W, 512)).astype(np.float32) * 2)
    return rng, q, codes, scales, idx, visible, win_codes


def _dense(q, xh, scale):
    z = scale * (q.astype(np.float64) @ xh.T)
    return softmax(z, axis=1) @ xh, logsumexp(z, axis=1)


@pytest.mark.parametrize("seed", [0, 1])
def test_joined_softmax_equals_dense_attention_over_the_concatenation(seed):
    rng, q, codes, scales, idx, visible, win_codes = _setup(seed)
    R = q.shape[0]
    win_start = rng.integers(0, 10, R).astype(np.int64)
    win_len = np.array([128, 1, 77])[:R].astype(np.int32)
    scale = 1 / np.sqrt(512)
    o, lse = oracle.attention_rows_swa(q, codes, scales, np.zeros(R, np.int64), idx, visible, win_codes,
                                       win_start, win_len, scale)
    xh_all = oracle.dequant(codes, scales)
    w_all = oracle.fp8_dequant(win_codes)
    for r in range(R):
        sel = [j for j in idx[r] if 0 <= j < visible[r]]
        xh = np.concatenate([xh_all[sel], w_all[win_start[r]:win_start[r] + win_len[r]]])
        want, want_lse = _dense(q[r], xh, scale)
        assert np.allclose(o[r], want, rtol=1e-6, atol=1e-6 * np.abs(want).max())
        assert np.allclose(lse[r], want_lse, rtol=1e-6, atol=1e-6)


def test_window_only_is_dense_attention_over_the_window():
    rng, q, codes, scales, idx, visible, win_codes = _setup(2, R=2)
    idx[:] = -1
    scale = 0.05
    o, lse = oracle.attention_rows_swa(q, codes, scales, np.zeros(2, np.int64), idx, visible, win_codes,
                                       np.array([0, 12], np.int64), np.array([128, 128], np.int32), scale)
    w_all = oracle.fp8_dequant(win_codes)
    for r, s0 in enumerate([0, 12]):
        want, want_lse = _dense(q[r], w_all[s0:s0 + 128], scale)
        assert np.allclose(o[r], want, rtol=1e-6, atol=1e-6 * np.abs(want).max())
        assert np.allclose(lse[r], want_lse, rtol=1e-6, atol=1e-6)


def test_empty_window_is_the_global_branch_alone():
    rng, q, codes, scales, idx, visible, win_codes = _setup(3)
    R = q.shape[0]
    z = np.zeros(R, np.int64)
    o, lse = oracle.attention_rows_swa(q, codes, scales, z, idx, visible, win_codes, z, np.zeros(R, np.int32), 0.04)
    o2, lse2 = oracle.attention_rows(q, codes, scales, z, idx, visible, 0.04)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_window_length_is_clamped_to_128():
    rng, q, codes, scales, idx, visible, win_codes = _setup(4, R=2)
    z = np.zeros(2, np.int64)
    a = oracle.attention_rows_swa(q, codes, scales, z, idx, visible, win_codes, z, np.array([128, 0], np.int32), 0.04)
    b = oracle.attention_rows_swa(q, codes, scales, z, idx, visible, win_codes, z, np.array([139, -5], np.int32), 0.04)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_window_copy_of_a_selected_entry_counts_like_a_duplicate_index():
    # With scale byte 0x38 (1.0) every dequantized FP4 value is an E4M3 value,
    # so a window entry can hold exactly a Main KV entry; joining it must equal
    # listing that entry twice in the selection.
    rng = np.random.default_rng(5)
    n = 50
    codes = rng.integers(0, 256, (n, 256)).astype(np.uint8)
    scales = np.full((n, 32), 0x38, np.uint8)
    xh = oracle.dequant(codes, scales)
    win_codes = oracle.e4m3_encode_signed(xh[[7, 30]].astype(np.float32))
    assert np.array_equal(oracle.fp8_dequant(win_codes), xh[[7, 30]])
    q = rng.standard_normal((1, 16, 512)).astype(np.float32)
    idx = np.array([[3, 7, 30, 41, -1]], np.int32)
    z = np.zeros(1, np.int64)
    o, lse = oracle.attention_rows_swa(q, codes, scales, z, idx, np.array([n]), win_codes, z,
                                       np.array([2], np.int32), 0.06)
    o2, lse2 = oracle.attention_rows(q, codes, scales, z, np.array([[3, 7, 30, 41, 7, 30]], np.int32),
                                     np.array([n]), 0.06)
    assert np.allclose(o, o2, rtol=1e-6, atol=1e-7) and np.allclose(lse, lse2, rtol=1e-6, atol=1e-7)


def test_nothing_to_attend_gives_zero_and_minus_inf():
    rng, q, codes, scales, idx, visible, win_codes = _setup(6, R=1)
    idx[:] = -1
    z = np.zeros(1, np.int64)
    o, lse = oracle.attention_rows_swa(q, codes, scales, z, idx, visible, win_codes, z, np.zeros(1, np.int32), 0.04)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_signed_e4m3_hand_worked_examples():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "e4m3_signed_examples.txt")
    rows = [l.split()[:2] for l in open(path) if l.strip() and not l.startswith("#")]
    v = np.array([float(a) for a, _ in rows], np.float32)
    want = np.array([int(b, 16) for _, b in rows], np.uint8)
    assert np.array_equal(oracle.e4m3_encode_signed(v), want)
