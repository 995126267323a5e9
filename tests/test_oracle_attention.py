"""Pins of the oracle's sparse attention.

Attention over the selected entries reduces to textbook dense softmax
attention when every entry is selected (scipy's softmax/logsumexp over the
dequantized cache); one selected entry returns that entry; q = 0 returns the
mean; order of the index list does not matter; an empty selection returns
zeros with lse = -inf.  K = V = the dequantized 512-channel latent shared by
all query heads ("The Paper" in the talk write-up "DeepSeek V4.1 Flash:
pushing the limits"; "The global branch" in the "DeepSeek-V4.1-Flash" brief).
"""
import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle


def _cache(n, seed, outliers=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 512)).astype(np.float32)
    if outliers:
        x[:, [5, 100, 222, 300, 511]] *= 20
    return oracle.quantize(x)


@pytest.mark.parametrize("Hq,n,seed", [(16, 200, 0), (64, 300, 1), (16, 33, 2)])
def test_all_selected_equals_dense_softmax_attention(Hq, n, seed):
    codes, scales = _cache(n, seed, outliers=seed == 1)
    rng = np.random.default_rng(100 + seed)
    q = rng.standard_normal((Hq, 512)).astype(np.float32)
    scale = 1 / np.sqrt(512)
    idx = np.concatenate([np.arange(n), -np.ones(7)]).astype(np.int32)
    o, lse = oracle.attention(q, codes, scales, idx, n, scale)
    xh = oracle.dequant(codes, scales)
    z = scale * (q.astype(np.float64) @ xh.T)
    want = softmax(z, axis=1) @ xh
    assert np.allclose(o, want, rtol=1e-6, atol=1e-6 * np.abs(want).max())
    assert np.allclose(lse, logsumexp(z, axis=1), rtol=1e-6, atol=1e-6)


def test_single_entry_returns_that_entry_and_zero_query_returns_mean():
    codes, scales = _cache(50, 3)
    xh = oracle.dequant(codes, scales)
    q = np.random.default_rng(4).standard_normal((16, 512)).astype(np.float32)
    idx = np.array([-1, 17, 999, -5], np.int32)  # only 17 is valid (visible = 50)
    o, lse = oracle.attention(q, codes, scales, idx, 50, 0.1)
    assert np.array_equal(o, np.broadcast_to(xh[17].astype(np.float32), o.shape))
    z = 0.1 * (q.astype(np.float64) @ xh[17])
    assert np.allclose(lse, z, rtol=1e-6)
    sel = np.array([1, 4, 9, 16, 25, 36, 49], np.int32)
    o0, lse0 = oracle.attention(np.zeros((16, 512), np.float32), codes, scales, sel, 50, 0.1)
    assert np.array_equal(o0, np.broadcast_to(xh[sel].mean(0).astype(np.float32), o0.shape))
    assert np.allclose(lse0, np.log(len(sel)))


def test_permutation_invariance_and_empty_selection():
    codes, scales = _cache(400, 5)
    q = np.random.default_rng(6).standard_normal((64, 512)).astype(np.float32)
    idx = np.random.default_rng(7).permutation(400)[:256].astype(np.int32)
    o1, l1 = oracle.attention(q, codes, scales, idx, 400, 0.05)
    o2, l2 = oracle.attention(q, codes, scales, idx[::-1].copy(), 400, 0.05)
    assert np.allclose(o1, o2, rtol=1e-6, atol=1e-7) and np.allclose(l1, l2, rtol=1e-7)
    oe, le = oracle.attention(q, codes, scales, -np.ones(10, np.int32), 400, 0.05)
    assert np.all(oe == 0) and np.all(np.isneginf(le))
    # visibility: entries >= visible are skipped
    ov, _ = oracle.attention(q, codes, scales, np.array([10, 300], np.int32), 200, 0.05)
    assert np.array_equal(ov, np.broadcast_to(oracle.dequant(codes, scales)[10].astype(np.float32), ov.shape))


def test_rows_variant_matches_single_rows():
    codes, scales = _cache(600, 8)
    rng = np.random.default_rng(9)
    R, Hq, K = 3, 16, 64
    q = rng.standard_normal((R, Hq, 512)).astype(np.float32)
    starts = np.array([0, 200, 400])
    vis = np.array([200, 150, 200])
    idx = np.stack([rng.permutation(200)[:K] for _ in range(R)]).astype(np.int32)
    o, lse = oracle.attention_rows(q, codes, scales, starts, idx, vis, 0.07)
    for r in range(R):
        o1, l1 = oracle.attention(q[r], codes[starts[r]:], scales[starts[r]:], idx[r], vis[r], 0.07)
        assert np.array_equal(o[r], o1) and np.array_equal(lse[r], l1)
