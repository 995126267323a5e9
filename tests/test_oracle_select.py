"""Pins of the oracle's indexer score, top-K, hierarchical pool and modes.

Scores: with integer-valued inputs every partial sum is exact, so any
summation order gives the integer closed form; with bf16-valued inputs every
product is exact in fp32, so the fixed fmaf chain equals plain sequential
fp32 addition, which numpy's float32 reproduces independently; with fp32
inputs the chain is recomputed in exact rational arithmetic with one
rounding to fp32 per fmaf step.  Selection:
brute force through numpy's lexsort on small inputs, with forced ties.
Modes: Reindex over a pool holding every position equals Full (the mode
table of the "DeepSeek-V4.1-Flash" course brief makes Reindex a re-scoring
of the same entries).
"""
import numpy as np
import pytest

import oracle
from gen import bf16_round


def _dense_relu_sum(q, k):
    return np.maximum(k @ q.T, 0).sum(axis=1)


def test_index_score_integer_inputs_closed_form():
    rng = np.random.default_rng(0)
    for H in (1, 4, 8):
        q = rng.integers(-8, 9, (H, 64)).astype(np.float32)
        k = rng.integers(-8, 9, (5000, 64)).astype(np.float32)
        want = _dense_relu_sum(q.astype(np.int64), k.astype(np.int64)).astype(np.float32)
        assert np.array_equal(oracle.index_scores(q, k), want)


def test_index_score_bf16_inputs_equal_sequential_fp32_sum():
    rng = np.random.default_rng(1)
    H = 8
    q = bf16_round(rng.standard_normal((H, 64)).astype(np.float32))
    k = bf16_round(rng.standard_normal((3000, 64)).astype(np.float32))
    acc = np.zeros((3000, H), dtype=np.float32)
    for c in range(64):  # product exact in fp32, one rounding per addition
        acc = (acc + (k[:, c:c + 1] * q[None, :, c])).astype(np.float32)
    rel = np.maximum(acc, np.float32(0))
    s = rel[:, 0].copy()
    for h in range(1, H):
        s = (s + rel[:, h]).astype(np.float32)
    assert np.array_equal(oracle.index_scores(q, k), s)


def test_index_score_fp32_inputs_within_rounding_of_exact():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((4, 64)).astype(np.float32)
    k = rng.standard_normal((4000, 64)).astype(np.float32)
    got = oracle.index_scores(q, k).astype(np.float64)
    d = k.astype(np.float64) @ q.astype(np.float64).T
    exact = np.maximum(d, 0).sum(1)
    bound = (64 + 4) * 2.0 ** -24 * (np.abs(k.astype(np.float64)) @ np.abs(q.astype(np.float64)).T).sum(1)
    assert np.all(np.abs(got - exact) <= bound + 1e-30)


def _round_f32(x):
    """The fp32 value nearest to the exact rational x, ties to even (normal and subnormal ranges)."""
    from fractions import Fraction
    if x == 0:
        return Fraction(0)
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()  # 2^e <= a < 2^(e+2)
    if a < Fraction(2) ** e:
        e -= 1
    if a >= Fraction(2) ** (e + 1):
        e += 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    n, rem = divmod(a, quantum)
    n = int(n)
    if rem * 2 > quantum or (rem * 2 == quantum and n % 2 == 1):
        n += 1
    return (n * quantum) if x > 0 else -(n * quantum)


def _score_exact_chain(q, k, fused=True):
    """The indexer score written with exact rationals: per head an fmaf chain over the 64 channels from
    0 (one rounding to fp32 per step; fused=False rounds the product too, i.e. multiply then add), ReLU,
    then the head sum left to right with one rounding per addition."""
    from fractions import Fraction
    qf = [[Fraction(float(v)) for v in row] for row in q]
    kf = [Fraction(float(v)) for v in k]
    rel = []
    for h in range(len(qf)):
        acc = Fraction(0)
        for c in range(len(kf)):
            p = qf[h][c] * kf[c]
            acc = _round_f32(p + acc) if fused else _round_f32(_round_f32(p) + acc)
        rel.append(acc if acc > 0 else Fraction(0))
    s = rel[0]
    for h in range(1, len(rel)):
        s = _round_f32(s + rel[h])
    return float(s)


def test_round_f32_matches_the_fp32_cast():
    from fractions import Fraction
    rng = np.random.default_rng(9)
    for v in rng.standard_normal(300) * np.exp2(rng.integers(-140, 100, 300)):
        # the exact value of a double, rounded once to fp32, is numpy's float32 cast of that double
        assert _round_f32(Fraction(float(v))) == Fraction(float(np.float32(v)))
    assert _round_f32(Fraction(1) + Fraction(2) ** -24) == 1  # tie to even, down
    assert _round_f32(Fraction(1) + Fraction(3, 2 ** 24)) == 1 + Fraction(2) ** -22  # tie to even, up
    assert _round_f32(Fraction(2) ** -150) == 0 and _round_f32(Fraction(3, 2 ** 151)) == Fraction(2) ** -149


def test_index_score_fp32_inputs_equal_the_exact_fmaf_chain():
    """fp32 queries and keys (the tiny decode workload's indexer): each step of a head's chain is one
    fmaf, i.e. the exact product plus the running sum rounded once.  Rational arithmetic with one
    rounding per step gives every score bit for bit, and the multiply-then-add chain, which rounds
    twice per step, differs on some of these keys (so the check tells the two apart)."""
    rng = np.random.default_rng(21)
    H, n = 4, 160
    q = (rng.standard_normal((H, 64)) * np.exp2(rng.integers(-3, 4, (H, 64)))).astype(np.float32)
    k = (rng.standard_normal((n, 64)) * np.exp2(rng.integers(-3, 4, (n, 64)))).astype(np.float32)
    got = oracle.index_scores(q, k)
    want = np.array([_score_exact_chain(q, k[j]) for j in range(n)], np.float32)
    assert np.array_equal(got, want)
    unfused = np.array([_score_exact_chain(q, k[j], fused=False) for j in range(n)], np.float32)
    assert np.count_nonzero(unfused != want) > 0


def _brute_topk(s, K, pos=None):
    pos = np.arange(len(s)) if pos is None else np.asarray(pos)
    ok = pos >= 0
    s, pos = s[ok], pos[ok]
    order = np.lexsort((pos, -s.astype(np.float64)))
    keep = np.sort(pos[order[:K]])
    out = np.full(K, -1, np.int32)
    out[:len(keep)] = keep
    return out


@pytest.mark.parametrize("n,K", [(1, 4), (7, 4), (100, 16), (1000, 256), (5000, 256), (300, 512)])
def test_topk_brute_force_random(n, K):
    rng = np.random.default_rng(n)
    s = np.abs(rng.standard_normal(n)).astype(np.float32)
    assert np.array_equal(oracle.topk(s, K), _brute_topk(s, K))


def test_topk_forced_ties_go_to_lower_position():
    rng = np.random.default_rng(3)
    s = rng.integers(0, 5, 4000).astype(np.float32)  # heavy ties
    for K in (1, 10, 801, 2048, 4000, 4100):
        got = oracle.topk(s, K)
        assert np.array_equal(got, _brute_topk(s, K))
    z = np.zeros(1000, np.float32)
    assert np.array_equal(oracle.topk(z, 256), np.arange(256, dtype=np.int32))


def test_topk_with_positions_skips_negative():
    rng = np.random.default_rng(4)
    pos = rng.permutation(10000)[:3000].astype(np.int64)
    pos[rng.integers(0, 3000, 100)] = -1
    s = rng.integers(0, 50, 3000).astype(np.float32)
    assert np.array_equal(oracle.topk(s, 300, pos), _brute_topk(s, 300, pos))


def _brute_pool(s, P, block):
    n = len(s)
    nb = -(-n // block)
    pad = np.full(nb * block, -np.inf)
    pad[:n] = s
    bs = pad.reshape(nb, block).max(1)
    order = np.lexsort((np.arange(nb), -bs))
    keep = np.sort(order[:P // block])
    pos = (keep[:, None] * block + np.arange(block)[None]).reshape(-1)
    pos = pos[pos < n]
    out = np.full(P, -1, np.int32)
    out[:len(pos)] = pos
    return out, len(pos)


@pytest.mark.parametrize("n,P", [(5, 16), (64, 64), (1000, 64), (1003, 128), (20000, 1024), (4096, 4096), (4100, 4096)])
def test_hsi_pool_brute_force(n, P):
    rng = np.random.default_rng(n + P)
    s = np.abs(rng.standard_normal(n)).astype(np.float32)
    s[rng.integers(0, n, n // 3)] = 1.0  # ties between blocks
    pool, ln = oracle.hsi_pool(s, P, 8)
    want, wl = _brute_pool(s, P, 8)
    assert ln == wl and np.array_equal(pool, want)


def test_pool_counts_match_pages():
    # the pages' pool: 2,048 blocks of 8 -> 16,384 candidates
    s = np.abs(np.random.default_rng(5).standard_normal(1 << 20)).astype(np.float32)
    pool, ln = oracle.hsi_pool(s, 16384, 8)
    assert ln == 16384 and np.all(np.diff(pool) > 0)
    assert len(np.unique(pool // 8)) == 2048


def test_reindex_over_all_positions_equals_full():
    rng = np.random.default_rng(6)
    n, K = 6000, 512
    q = bf16_round(rng.standard_normal((8, 64)).astype(np.float32))
    k = bf16_round(rng.standard_normal((n, 64)).astype(np.float32))
    full, _, _ = oracle.full_select(q, k, n, K)
    pool = np.concatenate([np.arange(n), -np.ones(40, np.int64)])
    assert np.array_equal(oracle.reindex_select(q, k, pool, n, K), full)


def test_reindex_equals_brute_force_on_pool():
    rng = np.random.default_rng(7)
    n, K = 8000, 300
    q = bf16_round(rng.standard_normal((8, 64)).astype(np.float32))
    k = bf16_round(rng.standard_normal((n, 64)).astype(np.float32))
    s_all = oracle.index_scores(q, k)
    pool, ln = oracle.hsi_pool(s_all, 2048, 8)
    visible = 7000
    got = oracle.reindex_select(q, k, pool, visible, K)
    cand = pool[(pool >= 0) & (pool < visible)]
    assert np.array_equal(got, _brute_topk(s_all[cand], K, cand))


def test_compressed_visibility_counts_only_complete_blocks():
    """m tokens per entry (encoder layers fold m = 2): a query sees only the entries whose whole
    block lies at or before it.  The oracle is pinned by the block count itself (brute force over
    tokens) and by m = 1 reducing to the causal t + 1; the library computes it on the device
    (csa2_visible_entries, checked against the oracle in the GPU tests)."""
    for m in (1, 2, 3, 4):
        for t in range(0, 50):
            complete = sum(1 for e in range(t + 1) if all(m * e + k <= t for k in range(m)))
            assert oracle.visible_entries(t, m) == complete
    assert all(oracle.visible_entries(t, 1) == t + 1 for t in range(100))
    assert [oracle.visible_entries(t, 2) for t in range(6)] == [0, 1, 1, 2, 2, 3]
