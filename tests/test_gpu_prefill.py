"""GPU parity of the shared-segment indexer (a prefill chunk over one cache).

Mode CSA2_FULL_SHARED scores the chunk's rows with a bf16 MFMA product,
keeps every entry its proven error bound cannot rule out, rescores those
exactly and selects exactly.  Its indices must equal the oracle's top-K
over each row's causal prefix bit for bit, in the ordinary case, with
forced ties, when fewer than K entries are visible, and when a row's
candidates overflow the list (the exact full-scan fallback).
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from gen import bf16_round
from gpu_util import DEV, dev, dev_bf16, index_topk, say
from sparse_attention_fp4_e4m3_amd import csa2

pytestmark = pytest.mark.gpu


def _chunk(P0, T, H, seed, keys=None, iq=None):
    rng = np.random.default_rng(seed)
    n = P0 + T
    ik = bf16_round(rng.standard_normal((n, 64), dtype=np.float32)) if keys is None else keys
    q = bf16_round(rng.standard_normal((T, H, 64), dtype=np.float32)) if iq is None else iq
    return ik, q


def _run_shared(ik, q, P0, K, start_pad=0):
    T = q.shape[0]
    n = ik.shape[0]
    # the segment sits at row start_pad of a larger key array
    kk = np.zeros((n + start_pad, 64), np.float32)
    kk[start_pad:] = ik
    starts = dev(np.full(T, start_pad, np.int64))
    vis = dev((P0 + 1 + np.arange(T)).astype(np.int32))
    idx, _, _ = index_topk(csa2.FULL_SHARED, dev_bf16(q), dev_bf16(kk), starts, vis, n, K)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


def _check_rows(idx, ik, q, P0, K, rows):
    for r in rows:
        want = oracle.topk(oracle.index_scores(q[r], ik[:P0 + r + 1]), K)
        assert np.array_equal(idx[r], want), "row %d differs" % r


@pytest.mark.parametrize("H", [4, 8, 16])
def test_shared_matches_oracle(H):
    P0, T, K = 12000, 96, 512
    ik, q = _chunk(P0, T, H, seed=10 + H)
    idx = _run_shared(ik, q, P0, K, start_pad=37)
    _check_rows(idx, ik, q, P0, K, range(T))
    say("H=%d: %d rows exact" % (H, T))


def test_shared_equals_full_mode():
    """Same result as the exact Full path run row by row over the shared segment."""
    P0, T, K, H = 30000, 40, 1024, 8
    ik, q = _chunk(P0, T, H, seed=3)
    got = _run_shared(ik, q, P0, K)
    starts = dev(np.zeros(T, np.int64))
    vis = dev((P0 + 1 + np.arange(T)).astype(np.int32))
    full, _, _ = index_topk(csa2.FULL, dev_bf16(q), dev_bf16(ik), starts, vis, P0 + T, K)
    assert np.array_equal(got, full.cpu().numpy())


def test_shared_few_visible_and_ragged_tail():
    """Rows that see fewer than K entries (all of them selected, -1 padded); a row count that is
    not a multiple of the row tile."""
    P0, T, K, H = 100, 203, 256, 8
    ik, q = _chunk(P0, T, H, seed=4)
    idx = _run_shared(ik, q, P0, K)
    _check_rows(idx, ik, q, P0, K, range(T))


def test_shared_ties_and_overflow_fallback():
    """Integer-valued keys give massive exact ties: rows whose candidate list would exceed its
    capacity take the exact full-scan fallback; ties resolve to the lower position."""
    P0, T, K, H = 40000, 24, 300, 8
    rng = np.random.default_rng(5)
    # 2 distinct key rows repeated: scores take 2 values per row -> ~20,000-entry ties, more
    # candidates than a row's list holds
    base = rng.integers(-2, 3, size=(2, 64)).astype(np.float32)
    ik = base[rng.integers(0, 2, size=P0 + T)]
    q = rng.integers(-2, 3, size=(T, H, 64)).astype(np.float32)
    idx = _run_shared(ik, q, P0, K)
    _check_rows(idx, ik, q, P0, K, range(T))


def test_shared_all_zero_scores():
    """Every dot product negative: all scores are +0 and the top-K are the first K positions."""
    P0, T, K, H = 20000, 16, 128, 8
    ik = np.ones((P0 + T, 64), np.float32)
    q = -np.ones((T, H, 64), np.float32)
    idx = _run_shared(ik, q, P0, K)
    assert np.array_equal(idx, np.tile(np.arange(K, dtype=np.int32), (T, 1)))


def test_shared_unrepresentative_sample():
    """Keys of large norm exactly at the positions the provisional bound samples: the sampled
    bound is too high, the exact selection among the candidates does not certify it, and the rows
    take the exact fallback scan."""
    P0, T, K, H = 30000, 40, 512, 8
    rng = np.random.default_rng(6)
    n = P0 + T
    ik = rng.standard_normal((n, 64), dtype=np.float32)
    sampled = ((np.arange(n) // 32) % 16) == 0
    ik[sampled] *= 8.0
    ik = bf16_round(ik)
    q = bf16_round(rng.standard_normal((T, H, 64), dtype=np.float32))
    idx = _run_shared(ik, q, P0, K)
    _check_rows(idx, ik, q, P0, K, range(T))


def test_shared_bound_holds_on_low_norm_sample():
    """The converse: large keys away from the sampled positions (a low sampled bound, many
    candidates, still exact)."""
    P0, T, K, H = 30000, 40, 512, 8
    rng = np.random.default_rng(7)
    n = P0 + T
    ik = rng.standard_normal((n, 64), dtype=np.float32)
    boosted = ((np.arange(n) // 32) % 16) == 5
    ik[boosted] *= 3.0
    ik = bf16_round(ik)
    q = bf16_round(rng.standard_normal((T, H, 64), dtype=np.float32))
    idx = _run_shared(ik, q, P0, K)
    _check_rows(idx, ik, q, P0, K, range(T))


def test_shared_with_pool_equals_full_and_feeds_reindex():
    """CSA2_FULL_SHARED asked for a pool returns exactly what CSA2_FULL returns (indices, pool, pool
    length), and a Reindex layer over that pool matches the oracle ("The hierarchical indexer" in the
    course brief: blocks of 8 ranked by their best member, members rescored by a later layer)."""
    P0, T, H, K, P = 6000, 40, 8, 256, 1024
    ik, q = _chunk(P0, T, H, seed=71)
    q2 = bf16_round(np.random.default_rng(72).standard_normal((T, H, 64), dtype=np.float32))
    n = ik.shape[0]
    starts = dev(np.zeros(T, np.int64))
    vis_np = (P0 + 1 + np.arange(T)).astype(np.int32)
    vis = dev(vis_np)
    kk = dev_bf16(ik)
    i_s, p_s, l_s = index_topk(csa2.FULL_SHARED, dev_bf16(q), kk, starts, vis, n, K, pool_size=P)
    i_f, p_f, l_f = index_topk(csa2.FULL, dev_bf16(q), kk, starts, vis, n, K, pool_size=P)
    torch.cuda.synchronize()
    assert torch.equal(i_s, i_f) and torch.equal(p_s, p_f) and torch.equal(l_s, l_f)
    i_r, _, _ = index_topk(csa2.REINDEX, dev_bf16(q2), kk, starts, vis, n, K, pool=p_s, pool_len=l_s)
    torch.cuda.synchronize()
    idx, pool, plen, ridx = i_s.cpu().numpy(), p_s.cpu().numpy(), l_s.cpu().numpy(), i_r.cpu().numpy()
    for r in range(T):
        sel, opool, olen = oracle.full_select(q[r], ik[:vis_np[r]], int(vis_np[r]), K, P)
        assert np.array_equal(idx[r], sel), "row %d: indices differ" % r
        assert np.array_equal(pool[r], opool) and plen[r] == olen, "row %d: pool differs" % r
        want = oracle.reindex_select(q2[r], ik, opool, int(vis_np[r]), K)
        assert np.array_equal(ridx[r], want), "row %d: Reindex over the shared pool differs" % r
    say("shared segment with pool: %d rows, pool and Reindex exact" % T)
