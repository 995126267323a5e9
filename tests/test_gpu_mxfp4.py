"""GPU parity of the MXFP4 indexer-key path against the CPU oracle.

Bit-exact: the MXFP4 codes and E8M0 scales the quantize call writes, and the
Full / Reindex / shared-segment selections (indices, pools, pool lengths)
over MXFP4 keys, which the oracle takes as its selection over the
dequantized keys.  Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import oracle
from gen import bf16_round
from gpu_util import DEV, as_dtype, dev, dev_bf16, say
from sparse_attention_fp4_e4m3_amd import csa2

pytestmark = pytest.mark.gpu

E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)


def _mx_edge_rows():
    """Blocks whose x / X land exactly on E2M1 midpoints (ties), clamp above 6, zero and
    subnormal-range blocks, negative zero, huge and tiny exponents."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0])
    rows = []
    for k in [-140, -126, -30, 0, 5, 100]:
        r = np.zeros(64)
        r[:8], r[8:16] = mids, -mids
        r[16] = 4.0  # block max 4..8: X = 1 before scaling
        r[32:64] = np.linspace(-7.9, 7.9, 32)
        rows.append(r * 2.0 ** k)
    z = np.zeros(64)
    z[40] = -0.0
    rows.append(z)
    return np.array(rows, dtype=np.float32)


def _mx_cache(k):
    codes = torch.zeros(k.shape[0], 32, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(k.shape[0], 2, dtype=torch.uint8, device=DEV)
    csa2.quantize_idx_mxfp4(dev(k), codes, scales)
    return codes, scales


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_mxfp4_quantize_bit_exact(kind):
    rng = np.random.default_rng(31)
    x = rng.standard_normal((500, 64)).astype(np.float32) * np.exp2(rng.uniform(-30, 30, (500, 1))).astype(np.float32)
    x = np.concatenate([x, _mx_edge_rows()])
    if kind == "bf16":
        x = bf16_round(x)
    n = x.shape[0]
    xs = np.zeros((n, 96), np.float32)
    xs[:, :64] = x
    dst = np.arange(n, dtype=np.int64)[::-1].copy()
    dst[::9] = -1
    codes = torch.full((n, 32), 0xAB, dtype=torch.uint8, device=DEV)
    scales = torch.full((n, 2), 0xAB, dtype=torch.uint8, device=DEV)
    csa2.quantize_idx_mxfp4(as_dtype(xs, kind), codes, scales, dev(dst))
    wc, ws = oracle.mxfp4_quantize(x)
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    for t in range(n):
        if dst[t] >= 0:
            assert np.array_equal(gc[dst[t]], wc[t]) and np.array_equal(gs[dst[t]], ws[t]), "token %d" % t
    skipped = dst[::9]
    assert np.all(gc[n - 1 - np.arange(0, n, 9)] == 0xAB)
    say("mxfp4 quantize %s: %d rows bit-exact (%d skipped)" % (kind, n, len(skipped)))


def _inputs(seed, R, H, lens, kind):
    rng = np.random.default_rng(seed)
    N = int(sum(lens))
    k = rng.standard_normal((N, 64)).astype(np.float32)
    q = rng.standard_normal((R, H, 64)).astype(np.float32)
    if kind == "bf16":
        q = bf16_round(q)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    kc, ks = oracle.mxfp4_quantize(k)
    return q, kc, ks, oracle.mxfp4_dequant(kc, ks), starts


def _run(mode, q, kind, kc, ks, starts, lens, K, pool=None, pool_len=None, pool_size=0, max_visible=None):
    R, H = q.shape[0], q.shape[1]
    maxv = int(max(lens)) if max_visible is None else max_visible
    pool_stride = pool.shape[1] if pool is not None else 0
    ws = torch.empty(max(256, csa2.index_topk_workspace_size(mode, R, H, maxv, pool_stride, K, pool_size)),
                     dtype=torch.uint8, device=DEV)
    idx = torch.empty(R, K, dtype=torch.int32, device=DEV)
    op = torch.empty(R, pool_size, dtype=torch.int32, device=DEV) if pool_size else None
    ol = torch.empty(R, dtype=torch.int32, device=DEV) if pool_size else None
    csa2.index_topk_mxfp4(mode, as_dtype(q, kind), dev(kc), dev(ks), dev(starts), dev(np.array(lens, np.int32)), maxv,
                          K, idx, ws, pool=pool, pool_len=pool_len, pool_size=pool_size, out_pool=op, out_pool_len=ol)
    return idx, op, ol


@pytest.mark.parametrize("kind,H,K,lens,P", [
    ("f32", 4, 256, [4096], 0),
    ("bf16", 8, 512, [20000, 9001, 300, 0, 1], 0),
    ("bf16", 8, 2048, [70000, 33333], 8192),
    ("f32", 3, 64, [3000, 2000], 1024),
])
def test_full_topk_over_mxfp4_keys_bit_exact(kind, H, K, lens, P):
    q, kc, ks, kh, starts = _inputs(H * 10 + K, len(lens), H, lens, kind)
    idx, pool, plen = _run(csa2.FULL, q, kind, kc, ks, starts, lens, K, pool_size=P)
    got = idx.cpu().numpy()
    for r in range(len(lens)):
        sel, wpool, wlen = oracle.full_select(q[r], kh[starts[r]:starts[r] + lens[r]], lens[r], K, P)
        assert np.array_equal(got[r], sel), "row %d" % r
        if P:
            assert np.array_equal(pool[r].cpu().numpy(), wpool) and int(plen[r]) == wlen, "pool row %d" % r


def test_reindex_over_mxfp4_keys_and_shared_segment():
    lens, P, H, K = [30000, 12345, 9000], 2048, 8, 512
    R = len(lens)
    q, kc, ks, kh, starts = _inputs(77, R, H, lens, "bf16")
    q2 = bf16_round(np.random.default_rng(78).standard_normal((R, H, 64)).astype(np.float32))
    _, pool, plen = _run(csa2.FULL, q, "bf16", kc, ks, starts, lens, K, pool_size=P)
    idx2, _, _ = _run(csa2.REINDEX, q2, "bf16", kc, ks, starts, lens, K, pool=pool, pool_len=plen)
    gpool, got = pool.cpu().numpy(), idx2.cpu().numpy()
    for r in range(R):
        want = oracle.reindex_select(q2[r], kh[starts[r]:starts[r] + lens[r]], gpool[r], lens[r], K)
        assert np.array_equal(got[r], want), "reindex row %d" % r
    # a prefill-style chunk: rows share one segment and see a growing prefix
    T, P0 = 96, 5000
    qs = bf16_round(np.random.default_rng(79).standard_normal((T, H, 64)).astype(np.float32))
    vis = [P0 + r + 1 for r in range(T)]
    idx3, _, _ = _run(csa2.FULL_SHARED, qs, "bf16", kc, ks, np.zeros(T, np.int64), vis, K, max_visible=P0 + T)
    got3 = idx3.cpu().numpy()
    for r in [0, 1, 50, T - 1]:
        sel, _, _ = oracle.full_select(qs[r], kh[:vis[r]], vis[r], K)
        assert np.array_equal(got3[r], sel), "shared row %d" % r


@pytest.mark.parametrize("kind,H", [("f32", 4), ("bf16", 16), ("f32", 3)])
def test_reindex_over_mxfp4_keys_query_types_and_head_counts(kind, H):
    lens, P, K = [12000, 5003], 1024, 256
    R = len(lens)
    q, kc, ks, kh, starts = _inputs(300 + H, R, H, lens, kind)
    q2 = np.random.default_rng(301 + H).standard_normal((R, H, 64)).astype(np.float32)
    if kind == "bf16":
        q2 = bf16_round(q2)
    _, pool, plen = _run(csa2.FULL, q, kind, kc, ks, starts, lens, K, pool_size=P)
    idx2, _, _ = _run(csa2.REINDEX, q2, kind, kc, ks, starts, lens, K, pool=pool, pool_len=plen)
    gpool, got = pool.cpu().numpy(), idx2.cpu().numpy()
    for r in range(R):
        want = oracle.reindex_select(q2[r], kh[starts[r]:starts[r] + lens[r]], gpool[r], lens[r], K)
        assert np.array_equal(got[r], want), "row %d" % r
