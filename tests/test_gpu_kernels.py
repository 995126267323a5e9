"""GPU parity of each library call against the CPU oracle, at oracle-sized shapes.

Bit-exact: FP4 codes, E4M3 scales, top-K indices, HSI pools and pool
lengths.  Attention outputs: within 2e-3 max relative error per row and
head (normwise), lse within 1e-3.  Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from gen import bf16_round
from gpu_util import DEV, as_dtype, attention, check_attention, dev, dev_bf16, index_topk, quantize, say
from sparse_attention_fp4_e4m3_amd import csa2

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- quantize

def _edge_rows():
    """Rows exercising every scale code, element ties, zero groups, signs."""
    rows = []
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    # every finite non-negative E4M3 scale value as amax/6 (groups with amax = 6*s)
    svals = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    for base in range(0, len(svals), 32):
        r = np.zeros(512)
        for g in range(32):
            s = svals[min(base + g, len(svals) - 1)]
            el = grid[np.arange(16) % 8] * np.where(np.arange(16) % 3 == 0, -1, 1) * s
            el[5] = 6 * s
            r[16 * g:16 * g + 16] = el
        rows.append(r)
    # element ties: x/s exactly at E2M1 midpoints for s = 1 (amax = 6)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    r = np.tile(np.concatenate([mids, -mids]), 32)
    rows.append(r)
    # zero group, tiny group (scale 0), negative tiny values, huge values (saturating scale)
    r = np.zeros(512)
    r[16:32] = -1e-4
    r[32:48] = 1e3
    r[48:64] = np.linspace(-3000, 3000, 16)
    r[64:80] = -0.0
    r[80:96] = 2.0 ** -10 * 6  # amax/6 exactly at the 0 / 2^-9 midpoint
    r[96:112] = 3 * 2.0 ** -10 * 6
    rows.append(r)
    return np.array(rows, dtype=np.float32)


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_quantize_bit_exact(kind):
    rng = np.random.default_rng(10)
    x = rng.standard_normal((3000, 512)).astype(np.float32)
    x[:, [7, 99, 200, 301, 444]] *= 20
    x[::7] *= rng.uniform(1e-3, 50, (len(x[::7]), 1)).astype(np.float32)
    x = np.concatenate([x, _edge_rows()])
    if kind == "bf16":
        x = bf16_round(x)
    codes, scales = quantize(as_dtype(x, kind))
    oc, os_ = oracle.quantize(x)
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    bad = np.nonzero((gc != oc).any(1) | (gs != os_).any(1))[0]
    assert bad.size == 0, "rows differ: %s" % bad[:10]


def test_quantize_dst_rows_and_strided_input():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((100, 640)).astype(np.float32)  # row stride 640, first 512 used
    dst = rng.permutation(300)[:100].astype(np.int64)
    dst[3] = -1  # skipped
    dst[4] = 5000  # out of range, skipped
    codes = torch.full((300, 256), 0xAB, dtype=torch.uint8, device=DEV)
    scales = torch.full((300, 32), 0xCD, dtype=torch.uint8, device=DEV)
    csa2.quantize_kv_fp4(dev(x), codes, scales, dev(dst))
    oc, os_ = oracle.quantize(x[:, :512])
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    ok = (dst >= 0) & (dst < 300)
    assert np.array_equal(gc[dst[ok]], oc[ok]) and np.array_equal(gs[dst[ok]], os_[ok])
    untouched = np.setdiff1d(np.arange(300), dst[ok])
    assert np.all(gc[untouched] == 0xAB) and np.all(gs[untouched] == 0xCD)


def test_dequant_exact_through_single_entry_attention():
    """Selecting one entry returns exactly its dequantized value (every code and scale byte)."""
    rng = np.random.default_rng(12)
    x = np.concatenate([_edge_rows(), rng.standard_normal((40, 512)).astype(np.float32) * 3])
    codes, scales = quantize(dev(x))
    n = x.shape[0]
    oc, os_ = oracle.quantize(x)
    xh = oracle.dequant(oc, os_)
    q = dev(rng.standard_normal((n, 16, 512)).astype(np.float32))
    starts = torch.zeros(n, dtype=torch.int64, device=DEV)
    idx = torch.full((n, 4), -1, dtype=torch.int32, device=DEV)
    idx[:, 1] = torch.arange(n, dtype=torch.int32, device=DEV)
    out, lse = attention(q, codes, scales, starts, idx, 0.05)
    o = out.cpu().numpy()
    assert np.array_equal(o, np.broadcast_to(xh[:, None, :].astype(np.float32), o.shape))


# ---------------------------------------------------------------- indexer

def _idx_inputs(seed, R, H, lens, kind, integer=False):
    rng = np.random.default_rng(seed)
    N = int(sum(lens))
    if integer:
        k = rng.integers(-4, 5, (N, 64)).astype(np.float32)
        q = rng.integers(-3, 4, (R, H, 64)).astype(np.float32)
    else:
        k = rng.standard_normal((N, 64)).astype(np.float32)
        q = rng.standard_normal((R, H, 64)).astype(np.float32)
    if kind == "bf16":
        k, q = bf16_round(k), bf16_round(q)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    return q, k, starts


def _oracle_full(q, k, starts, lens, K, P=0):
    idx, pools, plens = [], [], []
    for r in range(len(lens)):
        kr = k[starts[r]:starts[r] + lens[r]]
        sel, pool, pl = oracle.full_select(q[r], kr, lens[r], K, P)
        idx.append(sel)
        if P:
            pools.append(pool)
            plens.append(pl)
    return np.array(idx), (np.array(pools) if P else None), (np.array(plens) if P else None)


@pytest.mark.parametrize("kind,H,K,lens,integer", [
    ("f32", 4, 256, [4096], False),                         # the tiny decode shape
    ("bf16", 8, 512, [20000, 9001, 4097, 300, 0, 1], False),  # ragged rows, empty row, K > n
    ("bf16", 8, 2048, [70000, 33333], False),
    ("bf16", 8, 200, [12000, 5000], True),                  # integer scores: heavy ties
    ("f32", 3, 64, [3000, 2000], False),                    # runtime head count
])
def test_full_topk_bit_exact(kind, H, K, lens, integer):
    R = len(lens)
    q, k, starts = _idx_inputs(sum(lens) + H, R, H, lens, kind, integer)
    maxv = max(lens)
    idx, _, _ = index_topk(csa2.FULL, as_dtype(q, kind), as_dtype(k, kind), dev(starts),
                           dev(np.array(lens, np.int32)), maxv, K)
    want, _, _ = _oracle_full(q, k, starts, lens, K)
    got = idx.cpu().numpy()
    for r in range(R):
        assert np.array_equal(got[r], want[r]), "row %d differs" % r


@pytest.mark.parametrize("lens,P", [([20000, 8191, 100], 1024), ([65536, 40003], 8192), ([3000], 4096)])
def test_full_pool_bit_exact(lens, P):
    R, H, K = len(lens), 8, 256
    q, k, starts = _idx_inputs(P, R, H, lens, "bf16")
    idx, pool, plen = index_topk(csa2.FULL, dev_bf16(q), dev_bf16(k), dev(starts), dev(np.array(lens, np.int32)),
                                 max(lens), K, pool_size=P)
    want, wpool, wlen = _oracle_full(q, k, starts, lens, K, P)
    assert np.array_equal(idx.cpu().numpy(), want)
    assert np.array_equal(plen.cpu().numpy(), wlen)
    assert np.array_equal(pool.cpu().numpy(), wpool)


def test_pool_ties_between_blocks():
    lens, P, H, K = [10003, 777], 512, 8, 64
    q, k, starts = _idx_inputs(5, 2, H, lens, "bf16", integer=True)
    idx, pool, plen = index_topk(csa2.FULL, dev_bf16(q), dev_bf16(k), dev(starts), dev(np.array(lens, np.int32)),
                                 max(lens), K, pool_size=P)
    want, wpool, wlen = _oracle_full(q, k, starts, lens, K, P)
    assert np.array_equal(idx.cpu().numpy(), want)
    assert np.array_equal(plen.cpu().numpy(), wlen) and np.array_equal(pool.cpu().numpy(), wpool)


def test_reindex_bit_exact_and_all_positions_equals_full():
    lens, P, H, K = [30000, 12345, 9000], 2048, 8, 512
    R = len(lens)
    q, k, starts = _idx_inputs(77, R, H, lens, "bf16")
    q2 = bf16_round(np.random.default_rng(78).standard_normal((R, H, 64)).astype(np.float32))
    vis = dev(np.array(lens, np.int32))
    _, pool, plen = index_topk(csa2.FULL, dev_bf16(q), dev_bf16(k), dev(starts), vis, max(lens), K, pool_size=P)
    idx2, _, _ = index_topk(csa2.REINDEX, dev_bf16(q2), dev_bf16(k), dev(starts), vis, max(lens), K, pool=pool,
                            pool_len=plen)
    gpool = pool.cpu().numpy()
    got = idx2.cpu().numpy()
    for r in range(R):
        kr = k[starts[r]:starts[r] + lens[r]]
        want = oracle.reindex_select(q2[r], kr, gpool[r], lens[r], K)
        assert np.array_equal(got[r], want), "row %d" % r
    # Reindex over a pool listing every position (then -1 padding) equals Full
    width = max(lens) + 37
    allpos = np.full((R, width), -1, np.int32)
    for r in range(R):
        allpos[r, :lens[r]] = np.arange(lens[r])
    full_idx, _, _ = index_topk(csa2.FULL, dev_bf16(q2), dev_bf16(k), dev(starts), vis, max(lens), K)
    re_idx, _, _ = index_topk(csa2.REINDEX, dev_bf16(q2), dev_bf16(k), dev(starts), vis, max(lens), K,
                              pool=dev(allpos), pool_len=None)
    assert torch.equal(full_idx, re_idx)


def test_selection_massive_ties_and_partly_filled_pools():
    """All-zero queries tie every entry at score 0, so the threshold bin holds whole rows (more
    candidates than a selection workgroup keeps on chip): the K lowest positions must come out.
    Reindex pools are filled to different lengths, with valid-looking positions past each length
    that must be ignored."""
    lens, H, K = [40000, 20001, 3], 8, 2048
    R = len(lens)
    q, k, starts = _idx_inputs(11, R, H, lens, "bf16")
    q[:] = 0.0
    vis = dev(np.array(lens, np.int32))
    idx, _, _ = index_topk(csa2.FULL, dev_bf16(q), dev_bf16(k), dev(starts), vis, max(lens), K)
    want, _, _ = _oracle_full(q, k, starts, lens, K)
    assert np.array_equal(idx.cpu().numpy(), want)
    # Reindex: stride 6000, lengths 5000 / 1 / 0; slots past the length hold positions that would win
    rng = np.random.default_rng(12)
    q2 = bf16_round(rng.standard_normal((R, H, 64)).astype(np.float32))
    stride, plens = 6000, [5000, 1, 0]
    gpu_pool = np.zeros((R, stride), np.int32)
    ref_pool = np.full((R, stride), -1, np.int32)
    for r in range(R):
        kr = k[starts[r]:starts[r] + lens[r]]
        sc = oracle.index_scores(q2[r], kr)
        order = np.argsort(-sc, kind="stable")
        m = min(plens[r], lens[r])
        chosen = np.sort(order[len(order) - m:]) if m else np.zeros(0, np.int64)  # the lowest-scoring entries
        ref_pool[r, :m] = chosen
        gpu_pool[r, :m] = chosen
        gpu_pool[r, m:] = order[:stride - m] if len(order) >= stride - m else np.resize(order, stride - m)
    idx2, _, _ = index_topk(csa2.REINDEX, dev_bf16(q2), dev_bf16(k), dev(starts), vis, max(lens), K,
                            pool=dev(gpu_pool), pool_len=dev(np.array(plens, np.int32)))
    got = idx2.cpu().numpy()
    for r in range(R):
        kr = k[starts[r]:starts[r] + lens[r]]
        assert np.array_equal(got[r], oracle.reindex_select(q2[r], kr, ref_pool[r], lens[r], K)), "row %d" % r


def test_topk_deterministic():
    lens, H, K = [50000, 50000], 8, 2048
    q, k, starts = _idx_inputs(9, 2, H, lens, "bf16")
    args = (csa2.FULL, dev_bf16(q), dev_bf16(k), dev(starts), dev(np.array(lens, np.int32)), max(lens), K)
    a = index_topk(*args, pool_size=4096)
    b = index_topk(*args, pool_size=4096)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ---------------------------------------------------------------- attention

def _cache(seed, n, outliers=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 512)).astype(np.float32)
    if outliers:
        x[:, [1, 64, 130, 257, 400]] *= 20
    return x


@pytest.mark.parametrize("Hq,qkind,R,K,n", [
    (16, "f32", 1, 256, 4096),     # the tiny decode shape
    (64, "bf16", 3, 2048, 9000),   # several splits
    (64, "bf16", 16, 2048, 9000),  # pipelined 16-head workgroups, four steps per split
    (64, "bf16", 32, 2048, 9000),  # pipelined 32-head workgroups, four steps per split
    (64, "bf16", 24, 1500, 6000),  # pipelined 32-head workgroups, ragged last split
    (64, "bf16", 40, 300, 5000),   # many rows, one split each, ragged step
    (32, "bf16", 5, 1000, 7000),
    (48, "bf16", 2, 700, 3000),
    (128, "bf16", 2, 512, 3000),   # two head groups
    (32, "f32", 3, 640, 3000),
    (64, "bf16", 256, 300, 5000),  # rows alone fill the chip: 64-head workgroups, ragged step
    (128, "bf16", 160, 200, 3000),  # 64-head workgroups, two per row
])
def test_attention_matches_oracle(Hq, qkind, R, K, n):
    rng = np.random.default_rng(Hq * 1000 + K)
    x = _cache(K, n, outliers=True)
    oc, os_ = oracle.quantize(x)
    codes, scales = dev(oc), dev(os_)
    q = rng.standard_normal((R, Hq, 512)).astype(np.float32) * (1 / np.sqrt(512) if qkind == "f32" else 1)
    if qkind == "bf16":
        q = bf16_round(q)
    vis = rng.integers(n // 2, n + 1, R).astype(np.int32)
    idx = np.stack([rng.permutation(n)[:K] for _ in range(R)]).astype(np.int32)  # some >= visible
    idx[:, ::17] = -1
    starts = np.zeros(R, np.int64)
    scale = 1 / np.sqrt(512)
    out, lse = attention(as_dtype(q, qkind), codes, scales, dev(starts), dev(idx), scale, vis=dev(vis))
    ro, rl = oracle.attention_rows(q, oc, os_, starts, idx, vis.astype(np.int64), scale)
    check_attention(out, lse, ro, rl, "attn Hq=%d %s R=%d K=%d" % (Hq, qkind, R, K))


@pytest.mark.parametrize("R", [4, 256])  # 256 rows: 64-head workgroups
def test_attention_all_selected_equals_dense_and_edge_rows(R):
    n, Hq = 700, 64
    rng = np.random.default_rng(3)
    x = _cache(3, n)
    oc, os_ = oracle.quantize(x)
    q = bf16_round(rng.standard_normal((R, Hq, 512)).astype(np.float32))
    K = 1024  # K >= n: dense attention over every entry
    idx = np.full((R, K), -1, np.int32)
    idx[0, :n] = np.arange(n)
    idx[1, :n] = rng.permutation(n)
    idx[2, :] = -1  # empty selection: zeros and -inf
    idx[3, 5] = 17  # a single entry
    for r in range(4, R):
        idx[r, :300] = rng.permutation(n)[:300]
    out, lse = attention(dev_bf16(q), dev(oc), dev(os_), dev(np.zeros(R, np.int64)), dev(idx), 0.0441941738,
                         vis=dev(np.full(R, n, np.int32)))
    ro, rl = oracle.attention_rows(q, oc, os_, np.zeros(R, np.int64), idx, np.full(R, n), 0.0441941738)
    check_attention(out, lse, ro, rl, "dense/edge rows")
    o = out.cpu().numpy()
    assert np.all(o[2] == 0) and np.all(np.isneginf(lse.cpu().numpy()[2]))
    xh = oracle.dequant(oc, os_)
    assert np.array_equal(o[3], np.broadcast_to(xh[17].astype(np.float32), o[3].shape))


@pytest.mark.parametrize("Hq,qkind,R", [(64, "bf16", 4), (16, "f32", 2)])
def test_attention_error_bound_under_cancellation(Hq, qkind, R):
    """Entries in +/- pairs with nearly equal logits: the output is a small difference of large values
    (max|o| well below max|x_hat|), where a relative bound on max|o| would not follow from the
    arithmetic.  What does follow: probabilities rounded to fp16 (2^-11 relative, the row sum adds the
    same rounded values) move the normalized weights by at most about 2^-10 of themselves, and split
    partials stored in fp16 add 2^-11 of their size, so |o - o_exact| <= (2^-10 + 2^-11) max |x_hat|
    per channel over the selected entries; checked here with 2e-3."""
    rng = np.random.default_rng(60 + Hq)
    half = 512
    x = rng.standard_normal((half, 512)).astype(np.float32)
    x = np.concatenate([x, -x])  # quantization is sign-symmetric: the pairs dequantize to exact negatives
    oc, os_ = oracle.quantize(x)
    xh = oracle.dequant(oc, os_)
    assert np.array_equal(xh[half:], -xh[:half])
    n = x.shape[0]
    q = rng.standard_normal((R, Hq, 512)).astype(np.float32) * 2e-4
    if qkind == "bf16":
        q = bf16_round(q)
    idx = np.stack([rng.permutation(n) for _ in range(R)]).astype(np.int32)
    starts = np.zeros(R, np.int64)
    out, lse = attention(as_dtype(q, qkind), dev(oc), dev(os_), dev(starts), dev(idx), 0.0441941738)
    ro, rl = oracle.attention_rows(q, oc, os_, starts, idx, np.full(R, n, np.int64), 0.0441941738)
    o = out.cpu().numpy().astype(np.float64)
    xmax = np.abs(xh).max()
    assert np.abs(ro).max() < 0.05 * xmax  # heavy cancellation in the reference itself
    err = np.abs(o - ro).max()
    say("cancellation Hq=%d %s: max|o_ref| %.3g, max|x_hat| %.3g, max abs err %.3g (%.2e of max|x_hat|)"
        % (Hq, qkind, np.abs(ro).max(), xmax, err, err / xmax))
    assert err <= 2e-3 * xmax
    assert np.abs(lse.cpu().numpy() - rl).max() <= 1e-3


@pytest.mark.parametrize("R,Hq,exps", [
    # decode kernel (16 rows x 64 heads): each head's queries are scaled by a power of two into fp16,
    # so heads far below and above the fp16 range are used exactly
    (16, 64, (-40, -24, -14, -3, 0, 3, 20, 60)),
    # 64-head kernel (256 rows): bf16 converts to fp16 unscaled, exact for 2^-14 <= |q| < 65520
    (256, 64, (-12, -6, -3, 0, 2, 4, 6, 8)),
])
def test_attention_bf16_query_magnitudes(R, Hq, exps):
    """Heads whose bf16 queries sit at very different magnitudes (head h scaled by 2^exps[h % 8],
    the softmax scale chosen so that the largest logits stay near 10): outputs and lse against the
    oracle, which works on the exact bf16 values."""
    n, K = 3000, 512
    rng = np.random.default_rng(91 + R)
    x = _cache(91, n)
    oc, os_ = oracle.quantize(x)
    q = rng.standard_normal((R, Hq, 512)).astype(np.float32)
    e = np.array([exps[h % len(exps)] for h in range(Hq)], np.float64)
    q = bf16_round((q * np.exp2(e)[None, :, None]).astype(np.float32))
    idx = np.stack([rng.permutation(n)[:K] for _ in range(R)]).astype(np.int32)
    starts = np.zeros(R, np.int64)
    # one softmax scale per call: the heads' logits differ by their magnitude, which is the point
    scale = float(2.0 ** -(max(exps) + 4))
    out, lse = attention(dev_bf16(q), dev(oc), dev(os_), dev(starts), dev(idx), scale)
    ro, rl = oracle.attention_rows(q, oc, os_, starts, idx, np.full(R, n, np.int64), scale)
    assert np.all(np.isfinite(out.cpu().numpy()))
    check_attention(out, lse, ro, rl, "bf16 query magnitudes R=%d exps=%s" % (R, exps))


def test_attention_split_merge_shares_one_workspace():
    """Split launches hand their partials to merge workgroups through counters at the start of the
    workspace: one zero-filled workspace serves calls of several shapes in a row (the merge inside the
    launch for 8k (row, 32-head) pairs, a separate merge launch otherwise), each call matches the
    oracle and leaves the counters zero."""
    n = 6000
    rng = np.random.default_rng(12)
    x = _cache(12, n)
    oc, os_ = oracle.quantize(x)
    codes, scales = dev(oc), dev(os_)
    shapes = [(16, 64, 2048), (32, 64, 2048), (3, 64, 2048), (4, 64, 1024), (16, 64, 2048)]
    need = max(csa2.sparse_attn_workspace_size(R, Hq, csa2.BF16, K) for R, Hq, K in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for i, (R, Hq, K) in enumerate(shapes):
        q = bf16_round(rng.standard_normal((R, Hq, 512)).astype(np.float32))
        idx = np.stack([rng.permutation(n)[:K] for _ in range(R)]).astype(np.int32)
        starts = np.zeros(R, np.int64)
        out = torch.empty(R, Hq, 512, dtype=torch.float32, device=DEV)
        lse = torch.empty(R, Hq, dtype=torch.float32, device=DEV)
        csa2.sparse_attn(dev_bf16(q), codes, scales, dev(starts), dev(idx), out, 0.0441941738, lse=lse, workspace=ws)
        ro, rl = oracle.attention_rows(q, oc, os_, starts, idx, np.full(R, n, np.int64), 0.0441941738)
        check_attention(out, lse, ro, rl, "shared workspace call %d R=%d K=%d" % (i, R, K))
        assert int(ws[:4096].count_nonzero()) == 0, "call %d left split-merge counters set" % i


def test_attention_deterministic_and_bf16_output():
    n, R, Hq, K = 20000, 16, 64, 2048
    rng = np.random.default_rng(4)
    x = _cache(4, n)
    codes, scales = quantize(dev(x))
    q = dev_bf16(bf16_round(rng.standard_normal((R, Hq, 512)).astype(np.float32)))
    idx = dev(np.stack([np.sort(rng.permutation(n)[:K]) for _ in range(R)]).astype(np.int32))
    starts = dev(np.zeros(R, np.int64))
    a, la = attention(q, codes, scales, starts, idx, 0.044)
    b, lb = attention(q, codes, scales, starts, idx, 0.044)
    assert torch.equal(a, b) and torch.equal(la, lb), "attention is not bitwise reproducible"
    c, _ = attention(q, codes, scales, starts, idx, 0.044, out_dtype=torch.bfloat16)
    assert torch.equal(c, a.to(torch.bfloat16))
