"""GPU parity of whole layer-mode chains (Full -> Reindex -> Reuse) against the
CPU oracle at oracle-sized shapes drawn from the workload generators, and
HIP-graph replay of a chain step against eager execution."""
import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import DEV, check_attention, dev, say
from sparse_attention_fp4_e4m3_amd import Cache, LayerChain, LayerSpec, Window, csa2

pytestmark = pytest.mark.gpu


def _to_dev(a, kind):
    if kind == "bf16":
        return torch.from_numpy(gen.bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


def _setup(w):
    return _setup_lens(w, gen.seq_lens(w))


def _setup_lens(w, lens):
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    raw = [gen.kv_rows(w, b, 0, int(lens[b])) for b in range(w.B)]
    ik = [gen.idx_k_rows(w, b, 0, int(lens[b])) for b in range(w.B)]
    x = np.concatenate(raw)
    codes = torch.empty(len(x), 256, dtype=torch.uint8, device=DEV)
    scales = torch.empty(len(x), 32, dtype=torch.uint8, device=DEV)
    csa2.quantize_kv_fp4(torch.from_numpy(x).to(DEV), codes, scales)
    cache = Cache(codes, scales, _to_dev(np.concatenate(ik), w.idx_dtype), dev(starts),
                  dev(lens.astype(np.int32)), int(lens.max()))
    qs = [_to_dev(gen.attn_q(w, li), w.q_dtype) for li in range(len(w.layers))]
    iqs = [_to_dev(gen.index_q(w, li), w.idx_dtype) if L.mode != "reuse" else None for li, L in enumerate(w.layers)]
    return lens, starts, raw, ik, cache, qs, iqs


def _oracle_chain(w, lens, raw, ik, b):
    """The oracle's own quantization, selections and attention for sequence b."""
    oc, os_ = oracle.quantize(raw[b])
    n = int(lens[b])
    res = []
    pool = sel = None
    for li, L in enumerate(w.layers):
        q = gen.attn_q(w, li, b, b + 1)[0]
        if L.mode == "full":
            sel, pool, plen = oracle.full_select(gen.index_q(w, li, b, b + 1)[0], ik[b], n, w.K, L.pool_size)
        elif L.mode == "reindex":
            sel = oracle.reindex_select(gen.index_q(w, li, b, b + 1)[0], ik[b], pool, n, w.K)
        o, lse = oracle.attention(q, oc, os_, sel, n, w.softmax_scale)
        res.append((sel.copy(), None if pool is None else pool.copy(), o, lse))
    return oc, os_, res


def _run_and_compare(w, rows=None):
    lens, starts, raw, ik, cache, qs, iqs = _setup(w)
    chain = LayerChain([LayerSpec(L.mode, L.pool_size) for L in w.layers], w.B, w.Hq, w.H, w.K, cache.max_visible,
                       qs[0].dtype, DEV)
    chain.step(cache, qs, iqs, w.softmax_scale)
    torch.cuda.synchronize()
    gcodes, gscales = cache.kv_codes.cpu().numpy(), cache.kv_scales.cpu().numpy()
    rows = range(w.B) if rows is None else rows
    worst = 0.0
    for b in rows:
        oc, os_, ref = _oracle_chain(w, lens, raw, ik, b)
        s0, n = int(starts[b]), int(lens[b])
        assert np.array_equal(gcodes[s0:s0 + n], oc) and np.array_equal(gscales[s0:s0 + n], os_), "codes, seq %d" % b
        for li, (sel, pool, o, lse) in enumerate(ref):
            L = w.layers[li]
            if L.mode != "reuse":
                assert np.array_equal(chain.idx[li][b].cpu().numpy(), sel), "indices, layer %d seq %d" % (li, b)
            if L.mode == "full" and L.pool_size:
                gp, gl = chain.pool[li]
                assert np.array_equal(gp[b].cpu().numpy(), pool), "pool, seq %d" % b
            worst = max(worst, check_attention(chain.out[li][b:b + 1], chain.lse[li][b:b + 1], o[None], lse[None],
                                               "%s layer %d (%s) seq %d" % (w.name, li, L.mode, b)))
    return worst


def test_tiny_decode_full_at_workload_size():
    """The tiny decode workload at its own size: B=1, n=4096, fp32, K=256."""
    say("max err %.3e" % _run_and_compare(gen.get("c1")))


def test_layer_chain_128k_structure_scaled():
    """Full (pool) -> 2 x Reindex -> 3 x Reuse, the 128K chain's structure at oracle size."""
    w = gen.get("c3").scaled(B=3, n=24001, K=512, layers=(gen.Layer("full", 2048), gen.Layer("reindex"),
                                                         gen.Layer("reindex"), gen.Layer("reuse"),
                                                         gen.Layer("reuse"), gen.Layer("reuse")))
    say("max err %.3e" % _run_and_compare(w))


def test_decode_ragged_outliers_scaled():
    """Variable lengths and x20 outlier channels, Full mode, at oracle size."""
    w = gen.get("c2").scaled(B=6, n=20000, len_range=(7000, 20000), K=1024)
    say("max err %.3e" % _run_and_compare(w))


def test_long_decode_drift_scaled():
    """Drifting keys, Full (pool) -> Reindex -> Reuse, at oracle size."""
    w = gen.get("c5").scaled(B=2, n=65536, K=1024, layers=(gen.Layer("full", 4096), gen.Layer("reindex"),
                                                          gen.Layer("reuse")))
    say("max err %.3e" % _run_and_compare(w))


def _windows(w, lens):
    """Each layer's ring of 128 window rows per sequence (row = position mod 128) holding the
    sequence's last min(n, 128) tokens, written by the FP8 quantize call; plus the newest
    token of every sequence per layer and its ring row (what a decode step writes)."""
    wins, new = [], []
    B = w.B
    new_rows = dev(np.array([b * 128 + (int(lens[b]) - 1) % 128 for b in range(B)], np.int64))
    for li in range(len(w.layers)):
        codes = torch.zeros(B * 128, 512, dtype=torch.uint8, device=DEV)
        for b in range(B):
            n = int(lens[b])
            t0 = max(0, n - 128)
            dst = dev(np.array([b * 128 + t % 128 for t in range(t0, n)], np.int64))
            csa2.quantize_swa_fp8(torch.from_numpy(gen.window_rows(w, li, b, t0, n)).to(DEV), codes, dst)
        wins.append(Window(codes, dev(np.arange(B, dtype=np.int64) * 128), dev(np.minimum(lens, 128).astype(np.int32))))
        new.append(torch.from_numpy(np.concatenate([gen.window_rows(w, li, b, int(lens[b]) - 1, int(lens[b]))
                                                    for b in range(B)])).to(DEV))
    return wins, new, new_rows


def test_chain_with_local_windows_scaled():
    """Every layer of the 128K chain's structure joined with its own FP8 window, at oracle size,
    one layer's window shorter than 128 (a sequence of 100 tokens)."""
    w = gen.get("c3").scaled(B=3, n=24001, K=512, layers=(gen.Layer("full", 2048), gen.Layer("reindex"),
                                                         gen.Layer("reuse")), len_range=(100, 24001))
    lens = gen.seq_lens(w)
    lens[0] = 100  # first sequence: a window of 100 tokens
    lens, starts, raw, ik, cache, qs, iqs = _setup_lens(w, lens)
    wins, new_win, new_win_rows = _windows(w, lens)
    chain = LayerChain([LayerSpec(L.mode, L.pool_size) for L in w.layers], w.B, w.Hq, w.H, w.K, cache.max_visible,
                       qs[0].dtype, DEV, swa=True)
    chain.step(cache, qs, iqs, w.softmax_scale, windows=wins, new_win=new_win, new_win_rows=new_win_rows)
    torch.cuda.synchronize()
    worst = 0.0
    for b in range(w.B):
        oc, os_, ref = _oracle_chain(w, lens, raw, ik, b)
        n = int(lens[b])
        for li, (sel, pool, o, lse) in enumerate(ref):
            wc = oracle.e4m3_encode_signed(gen.window_rows(w, li, b, max(0, n - 128), n))
            ring = wins[li].codes[b * 128:b * 128 + 128].cpu().numpy()
            assert np.array_equal(ring[[t % 128 for t in range(max(0, n - 128), n)]], wc), "window codes"
            z = np.zeros(1, np.int64)
            o2, lse2 = oracle.attention_rows_swa(gen.attn_q(w, li, b, b + 1), oc, os_, z, sel[None], np.array([n]),
                                                 wc, z, np.array([len(wc)], np.int32), w.softmax_scale)
            worst = max(worst, check_attention(chain.out[li][b:b + 1], chain.lse[li][b:b + 1], o2, lse2,
                                               "swa chain layer %d seq %d" % (li, b)))
    say("max err %.3e" % worst)


def test_verification_rows_scaled():
    """Checking 5 draft tokens per sequence in one pass (the 5-row verification workload at oracle
    size): rows (b, 0..4) share sequence b's cache and see it up to their own draft; the step
    writes the drafts' KV first."""
    w = gen.get("c3v").scaled(B=2, n=20000, K=512, layers=(gen.Layer("full", 2048), gen.Layer("reindex"),
                                                           gen.Layer("reuse")))
    V = w.verify
    lens, starts, raw, ik, cache, qs, iqs = _setup(w)
    cache.row_kv_start = dev(np.repeat(starts, V).astype(np.int64))
    vis = np.concatenate([lens[b] - V + 1 + np.arange(V) for b in range(w.B)]).astype(np.int32)
    cache.row_visible = dev(vis)
    chain = LayerChain([LayerSpec(L.mode, L.pool_size) for L in w.layers], w.rows, w.Hq, w.H, w.K, cache.max_visible,
                       qs[0].dtype, DEV)
    new_rows = dev(np.concatenate([starts[b] + np.arange(lens[b] - V, lens[b]) for b in range(w.B)]).astype(np.int64))
    new_kv = torch.from_numpy(np.concatenate([r[-V:] for r in raw])).to(DEV)
    chain.step(cache, qs, iqs, w.softmax_scale, new_kv=new_kv, new_kv_rows=new_rows)
    torch.cuda.synchronize()
    worst = 0.0
    for b in range(w.B):
        oc, os_ = oracle.quantize(raw[b])
        for i in range(V):
            r, n = b * V + i, int(vis[b * V + i])
            pool = sel = None
            for li, L in enumerate(w.layers):
                if L.mode == "full":
                    sel, pool, _ = oracle.full_select(gen.index_q(w, li, r, r + 1)[0], ik[b], n, w.K, L.pool_size)
                elif L.mode == "reindex":
                    sel = oracle.reindex_select(gen.index_q(w, li, r, r + 1)[0], ik[b], pool, n, w.K)
                if L.mode != "reuse":
                    assert np.array_equal(chain.idx[li][r].cpu().numpy(), sel), "indices, layer %d row %d" % (li, r)
                o, lse = oracle.attention(gen.attn_q(w, li, r, r + 1)[0], oc, os_, sel, n, w.softmax_scale)
                worst = max(worst, check_attention(chain.out[li][r:r + 1], chain.lse[li][r:r + 1], o[None],
                                                   lse[None], "verify layer %d row %d" % (li, r)))
    say("max err %.3e" % worst)


def test_chain_with_mxfp4_indexer_keys_scaled():
    """The 128K chain's structure with MXFP4 indexer keys written by the library: every selection
    equals the oracle's over the dequantized keys."""
    w = gen.get("c3").scaled(B=3, n=24001, K=512, layers=(gen.Layer("full", 2048), gen.Layer("reindex"),
                                                         gen.Layer("reindex"), gen.Layer("reuse")))
    lens, starts, raw, ik, cache, qs, iqs = _setup(w)
    kc = torch.empty(cache.idx_k.shape[0], 32, dtype=torch.uint8, device=DEV)
    ks = torch.empty(cache.idx_k.shape[0], 2, dtype=torch.uint8, device=DEV)
    csa2.quantize_idx_mxfp4(cache.idx_k, kc, ks)
    mx = Cache(cache.kv_codes, cache.kv_scales, kc, cache.row_kv_start, cache.row_visible, cache.max_visible,
               idx_k_scales=ks)
    chain = LayerChain([LayerSpec(L.mode, L.pool_size) for L in w.layers], w.B, w.Hq, w.H, w.K, mx.max_visible,
                       qs[0].dtype, DEV)
    chain.step(mx, qs, iqs, w.softmax_scale)
    torch.cuda.synchronize()
    ikh = [oracle.mxfp4_dequant(*oracle.mxfp4_quantize(k)) for k in ik]
    worst = 0.0
    for b in range(w.B):
        oc, os_, ref = _oracle_chain(w, lens, raw, ikh, b)
        for li, (sel, pool, o, lse) in enumerate(ref):
            if w.layers[li].mode != "reuse":
                assert np.array_equal(chain.idx[li][b].cpu().numpy(), sel), "indices, layer %d seq %d" % (li, b)
            worst = max(worst, check_attention(chain.out[li][b:b + 1], chain.lse[li][b:b + 1], o[None], lse[None],
                                               "mxfp4 chain layer %d seq %d" % (li, b)))
    say("max err %.3e" % worst)


@pytest.mark.parametrize("swa", [False, True])
def test_graph_replay_matches_eager(swa):
    w = gen.get("c3").scaled(B=4, n=30000, K=512, layers=(gen.Layer("full", 2048), gen.Layer("reindex"),
                                                         gen.Layer("reuse")))
    lens, starts, raw, ik, cache, qs, iqs = _setup(w)
    chain = LayerChain([LayerSpec(L.mode, L.pool_size) for L in w.layers], w.B, w.Hq, w.H, w.K, cache.max_visible,
                       qs[0].dtype, DEV, swa=swa)
    new_rows = dev((starts + lens - 1).astype(np.int64))
    new_kv = torch.from_numpy(np.stack([r[-1] for r in raw])).to(DEV)
    wins = new_win = new_win_rows = None
    if swa:
        wins, new_win, new_win_rows = _windows(w, lens)

    def step():
        chain.step(cache, qs, iqs, w.softmax_scale, new_kv=new_kv, new_kv_rows=new_rows, windows=wins,
                   new_win=new_win, new_win_rows=new_win_rows)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in chain.out + chain.lse + [i for i in chain.idx if i is not None]]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in chain.out + chain.lse:
            t.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = chain.out + chain.lse + [i for i in chain.idx if i is not None]
        for a, b in zip(got, eager):
            assert torch.equal(a, b), "replay %d differs from eager" % rep


def test_compressed_entries_visibility_in_a_chunk():
    """Encoder-style entries that fold m = 2 tokens: chunk token t (rows of one shared segment) may
    attend only complete blocks, row_visible = (t + 1) // 2.  Selection and attention against the
    oracle at those visible counts."""
    from sparse_attention_fp4_e4m3_amd import compressed_visible
    T, P0, H, Hq, K = 64, 8001, 8, 64, 256
    nc = (P0 + T) // 2
    rng = np.random.default_rng(41)
    x = rng.standard_normal((nc, 512)).astype(np.float32)
    k = gen.bf16_round(rng.standard_normal((nc, 64)).astype(np.float32))
    oc, os_ = oracle.quantize(x)
    # the library's visible counts (device) against the oracle's, counted block by block
    vis_gpu = compressed_visible(dev((P0 + np.arange(T)).astype(np.int64)), 2)
    vis = np.array([oracle.visible_entries(P0 + r, 2) for r in range(T)], np.int32)
    assert np.array_equal(vis_gpu.cpu().numpy(), vis)
    assert vis.min() == (P0 + 1) // 2 and vis.max() == nc
    cache = Cache(dev(oc), dev(os_), _to_dev(k, "bf16"), dev(np.zeros(T, np.int64)), vis_gpu, nc,
                  shared_segment=True)
    q = gen.bf16_round(rng.standard_normal((T, Hq, 512)).astype(np.float32))
    iq = gen.bf16_round(rng.standard_normal((T, H, 64)).astype(np.float32))
    chain = LayerChain([LayerSpec("full")], T, Hq, H, K, nc, torch.bfloat16, DEV, shared_segment=True)
    chain.step(cache, [_to_dev(q, "bf16")], [_to_dev(iq, "bf16")], 1 / np.sqrt(512))
    torch.cuda.synchronize()
    got = chain.idx[0].cpu().numpy()
    worst = 0.0
    for r in [0, 1, 2, 31, 62, 63]:
        sel, _, _ = oracle.full_select(iq[r], k, int(vis[r]), K)
        assert np.array_equal(got[r], sel), "row %d" % r
        assert got[r].max() < vis[r]
        o, lse = oracle.attention(q[r], oc, os_, sel, int(vis[r]), 1 / np.sqrt(512))
        worst = max(worst, check_attention(chain.out[0][r:r + 1], chain.lse[0][r:r + 1], o[None], lse[None],
                                           "m=2 row %d" % r))
    say("max err %.3e" % worst)
