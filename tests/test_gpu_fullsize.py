"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times, checked against the CPU oracle on sampled sequences/rows.

For every sampled sequence the oracle regenerates the raw inputs from the
seeded generators and computes, on its own: FP4 codes of every entry the
check touches, the Full indexer scores over the whole visible context, the
top-K, the hierarchical pool, Reindex selections and the attention of every
layer (joined with the layer's FP8 window, over MXFP4 indexer keys, or for
every draft row of a sequence, in the corresponding variants).  Indices, pools and codes must match bit for bit; attention outputs
within 2e-3 (row-normwise per head).
"""
import numpy as np
import pytest
import torch

import bench
import gen
import oracle
from gpu_util import DEV, check_attention, dev, say
from sparse_attention_fp4_e4m3_amd import Cache, LayerChain, LayerSpec, csa2

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


def _chain_fullsize(name, sample, swa=False, mxfp4=False, select_all=False):
    """The named decode workload at full size, as the benchmark runs it (optionally with every
    layer's FP8 window, or with MXFP4 indexer keys), checked on the sampled sequences (every
    draft row of a sequence for the verification workload).  select_all: the indices and pools
    of every selecting layer are also checked for every other sequence."""
    w = gen.get(name)
    V = w.verify
    lens = gen.seq_lens(w)
    say("%s: building the FP4 cache (%d entries)" % (name, int(lens.sum())))
    cache, starts = bench.build_cache(w, lens, DEV, mxfp4=mxfp4)
    vis_rows = np.concatenate([lens[b] - V + 1 + np.arange(V) for b in range(w.B)]).astype(np.int32)
    if V > 1:
        cache.row_kv_start = dev(np.repeat(starts, V).astype(np.int64))
        cache.row_visible = dev(vis_rows)
    qs, iqs = bench.layer_inputs(w, DEV)
    wins = bench.build_windows(w, lens, DEV)[0] if swa else None
    chain = LayerChain([LayerSpec(L.mode, L.pool_size) for L in w.layers], w.rows, w.Hq, w.H, w.K, cache.max_visible,
                       qs[0].dtype, DEV, swa=swa)
    chain.step(cache, qs, iqs, w.softmax_scale, windows=wins)
    torch.cuda.synchronize()
    if select_all:
        for b in range(w.B):
            if b in sample:
                continue  # checked in full below
            n = int(lens[b])
            ik = gen.idx_k_rows(w, b, 0, n)
            if mxfp4:
                ik = oracle.mxfp4_dequant(*oracle.mxfp4_quantize(ik))
            for i in range(V):
                r, nv = b * V + i, int(vis_rows[b * V + i])
                pool = None
                for li, L in enumerate(w.layers):
                    if L.mode == "full":
                        sel, pool, _ = oracle.full_select(gen.index_q(w, li, r, r + 1)[0], ik, nv, w.K, L.pool_size)
                        if L.pool_size:
                            assert np.array_equal(chain.pool[li][0][r].cpu().numpy(), pool), "pool differs: row %d" % r
                    elif L.mode == "reindex":
                        sel = oracle.reindex_select(gen.index_q(w, li, r, r + 1)[0], ik, pool, nv, w.K)
                    else:
                        continue
                    assert np.array_equal(chain.idx[li][r].cpu().numpy(), sel), "indices differ: layer %d row %d" % (li, r)
            say("%s: sequence %d selections exact" % (name, b))
    for b in sample:
        n, s0 = int(lens[b]), int(starts[b])
        say("%s: oracle for sequence %d (n=%d)" % (name, b, n))
        ik = gen.idx_k_rows(w, b, 0, n)
        if mxfp4:  # the keys the GPU scores: MXFP4 of the same values, dequantized exactly
            ik = oracle.mxfp4_dequant(*oracle.mxfp4_quantize(ik))
        raw = gen.kv_rows(w, b, 0, n)
        touched = set()
        ref = {}
        for i in range(V):
            r, nv = b * V + i, int(vis_rows[b * V + i])
            pool = sel = None
            for li, L in enumerate(w.layers):
                if L.mode == "full":
                    sel, pool, plen = oracle.full_select(gen.index_q(w, li, r, r + 1)[0], ik, nv, w.K, L.pool_size)
                elif L.mode == "reindex":
                    sel = oracle.reindex_select(gen.index_q(w, li, r, r + 1)[0], ik, pool, nv, w.K)
                ref[r, li] = (sel.copy(), None if pool is None else pool.copy(), nv)
                touched.update(int(j) for j in sel if j >= 0)
        rng = np.random.default_rng(b)
        rows = np.array(sorted(touched | set(rng.integers(0, n, 2000).tolist()) | {0, n - 1}), np.int64)
        oc_rows, os_rows = oracle.quantize(raw[rows])
        gc = cache.kv_codes[s0 + torch.from_numpy(rows).to(DEV)].cpu().numpy()
        gs = cache.kv_scales[s0 + torch.from_numpy(rows).to(DEV)].cpu().numpy()
        assert np.array_equal(gc, oc_rows) and np.array_equal(gs, os_rows), "codes differ, sequence %d" % b
        # the oracle's own cache for the rows attention reads (others stay zero and are never selected)
        oc = np.zeros((n, 256), np.uint8)
        os_ = np.zeros((n, 32), np.uint8)
        oc[rows], os_[rows] = oc_rows, os_rows
        for (r, li), (sel, pool, nv) in sorted(ref.items()):
            L = w.layers[li]
            if L.mode != "reuse":
                got = chain.idx[li][r].cpu().numpy()
                assert np.array_equal(got, sel), "indices differ: layer %d row %d" % (li, r)
            if L.mode == "full" and L.pool_size:
                gp, gl = chain.pool[li]
                assert np.array_equal(gp[r].cpu().numpy(), pool), "pool differs: row %d" % r
            q = gen.attn_q(w, li, r, r + 1)
            if swa:
                wc = oracle.e4m3_encode_signed(gen.window_rows(w, li, b, max(0, n - 128), n))
                z = np.zeros(1, np.int64)
                o, lse = oracle.attention_rows_swa(q, oc, os_, z, sel[None], np.array([nv]), wc, z,
                                                   np.array([len(wc)], np.int32), w.softmax_scale)
                o, lse = o[0], lse[0]
            else:
                o, lse = oracle.attention(q[0], oc, os_, sel, nv, w.softmax_scale)
            check_attention(chain.out[li][r:r + 1], chain.lse[li][r:r + 1], o[None], lse[None],
                            "%s layer %d (%s) row %d" % (name, li, L.mode, r))


def test_decode_full_32x_32k_64k():
    _chain_fullsize("c2", sample=[0, 17, 31], select_all=True)


def test_chain_128k_batch16():
    _chain_fullsize("c3", sample=[0, 9], select_all=True)


def test_chain_128k_batch16_with_local_windows():
    _chain_fullsize("c3", sample=[0, 9], swa=True)


def test_chain_128k_batch16_mxfp4_indexer_keys():
    _chain_fullsize("c3", sample=[0, 9], mxfp4=True)


def test_chain_128k_verification_5_draft_rows():
    _chain_fullsize("c3v", sample=[3], select_all=True)


def test_long_decode_1m_batch4():
    _chain_fullsize("c5", sample=[0, 1, 2, 3])


def test_prefill_4096_on_256k():
    """4096 new tokens appended causally to 262,144 cached: row r sees [0, 262144 + r]; then the same
    attention joined with each row's 128-token FP8 window."""
    w = gen.get("c4")
    T = w.prefill_tokens
    P0 = w.n - T
    lens = np.array([w.n], np.int64)
    say("c4: building the FP4 cache of the %d cached tokens" % P0)
    codes = torch.empty(w.n, 256, dtype=torch.uint8, device=DEV)
    scales = torch.empty(w.n, 32, dtype=torch.uint8, device=DEV)
    for t0 in range(0, P0, 65536):
        t1 = min(P0, t0 + 65536)
        csa2.quantize_kv_fp4(torch.from_numpy(gen.kv_rows(w, 0, t0, t1)).to(DEV), codes[t0:t1], scales[t0:t1])
    ik_all = gen.idx_k_rows(w, 0, 0, w.n)
    idx_k = torch.from_numpy(gen.bf16_bits(ik_all).view(np.int16)).view(torch.bfloat16).to(DEV)
    # the chunk writes its own KV first (quantize-on-write at rows P0..P0+T-1)
    new = torch.from_numpy(gen.kv_rows(w, 0, P0, w.n)).to(DEV)
    csa2.quantize_kv_fp4(new, codes, scales, dev(np.arange(P0, w.n, dtype=np.int64)))
    starts = dev(np.zeros(T, np.int64))
    vis = dev((P0 + 1 + np.arange(T)).astype(np.int32))
    iq = bench.to_dev(gen.index_q(w, 0), w.idx_dtype, DEV)
    q = bench.to_dev(gen.attn_q(w, 0), w.q_dtype, DEV)
    # the benchmark's configuration: one shared segment (approximate MFMA passes + exact rescoring)
    ws = torch.empty(csa2.index_topk_workspace_size(csa2.FULL_SHARED, T, w.H, w.n, 0, w.K, 0), dtype=torch.uint8,
                     device=DEV)
    idx = torch.empty(T, w.K, dtype=torch.int32, device=DEV)
    csa2.index_topk(csa2.FULL_SHARED, iq, idx_k, starts, vis, w.n, w.K, idx, ws)
    del ws
    out = torch.empty(T, w.Hq, 512, dtype=torch.float32, device=DEV)
    lse = torch.empty(T, w.Hq, dtype=torch.float32, device=DEV)
    aws = torch.zeros(max(256, csa2.sparse_attn_workspace_size(T, w.Hq, csa2.BF16, w.K)), dtype=torch.uint8,
                      device=DEV)
    csa2.sparse_attn(q, codes, scales, starts, idx, out, w.softmax_scale, row_visible=vis, lse=lse, workspace=aws)
    torch.cuda.synchronize()
    raw = gen.kv_rows(w, 0, 0, w.n)
    # 64 rows spread over the chunk plus the edges.  None of this workload's rows takes the
    # certification-failure or candidate-overflow fallbacks; test_gpu_prefill.py forces both.
    sample_rows = sorted(set(np.linspace(0, T - 1, 64).astype(int).tolist()) | {0, 1, 777, 2048, T - 1})
    for r in sample_rows:
        say("c4: oracle for query row %d (sees %d entries)" % (r, P0 + r + 1))
        nvis = P0 + r + 1
        sel = oracle.topk(oracle.index_scores(gen.index_q(w, 0, r, r + 1)[0], ik_all[:nvis]), w.K)
        assert np.array_equal(idx[r].cpu().numpy(), sel), "indices differ, row %d" % r
        rows = np.array(sorted(set(int(j) for j in sel if j >= 0) | {P0 + r}), np.int64)
        oc_rows, os_rows = oracle.quantize(raw[rows])
        assert np.array_equal(codes[torch.from_numpy(rows).to(DEV)].cpu().numpy(), oc_rows)
        assert np.array_equal(scales[torch.from_numpy(rows).to(DEV)].cpu().numpy(), os_rows)
        oc = np.zeros((w.n, 256), np.uint8)
        os_ = np.zeros((w.n, 32), np.uint8)
        oc[rows], os_[rows] = oc_rows, os_rows
        o, l = oracle.attention(gen.attn_q(w, 0, r, r + 1)[0], oc, os_, sel, nvis, w.softmax_scale)
        check_attention(out[r:r + 1], lse[r:r + 1], o[None], l[None], "c4 row %d" % r)
    # the same chunk with the local windows joined (the benchmark's --swa configuration): each row's
    # 128-token FP8 window ends at its own position; the chunk's window rows are written first
    wins, new_win, new_win_rows = bench.build_windows(w, lens, DEV)
    csa2.quantize_swa_fp8(new_win[0], wins[0].codes, new_win_rows)
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    aws = torch.zeros(max(256, csa2.sparse_attn_swa_workspace_size(T, w.Hq, csa2.BF16, w.K)), dtype=torch.uint8,
                      device=DEV)
    csa2.sparse_attn_swa(q, wins[0].codes, wins[0].row_start, wins[0].row_len, out2, w.softmax_scale,
                         kv_codes=codes, kv_scales=scales, row_kv_start=starts, idx=idx, row_visible=vis, lse=lse2,
                         workspace=aws)
    torch.cuda.synchronize()
    for r in [0, 1, 2048, T - 1]:
        nvis = P0 + r + 1
        sel = idx[r].cpu().numpy()
        rows = np.array(sorted(set(int(j) for j in sel if j >= 0)), np.int64)
        oc = np.zeros((w.n, 256), np.uint8)
        os_ = np.zeros((w.n, 32), np.uint8)
        oc[rows], os_[rows] = oracle.quantize(raw[rows])
        wc = oracle.e4m3_encode_signed(gen.window_rows(w, 0, 0, nvis - 128, nvis))
        z = np.zeros(1, np.int64)
        o, l = oracle.attention_rows_swa(gen.attn_q(w, 0, r, r + 1), oc, os_, z, sel[None], np.array([nvis]), wc, z,
                                         np.array([128], np.int32), w.softmax_scale)
        check_attention(out2[r:r + 1], lse2[r:r + 1], o, l, "c4 window row %d" % r)
    # the same chunk's selection over MXFP4 indexer keys (MFMA passes on the widened keys, exact
    # rescoring on the dequantized ones), against the oracle over the dequantized keys
    kc = torch.empty(w.n, 32, dtype=torch.uint8, device=DEV)
    kscl = torch.empty(w.n, 2, dtype=torch.uint8, device=DEV)
    csa2.quantize_idx_mxfp4(idx_k, kc, kscl)
    ws = torch.empty(csa2.index_topk_workspace_size(csa2.FULL_SHARED, T, w.H, w.n, 0, w.K, 0), dtype=torch.uint8,
                     device=DEV)
    idx_mx = torch.empty(T, w.K, dtype=torch.int32, device=DEV)
    csa2.index_topk_mxfp4(csa2.FULL_SHARED, iq, kc, kscl, starts, vis, w.n, w.K, idx_mx, ws)
    torch.cuda.synchronize()
    del ws
    ikh = oracle.mxfp4_dequant(*oracle.mxfp4_quantize(ik_all))
    for r in sample_rows[::4]:
        nvis = P0 + r + 1
        sel = oracle.topk(oracle.index_scores(gen.index_q(w, 0, r, r + 1)[0], ikh[:nvis]), w.K)
        assert np.array_equal(idx_mx[r].cpu().numpy(), sel), "MXFP4 indices differ, row %d" % r
    # causality: no row selects a position it cannot see
    idx_np = idx.cpu().numpy()
    limit = (P0 + np.arange(T))[:, None]
    assert np.all((idx_np == -1) | ((idx_np >= 0) & (idx_np <= limit)))
