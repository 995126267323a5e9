"""GPU parity of the local sliding-window branch against the CPU oracle.

Bit-exact: the FP8 (signed E4M3) window codes.  Attention with the window
joined to the selected entries: within 2e-3 max relative error per row and
head (normwise), lse within 1e-3, on every launch path (split-K partials
of 16-head and pipelined workgroups with a window kernel, 64-head
workgroups that take the window as one more step, window only).
Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import oracle
from gen import bf16_round
from gpu_util import DEV, as_dtype, check_attention, dev, dev_bf16, say
from sparse_attention_fp4_e4m3_amd import csa2

pytestmark = pytest.mark.gpu


def _fp8_edge_values():
    grid = np.array([oracle.e4m3_value(b) for b in range(0x7F)])
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)  # every tie
    v = np.concatenate([grid.astype(np.float32), mids, [449.0, 464.0, 1e6, 1e-9, 0.0, -0.0]]).astype(np.float32)
    v = np.concatenate([v, -v])
    return np.resize(v, (len(v) + 511) // 512 * 512).reshape(-1, 512)


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_window_quantize_bit_exact(kind):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((300, 512)).astype(np.float32) * np.exp2(rng.uniform(-10, 8, (300, 1))).astype(np.float32)
    x = np.concatenate([x, _fp8_edge_values()])
    if kind == "bf16":
        x = bf16_round(x)
    n = x.shape[0]
    # a strided input (row stride 640) and a scatter with skipped destinations
    xs = np.zeros((n, 640), np.float32)
    xs[:, :512] = x
    xt = as_dtype(xs, kind)[:, :]
    dst = np.arange(n, dtype=np.int64)[::-1].copy()
    dst[::7] = -1
    dst[3] = n + 5
    codes = torch.full((n, 512), 0xAB, dtype=torch.uint8, device=DEV)
    csa2.quantize_swa_fp8(xt, codes, dev(dst))
    want = oracle.e4m3_encode_signed(x)
    got = codes.cpu().numpy()
    for t in range(n):
        d = dst[t]
        if 0 <= d < n:
            assert np.array_equal(got[d], want[t]), "token %d" % t
    untouched = np.setdiff1d(np.arange(n), dst[(dst >= 0) & (dst < n)])
    assert np.all(got[untouched] == 0xAB)
    say("window quantize %s: %d rows bit-exact" % (kind, n))


def _window_case(seed, R, Hq, qkind, K, n, lens, W=600):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 512)).astype(np.float32)
    x[:, [3, 77, 200, 311, 500]] *= 20
    oc, os_ = oracle.quantize(x)
    wx = rng.standard_normal((W, 512)).astype(np.float32)
    wx[:, [3, 77, 200, 311, 500]] *= 20
    wc = oracle.e4m3_encode_signed(wx)
    q = rng.standard_normal((R, Hq, 512)).astype(np.float32) * (1 / np.sqrt(512) if qkind == "f32" else 1)
    if qkind == "bf16":
        q = bf16_round(q)
    vis = rng.integers(n // 2, n + 1, R).astype(np.int32)
    if K > 0:
        idx = np.stack([rng.permutation(n)[:K] for _ in range(R)]).astype(np.int32)
        idx[:, ::13] = -1
    else:
        idx = np.zeros((R, 0), np.int32)
    wlen = np.resize(np.array(lens, np.int32), R)
    wstart = rng.integers(0, W - 128, R).astype(np.int64)
    return q, oc, os_, wc, idx, vis, wstart, wlen


def _run(q, qkind, oc, os_, wc, idx, vis, wstart, wlen, scale, out_dtype=torch.float32):
    R, Hq, _ = q.shape
    K = idx.shape[1]
    qdt = csa2.F32 if qkind == "f32" else csa2.BF16
    ws = torch.zeros(max(256, csa2.sparse_attn_swa_workspace_size(R, Hq, qdt, K)), dtype=torch.uint8, device=DEV)
    out = torch.empty(R, Hq, 512, dtype=out_dtype, device=DEV)
    lse = torch.empty(R, Hq, dtype=torch.float32, device=DEV)
    kw = {}
    if K > 0:
        kw = dict(kv_codes=dev(oc), kv_scales=dev(os_), row_kv_start=dev(np.zeros(R, np.int64)), idx=dev(idx),
                  row_visible=dev(vis))
    csa2.sparse_attn_swa(as_dtype(q, qkind), dev(wc), dev(wstart), dev(wlen), out, scale, lse=lse, workspace=ws, **kw)
    return out, lse


@pytest.mark.parametrize("Hq,qkind,R,K,n,lens", [
    (16, "f32", 2, 256, 4096, [128, 37]),          # the tiny decode shape: fp32 queries, hi/lo halves
    (64, "bf16", 4, 2048, 9000, [128, 1, 77, 0]),  # decode: split-K partials + window slot, ragged windows
    (64, "bf16", 16, 2048, 9000, [128]),           # pipelined 16-head workgroups
    (64, "bf16", 32, 1500, 6000, [128, 100]),      # pipelined 32-head workgroups, ragged last split
    (32, "bf16", 5, 300, 3000, [64, 128, 5]),
    (64, "bf16", 256, 300, 5000, [128, 127, 31]),  # 64-head workgroups: the window as their last step
    (128, "bf16", 160, 200, 3000, [128, 0, 96, 33]),  # 64-head workgroups, two per row
    (128, "bf16", 3, 0, 100, [128, 9, 0]),         # window only (the first, local-only layers)
    (32, "f32", 3, 0, 100, [128, 64, 1]),
])
def test_window_attention_matches_oracle(Hq, qkind, R, K, n, lens):
    q, oc, os_, wc, idx, vis, wstart, wlen = _window_case(Hq * 100 + K + R, R, Hq, qkind, K, n, lens)
    scale = 1 / np.sqrt(512)
    out, lse = _run(q, qkind, oc, os_, wc, idx, vis, wstart, wlen, scale)
    ro, rl = oracle.attention_rows_swa(q, oc, os_, np.zeros(R, np.int64), idx, vis.astype(np.int64), wc, wstart,
                                       wlen, scale)
    check_attention(out, lse, ro, rl, "swa Hq=%d %s R=%d K=%d" % (Hq, qkind, R, K))


def test_window_edge_rows_and_output_dtypes():
    R, Hq, K, n = 5, 64, 512, 2000
    q, oc, os_, wc, idx, vis, wstart, wlen = _window_case(7, R, Hq, "bf16", K, n, [0])
    idx[0, :] = -1   # nothing selected, empty window: zeros and -inf
    idx[1, :] = -1   # one window entry alone: that entry exactly
    wlen[1] = 1
    wlen[2] = 200    # clamped to 128
    wlen[3] = -4     # clamped to 0: the global branch alone
    out, lse = _run(q, "bf16", oc, os_, wc, idx, vis, wstart, wlen, 0.05)
    ro, rl = oracle.attention_rows_swa(q, oc, os_, np.zeros(R, np.int64), idx, vis.astype(np.int64), wc, wstart,
                                       wlen, 0.05)
    check_attention(out, lse, ro, rl, "swa edge rows")
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))
    w1 = oracle.fp8_dequant(wc[wstart[1]]).astype(np.float32)
    assert np.array_equal(o[1], np.broadcast_to(w1, o[1].shape))
    again, lse2 = _run(q, "bf16", oc, os_, wc, idx, vis, wstart, wlen, 0.05)
    assert torch.equal(out, again) and torch.equal(lse, lse2), "not bitwise reproducible"
    b, _ = _run(q, "bf16", oc, os_, wc, idx, vis, wstart, wlen, 0.05, out_dtype=torch.bfloat16)
    assert torch.equal(b, out.to(torch.bfloat16))


def test_decode_ring_window_after_quantize():
    """A per-sequence ring of 128 window rows written by the FP8 quantize call
    (row = position mod 128): after t + 1 tokens the valid rows are the first
    min(t + 1, 128), whatever order the ring holds them in."""
    B, Hq, K, n = 3, 64, 1024, 5000
    rng = np.random.default_rng(21)
    steps = [5, 128, 300]  # tokens written so far, per sequence
    ring = torch.zeros(B * 128, 512, dtype=torch.uint8, device=DEV)
    hist = []
    for b in range(B):
        xs = bf16_round(rng.standard_normal((steps[b], 512)).astype(np.float32))
        dst = b * 128 + (np.arange(steps[b]) % 128)
        for c0 in range(0, steps[b], 128):  # one call per lap of the ring: no repeated destination in a call
            csa2.quantize_swa_fp8(dev_bf16(xs[c0:c0 + 128]), ring, dev(dst[c0:c0 + 128].astype(np.int64)))
        hist.append(xs)
    x = rng.standard_normal((n, 512)).astype(np.float32)
    oc, os_ = oracle.quantize(x)
    q = bf16_round(rng.standard_normal((B, Hq, 512)).astype(np.float32))
    idx = np.stack([np.sort(rng.permutation(n)[:K]) for _ in range(B)]).astype(np.int32)
    wstart = np.arange(B, dtype=np.int64) * 128
    wlen = np.minimum(np.array(steps), 128).astype(np.int32)
    vis = np.full(B, n, np.int32)
    out, lse = _run(q, "bf16", oc, os_, ring.cpu().numpy(), idx, vis, wstart, wlen, 0.044)
    # oracle: the last min(t+1, 128) tokens of each sequence, in position order
    wc = np.concatenate([oracle.e4m3_encode_signed(h[-128:]) for h in hist])
    wst = np.cumsum([0] + [min(len(h), 128) for h in hist[:-1]]).astype(np.int64)
    ro, rl = oracle.attention_rows_swa(q, oc, os_, np.zeros(B, np.int64), idx, vis.astype(np.int64), wc, wst, wlen,
                                       0.044)
    check_attention(out, lse, ro, rl, "decode ring window")


@pytest.mark.parametrize("R,Hq,K", [(4, 64, 2048), (256, 64, 300), (3, 32, 0)])
def test_window_write_inside_the_attention_call(R, Hq, K):
    """The attention call writing each row's newest token itself (decode rings) gives the same
    window bytes and the same outputs, bit for bit, as the FP8 quantize call followed by the
    attention call: on the split path, the 64-head path and window only; a token landing outside
    its row's window and a row with no token (-1) included."""
    n = 3000
    rng = np.random.default_rng(R + K)
    oc, os_ = oracle.quantize(rng.standard_normal((n, 512)).astype(np.float32))
    q = bf16_round(rng.standard_normal((R, Hq, 512)).astype(np.float32))
    idx = np.stack([rng.permutation(n)[:K] for _ in range(R)]).astype(np.int32) if K else np.zeros((R, 0), np.int32)
    vis = np.full(R, n, np.int32)
    wstart = np.arange(R, dtype=np.int64) * 128
    wlen = np.resize(np.array([128, 77, 1, 128], np.int32), R)
    ring0 = oracle.e4m3_encode_signed(rng.standard_normal((R * 128, 512)).astype(np.float32))
    new_rows = wstart + rng.integers(0, 128, R)
    new_rows[0] = wstart[0] + 5
    if R > 1:
        new_rows[1] = wstart[1] + 100  # past its 77-entry window: written, not attended
    if R > 2:
        new_rows[2] = -1
    x = rng.standard_normal((R, 512)).astype(np.float32) * 3
    kw = {}
    if K:
        kw = dict(kv_codes=dev(oc), kv_scales=dev(os_), row_kv_start=dev(np.zeros(R, np.int64)), idx=dev(idx),
                  row_visible=dev(vis))
    ws = torch.zeros(max(256, csa2.sparse_attn_swa_workspace_size(R, Hq, csa2.BF16, K)), dtype=torch.uint8,
                     device=DEV)
    outs = []
    rings = []
    for fused in (False, True):
        ring = dev(ring0)
        out = torch.empty(R, Hq, 512, dtype=torch.float32, device=DEV)
        lse = torch.empty(R, Hq, dtype=torch.float32, device=DEV)
        if not fused:
            sel = new_rows >= 0
            csa2.quantize_swa_fp8(dev(x[sel]), ring, dev(new_rows[sel]))
        csa2.sparse_attn_swa(dev_bf16(q), ring, dev(wstart), dev(wlen), out, 0.044, lse=lse, workspace=ws,
                             new_x=dev(x) if fused else None, new_rows=dev(new_rows) if fused else None, **kw)
        torch.cuda.synchronize()
        outs.append((out, lse))
        rings.append(ring.cpu().numpy())
    assert np.array_equal(rings[0], rings[1]), "window bytes differ"
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1]), "outputs differ"
    ro, rl = oracle.attention_rows_swa(q, oc, os_, np.zeros(R, np.int64), idx, vis.astype(np.int64), rings[0],
                                       wstart, wlen, 0.044)
    check_attention(outs[1][0], outs[1][1], ro, rl, "fused window write R=%d K=%d" % (R, K))


@pytest.mark.parametrize("R,Hq,K,out_dtype", [(256, 64, 300, torch.bfloat16), (4, 64, 2048, torch.bfloat16)])
def test_window_attention_bf16_output_matches_fp32_rounded(R, Hq, K, out_dtype):
    """bf16 outputs are the fp32 results rounded to nearest even, on the 64-head path (window as a
    step) and the split path (window partial + combine); the fp32 results meet the attention bar
    (bf16 rounding alone is up to 2^-9 relative, so the bar applies before it)."""
    q, oc, os_, wc, idx, vis, wstart, wlen = _window_case(900 + R, R, Hq, "bf16", K, 6000, [128, 64, 1])
    a, la = _run(q, "bf16", oc, os_, wc, idx, vis, wstart, wlen, 0.044)
    b, lb = _run(q, "bf16", oc, os_, wc, idx, vis, wstart, wlen, 0.044, out_dtype=out_dtype)
    assert torch.equal(b, a.to(torch.bfloat16)) and torch.equal(la, lb)
    ro, rl = oracle.attention_rows_swa(q, oc, os_, np.zeros(R, np.int64), idx, vis.astype(np.int64), wc, wstart,
                                       wlen, 0.044)
    check_attention(a, la, ro, rl, "swa fp32 out R=%d" % R)
