"""csa2_sparse_attn_noalloc: the attention call that allocates nothing and keeps its split
partials in the library's own scratch.  Checked against csa2_sparse_attn with a workspace (the
same kernels, so the same bits) on calls in a row that shrink, and for its size limit."""
import numpy as np
import pytest
import torch

import oracle
from gen import bf16_round
from gpu_util import DEV, dev, dev_bf16, say
from sparse_attention_fp4_e4m3_amd import csa2

pytestmark = pytest.mark.gpu


def _inputs(rng, n, R, Hq, K, qkind):
    q = rng.standard_normal((R, Hq, 512)).astype(np.float32)
    q = dev_bf16(bf16_round(q)) if qkind == "bf16" else dev((q / np.sqrt(512)).astype(np.float32))
    idx = np.stack([rng.permutation(n)[:K] for _ in range(R)]).astype(np.int32)
    idx[:, ::29] = -1
    vis = rng.integers(n // 2, n + 1, R).astype(np.int32)
    return q, dev(idx), dev(vis), dev(np.zeros(R, np.int64))


def _with_workspace(q, codes, scales, starts, idx, vis, out_dtype):
    R, Hq, _ = q.shape
    qdt = csa2.F32 if q.dtype == torch.float32 else csa2.BF16
    ws = torch.zeros(max(256, csa2.sparse_attn_workspace_size(R, Hq, qdt, idx.shape[1])), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty(R, Hq, 512, dtype=out_dtype, device=DEV)
    lse = torch.empty(R, Hq, dtype=torch.float32, device=DEV)
    csa2.sparse_attn(q, codes, scales, starts, idx, out, 0.0441941738, row_visible=vis, lse=lse, workspace=ws)
    return out, lse


def test_noalloc_equals_workspace_call_on_shrinking_calls():
    n = 9000
    rng = np.random.default_rng(77)
    x = rng.standard_normal((n, 512)).astype(np.float32)
    oc, os_ = oracle.quantize(x)
    codes, scales = dev(oc), dev(os_)
    # split merge in the launch (32 and 8 pairs), then a separate merge launch (6 pairs), then the
    # general kernel (fp32 queries), then no partials at all (one split per row)
    calls = [(32, 64, 2048, "bf16", torch.float32), (4, 64, 1024, "bf16", torch.bfloat16),
             (3, 64, 2048, "bf16", torch.float32), (2, 16, 640, "f32", torch.float32),
             (1, 16, 100, "bf16", torch.float32)]
    for i, (R, Hq, K, qkind, odt) in enumerate(calls):
        q, idx, vis, starts = _inputs(rng, n, R, Hq, K, qkind)
        ref_o, ref_l = _with_workspace(q, codes, scales, starts, idx, vis, odt)
        out = torch.full((R, Hq, 512), float("nan"), dtype=odt, device=DEV)
        lse = torch.full((R, Hq), float("nan"), dtype=torch.float32, device=DEV)
        csa2.sparse_attn_noalloc(q, codes, scales, starts, idx, out, 0.0441941738, row_visible=vis, lse=lse)
        torch.cuda.synchronize()
        say("noalloc call %d: R=%d Hq=%d K=%d %s" % (i, R, Hq, K, qkind))
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), "call %d differs from the workspace call" % i
        # and the same again: the scratch keeps the previous call's partials, the counters are zero
        csa2.sparse_attn_noalloc(q, codes, scales, starts, idx, out, 0.0441941738, row_visible=vis, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), "repeat of call %d differs" % i


def test_noalloc_rejects_shapes_beyond_its_scratch():
    R, Hq, K = 255, 32, 4096
    need = csa2.sparse_attn_workspace_size(R, Hq, csa2.BF16, K)
    assert need > 16 << 20
    q = torch.zeros(R, Hq, 512, dtype=torch.bfloat16, device=DEV)
    codes = torch.zeros(16, 256, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(16, 32, dtype=torch.uint8, device=DEV)
    idx = torch.full((R, K), -1, dtype=torch.int32, device=DEV)
    out = torch.full((R, Hq, 512), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(csa2.CSA2Error) as e:
        csa2.sparse_attn_noalloc(q, codes, scales, torch.zeros(R, dtype=torch.int64, device=DEV), idx, out, 0.04)
    assert e.value.code == -3 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a rejected call launched work"


def test_noalloc_in_a_graph_replays():
    """Under graph capture (the caller it is for): replays equal the eager call."""
    n = 6000
    rng = np.random.default_rng(78)
    oc, os_ = oracle.quantize(rng.standard_normal((n, 512)).astype(np.float32))
    codes, scales = dev(oc), dev(os_)
    q, idx, vis, starts = _inputs(rng, n, 16, 64, 2048, "bf16")
    ref_o, ref_l = _with_workspace(q, codes, scales, starts, idx, vis, torch.float32)
    out = torch.empty(16, 64, 512, dtype=torch.float32, device=DEV)
    lse = torch.empty(16, 64, dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        csa2.sparse_attn_noalloc(q, codes, scales, starts, idx, out, 0.0441941738, row_visible=vis, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        csa2.sparse_attn_noalloc(q, codes, scales, starts, idx, out, 0.0441941738, row_visible=vis, lse=lse)
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), "replay %d differs" % rep
