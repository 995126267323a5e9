"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects bad host-side arguments before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

from sparse_attention_fp4_e4m3_amd import csa2
from sparse_attention_fp4_e4m3_amd.chain import LayerSpec, validate_modes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(csa2_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    if not os.path.exists(csa2.LIB_PATH):
        pytest.skip("libcsa2.so not built")
    csa2.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", csa2.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (csa2_\w+)", out))
    declared = _declared()
    assert declared and set(declared) <= exported, set(declared) - exported
    assert set(csa2.EXPORTED) == set(declared)


def _L():
    if not os.path.exists(csa2.LIB_PATH):
        pytest.skip("libcsa2.so not built")
    return csa2.lib()


def _err():
    return _L().csa2_last_error().decode()


def test_quantize_rejects_bad_arguments():
    L = _L()
    fake = ctypes.c_void_p(0x1000)
    assert L.csa2_quantize_kv_fp4(fake, 7, 4, 512, None, fake, fake, 10, None) == -1 and "dtype" in _err()
    assert L.csa2_quantize_kv_fp4(None, 0, 4, 512, None, fake, fake, 10, None) == -1 and "null" in _err()
    assert L.csa2_quantize_kv_fp4(fake, 0, 4, 100, None, fake, fake, 10, None) == -1 and "stride" in _err()
    assert L.csa2_quantize_kv_fp4(fake, 0, 40, 512, None, fake, fake, 10, None) == -1 and "cap_rows" in _err()
    assert L.csa2_quantize_kv_fp4(ctypes.c_void_p(0x1004), 0, 4, 512, None, fake, fake, 10, None) == -1
    assert L.csa2_quantize_kv_fp4(fake, 0, -1, 512, None, fake, fake, 10, None) == -1
    assert L.csa2_quantize_kv_fp4(None, 0, 0, 512, None, None, None, 10, None) == 0  # nothing to do


def _topk(L, **kw):
    f = ctypes.c_void_p(0x10000)
    a = dict(mode=0, n_rows=2, q=f, qd=1, H=8, D=64, k=f, kd=1, kh=1, start=f, vis=f, maxv=1000, pool=None,
             plen=None, pstride=0, K=256, out=f, P=0, blk=0, opool=None, oplen=None, ws=f, wsb=1 << 30)
    a.update(kw)
    return L.csa2_index_topk(a["mode"], a["n_rows"], a["q"], a["qd"], a["H"], a["D"], a["k"], a["kd"], a["kh"],
                             a["start"],
                             a["vis"], a["maxv"], a["pool"], a["plen"], a["pstride"], a["K"], a["out"], a["P"],
                             a["blk"], a["opool"], a["oplen"], a["ws"], a["wsb"], None)


def test_index_topk_rejects_bad_arguments():
    L = _L()
    assert _topk(L, mode=5) == -1
    assert _topk(L, D=128) == -2 and "head_dim" in _err()
    assert _topk(L, H=0) == -2 and _topk(L, H=33) == -2
    assert _topk(L, K=0) == -1 and _topk(L, K=4097) == -1 and "top_k" in _err()
    assert _topk(L, q=None) == -1 and "null" in _err()
    assert _topk(L, mode=1) == -1 and "pool" in _err()  # Reindex without a pool
    assert _topk(L, P=100, blk=8, opool=ctypes.c_void_p(0x10000), oplen=ctypes.c_void_p(0x10000)) == -1
    assert _topk(L, P=1024, blk=4, opool=ctypes.c_void_p(0x10000), oplen=ctypes.c_void_p(0x10000)) == -1
    assert _topk(L, P=1024, blk=8) == -1  # pool outputs missing
    assert _topk(L, wsb=16) == -3 and "workspace" in _err()
    assert _topk(L, ws=None) == -3
    assert _topk(L, n_rows=0) == 0
    # one key shared by the query heads is the only key layout built
    assert _topk(L, kh=8) == -2 and "k_heads" in _err()
    assert _topk(L, kh=0) == -2


def test_visible_entries_rejects_bad_arguments():
    L = _L()
    f = ctypes.c_void_p(0x10000)
    assert L.csa2_visible_entries(f, 0, 4, f, None) == -1 and "tokens_per_entry" in _err()
    assert L.csa2_visible_entries(None, 2, 4, f, None) == -1 and "null" in _err()
    assert L.csa2_visible_entries(f, 2, -1, f, None) == -1
    assert L.csa2_visible_entries(None, 2, 0, None, None) == 0  # nothing to do


def test_workspace_sizes_grow_with_the_problem():
    L = _L()
    a = L.csa2_index_topk_workspace_size(0, 16, 8, 131072, 0, 2048, 8192)
    b = L.csa2_index_topk_workspace_size(0, 16, 8, 131072, 0, 2048, 0)
    c = L.csa2_index_topk_workspace_size(0, 16, 8, 1 << 20, 0, 2048, 0)
    assert a > b > 16 * 131072 * 4 - 1 and c > b
    assert L.csa2_sparse_attn_workspace_size(16, 64, 1, 2048) > 0  # split-K partials
    assert L.csa2_sparse_attn_workspace_size(4096, 64, 1, 2048) == 0  # one split per row
    assert L.csa2_sparse_attn_workspace_size(16, 60, 1, 2048) == 0  # invalid head count


def _attn(L, **kw):
    f = ctypes.c_void_p(0x10000)
    a = dict(R=2, q=f, qd=1, H=64, D=512, codes=f, scales=f, start=f, idx=f, K=256, vis=None, scale=0.1, out=f,
             od=0, lse=None, ws=f, wsb=1 << 30)
    a.update(kw)
    return L.csa2_sparse_attn(a["R"], a["q"], a["qd"], a["H"], a["D"], a["codes"], a["scales"], a["start"],
                              a["idx"], a["K"], a["vis"], a["scale"], a["out"], a["od"], a["lse"], a["ws"], a["wsb"],
                              None)


def test_sparse_attn_rejects_bad_arguments():
    L = _L()
    assert _attn(L, D=576) == -2 and "head_dim" in _err()
    assert _attn(L, H=40) == -1 and _attn(L, H=256) == -1
    assert _attn(L, K=0) == -1
    assert _attn(L, qd=3) == -1 and _attn(L, od=9) == -1
    assert _attn(L, q=None) == -1 and "null" in _err()
    assert _attn(L, q=ctypes.c_void_p(0x10008)) == -1 and "aligned" in _err()
    assert _attn(L, K=2048, ws=None, wsb=0) == -3  # split keys need partials
    assert _attn(L, scale=float("nan")) == -1
    assert _attn(L, R=0) == 0


def _swa(L, **kw):
    f = ctypes.c_void_p(0x10000)
    a = dict(R=2, q=f, qd=1, H=64, D=512, codes=f, scales=f, start=f, idx=f, K=256, vis=None, win=f, ws0=f, wl=f,
             nx=None, nxd=0, nxs=0, nr=None, scale=0.1, out=f, od=0, lse=None, ws=f, wsb=1 << 30)
    a.update(kw)
    return L.csa2_sparse_attn_swa(a["R"], a["q"], a["qd"], a["H"], a["D"], a["codes"], a["scales"], a["start"],
                                  a["idx"], a["K"], a["vis"], a["win"], a["ws0"], a["wl"], a["nx"], a["nxd"], a["nxs"],
                                  a["nr"], a["scale"], a["out"], a["od"], a["lse"], a["ws"], a["wsb"], None)


def test_window_calls_reject_bad_arguments():
    L = _L()
    f = ctypes.c_void_p(0x10000)
    assert _swa(L, D=576) == -2 and "head_dim" in _err()
    assert _swa(L, H=40) == -1 and _swa(L, K=-1) == -1
    assert _swa(L, win=None) == -1 and "null" in _err()
    assert _swa(L, wl=None) == -1 and _swa(L, ws0=None) == -1
    assert _swa(L, idx=None) == -1 and "top_k" in _err()
    assert _swa(L, win=ctypes.c_void_p(0x10008)) == -1 and "aligned" in _err()
    assert _swa(L, ws=None, wsb=0) == -3
    assert _swa(L, R=0) == 0
    assert _swa(L, nx=f, nxd=5, nxs=512, nr=f) == -1 and "new_x_dtype" in _err()
    assert _swa(L, nx=f, nxd=0, nxs=512, nr=None) == -1 and "new_rows" in _err()
    assert _swa(L, nx=f, nxd=0, nxs=100, nr=f) == -1 and "stride" in _err()
    assert _swa(L, nx=ctypes.c_void_p(0x10004), nxd=0, nxs=512, nr=f) == -1 and "aligned" in _err()
    # window only: the cache and index arguments are not needed
    assert L.csa2_sparse_attn_swa_workspace_size(2, 64, 1, 0) == 0  # one slot: written directly
    assert L.csa2_sparse_attn_swa_workspace_size(2, 64, 1, 256) > 0
    assert L.csa2_sparse_attn_swa_workspace_size(16, 64, 1, 2048) > L.csa2_sparse_attn_workspace_size(16, 64, 1, 2048)
    assert L.csa2_sparse_attn_swa_workspace_size(4096, 64, 1, 2048) == 0  # 64-head workgroups: the window is a step
    assert L.csa2_quantize_swa_fp8(f, 7, 4, 512, None, f, 10, None) == -1 and "dtype" in _err()
    assert L.csa2_quantize_swa_fp8(None, 0, 4, 512, None, f, 10, None) == -1 and "null" in _err()
    assert L.csa2_quantize_swa_fp8(f, 0, 4, 100, None, f, 10, None) == -1 and "stride" in _err()
    assert L.csa2_quantize_swa_fp8(f, 0, 40, 512, None, f, 10, None) == -1 and "cap_rows" in _err()
    assert L.csa2_quantize_swa_fp8(f, 0, 4, 512, None, ctypes.c_void_p(0x10004), 10, None) == -1
    assert L.csa2_quantize_swa_fp8(None, 0, 0, 512, None, None, 10, None) == 0


def test_mxfp4_calls_reject_bad_arguments():
    L = _L()
    f = ctypes.c_void_p(0x10000)
    assert L.csa2_quantize_idx_mxfp4(f, 7, 4, 64, None, f, f, 10, None) == -1 and "dtype" in _err()
    assert L.csa2_quantize_idx_mxfp4(f, 0, 4, 64, None, f, None, 10, None) == -1 and "null" in _err()
    assert L.csa2_quantize_idx_mxfp4(f, 0, 4, 32, None, f, f, 10, None) == -1 and "stride" in _err()
    assert L.csa2_quantize_idx_mxfp4(f, 0, 40, 64, None, f, f, 10, None) == -1 and "cap_rows" in _err()
    assert L.csa2_quantize_idx_mxfp4(f, 0, 4, 64, None, ctypes.c_void_p(0x10008), f, 10, None) == -1
    assert L.csa2_quantize_idx_mxfp4(None, 0, 0, 64, None, None, None, 10, None) == 0
    args = [0, 2, f, 1, 8, 64, f, f, 1, f, f, 1000, None, None, 0, 64, f, 0, 0, None, None, f, 1 << 30, None]
    bad = list(args)
    bad[7] = None  # scales
    assert L.csa2_index_topk_mxfp4(*bad) == -1 and "null" in _err()
    bad = list(args)
    bad[7] = ctypes.c_void_p(0x10001)
    assert L.csa2_index_topk_mxfp4(*bad) == -1 and "aligned" in _err()
    bad = list(args)
    bad[5] = 128
    assert L.csa2_index_topk_mxfp4(*bad) == -2
    # MXFP4 keys are not accepted by the two-format call
    assert L.csa2_index_topk(0, 2, f, 1, 8, 64, f, 2, 1, f, f, 1000, None, None, 0, 64, f, 0, 0, None, None, f,
                             1 << 30, None) == -1 and "mxfp4" in _err()
    bad = list(args)
    bad[8] = 2  # k_heads
    assert L.csa2_index_topk_mxfp4(*bad) == -2 and "k_heads" in _err()


def test_profile_hook_ids():
    L = _L()
    assert L.csa2_profile_kernel_events(99, None, None) == -1
    assert L.csa2_profile_kernel_events(2, None, None) == 0
    assert L.csa2_profile_kernel_events(8, None, None) == 0 and L.csa2_profile_kernel_events(9, None, None) == -1


def test_layer_mode_rules():
    F, X, R = LayerSpec("full", 8192), LayerSpec("reindex"), LayerSpec("reuse")
    validate_modes([F, X, X, R, R, R])
    validate_modes([LayerSpec("full"), R, R])
    with pytest.raises(ValueError):
        validate_modes([R, F])
    with pytest.raises(ValueError):
        validate_modes([LayerSpec("full"), X])  # the Full layer emits no pool
    with pytest.raises(ValueError):
        validate_modes([X])
    with pytest.raises(ValueError):
        validate_modes([F, LayerSpec("reuse", 16)])
