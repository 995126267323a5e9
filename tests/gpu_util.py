"""Helpers of the GPU parity tests: upload, run the C ABI, compare.

The GPU side runs only through sparse_attention_fp4_e4m3_amd (libcsa2.so);
expected values come only from the CPU oracle.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from gen import bf16_bits
from sparse_attention_fp4_e4m3_amd import csa2

DEV = torch.device("cuda:0")
TOL = 2e-3  # max relative error of attention outputs (row-normwise per row and head)


def say(msg: str) -> None:
    print(msg, flush=True)


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    """fp32 values that are bf16-exact -> a bf16 device tensor with the same bits."""
    bits = bf16_bits(np.asarray(a, np.float32))
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)


def as_dtype(a: np.ndarray, kind: str) -> torch.Tensor:
    return dev_bf16(a) if kind == "bf16" else dev(a.astype(np.float32))


def quantize(x: torch.Tensor, cap: int = None, dst_rows: torch.Tensor = None):
    n = x.shape[0] if cap is None else cap
    codes = torch.zeros(n, 256, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(n, 32, dtype=torch.uint8, device=DEV)
    csa2.quantize_kv_fp4(x, codes, scales, dst_rows)
    return codes, scales


def index_topk(mode, idx_q, idx_k, starts, vis, max_visible, K, pool=None, pool_len=None, pool_size=0):
    R, H = idx_q.shape[0], idx_q.shape[1]
    pool_stride = pool.shape[1] if pool is not None else 0
    ws = torch.empty(max(256, csa2.index_topk_workspace_size(mode, R, H, max_visible, pool_stride, K, pool_size)),
                     dtype=torch.uint8, device=DEV)
    idx = torch.empty(R, K, dtype=torch.int32, device=DEV)
    out_pool = torch.empty(R, pool_size, dtype=torch.int32, device=DEV) if pool_size else None
    out_len = torch.empty(R, dtype=torch.int32, device=DEV) if pool_size else None
    csa2.index_topk(mode, idx_q, idx_k, starts, vis, max_visible, K, idx, ws, pool=pool, pool_len=pool_len,
                    pool_size=pool_size, out_pool=out_pool, out_pool_len=out_len)
    return idx, out_pool, out_len


def attention(q, codes, scales, starts, idx, scale, vis=None, out_dtype=torch.float32):
    R, Hq, _ = q.shape
    qdt = csa2.F32 if q.dtype == torch.float32 else csa2.BF16
    ws = torch.zeros(max(256, csa2.sparse_attn_workspace_size(R, Hq, qdt, idx.shape[1])), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty(R, Hq, 512, dtype=out_dtype, device=DEV)
    lse = torch.empty(R, Hq, dtype=torch.float32, device=DEV)
    csa2.sparse_attn(q, codes, scales, starts, idx, out, scale, row_visible=vis, lse=lse, workspace=ws)
    return out, lse


def attn_error(o: np.ndarray, ref: np.ndarray) -> float:
    """Largest per-(row, head) max|o - ref| / max|ref|; rows with ref == 0 must be exactly 0."""
    o = o.reshape(-1, o.shape[-1]).astype(np.float64)
    ref = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    den = np.abs(ref).max(1)
    num = np.abs(o - ref).max(1)
    zero = den == 0
    if np.any(num[zero] != 0):
        return float("inf")
    return float((num[~zero] / den[~zero]).max()) if np.any(~zero) else 0.0


def check_attention(o: torch.Tensor, lse: torch.Tensor, ref_o: np.ndarray, ref_lse: np.ndarray, label: str):
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    err = attn_error(o, ref_o)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin), label + ": lse finiteness differs"
    lerr = float(np.abs(lse[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    say("%s: attention max rel err %.3e, lse max abs err %.3e" % (label, err, lerr))
    assert err <= TOL, "%s: attention error %g > %g" % (label, err, TOL)
    assert lerr <= 1e-3, "%s: lse error %g" % (label, lerr)
    return err
