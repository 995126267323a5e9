"""ctypes binding of libcsa2.so (the C ABI in include/csa2.h).

Argument marshalling only: torch tensors supply device pointers, the
current HIP stream is passed through, and every non-zero status raises
``CSA2Error`` with the library's message.  All arithmetic runs in the HIP
kernels of libcsa2.so; there is no other path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcsa2.so")

F32, BF16, MXFP4 = 0, 1, 2
FULL, REINDEX, FULL_SHARED = 0, 1, 2
MAX_TOP_K = 4096
KERNEL_QUANT, KERNEL_INDEX_SCAN, KERNEL_REINDEX_SCORE, KERNEL_ATTN, KERNEL_ATTN_COMBINE = 1, 2, 3, 4, 5
KERNEL_QUANT_FP8, KERNEL_SWA_ATTN, KERNEL_QUANT_MXFP4 = 6, 7, 8
SWA_WINDOW = 128
EXPORTED = (
    "csa2_quantize_kv_fp4",
    "csa2_index_topk",
    "csa2_index_topk_workspace_size",
    "csa2_sparse_attn",
    "csa2_sparse_attn_workspace_size",
    "csa2_sparse_attn_noalloc",
    "csa2_quantize_swa_fp8",
    "csa2_quantize_idx_mxfp4",
    "csa2_index_topk_mxfp4",
    "csa2_sparse_attn_swa",
    "csa2_sparse_attn_swa_workspace_size",
    "csa2_visible_entries",
    "csa2_last_error",
    "csa2_profile_kernel_events",
)

_LIB = None


class CSA2Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("csa2 status %d: %s" % (code, msg))
        self.code = code


def lib():
    """Load libcsa2.so; raises if it has not been built (no fallback exists)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libcsa2.so is not built; run __graft_entry__.build() or "
                              "python sparse_attention_fp4_e4m3_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.csa2_quantize_kv_fp4.argtypes = [P, i32, i64, i64, P, P, P, i64, P]
        L.csa2_quantize_kv_fp4.restype = i32
        L.csa2_index_topk.argtypes = [i32, i32, P, i32, i32, i32, P, i32, i32, P, P, i32, P, P, i32, i32, P, i32,
                                      i32, P, P, P, sz, P]
        L.csa2_index_topk.restype = i32
        L.csa2_index_topk_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.csa2_index_topk_workspace_size.restype = sz
        L.csa2_sparse_attn.argtypes = [i32, P, i32, i32, i32, P, P, P, P, i32, P, ctypes.c_float, P, i32, P, P, sz, P]
        L.csa2_sparse_attn.restype = i32
        L.csa2_sparse_attn_workspace_size.argtypes = [i32, i32, i32, i32]
        L.csa2_sparse_attn_workspace_size.restype = sz
        L.csa2_sparse_attn_noalloc.argtypes = [i32, P, i32, i32, i32, P, P, P, P, i32, P, ctypes.c_float, P, i32, P,
                                               P]
        L.csa2_sparse_attn_noalloc.restype = i32
        L.csa2_quantize_idx_mxfp4.argtypes = [P, i32, i64, i64, P, P, P, i64, P]
        L.csa2_quantize_idx_mxfp4.restype = i32
        L.csa2_index_topk_mxfp4.argtypes = [i32, i32, P, i32, i32, i32, P, P, i32, P, P, i32, P, P, i32, i32, P,
                                            i32, i32, P, P, P, sz, P]
        L.csa2_index_topk_mxfp4.restype = i32
        L.csa2_quantize_swa_fp8.argtypes = [P, i32, i64, i64, P, P, i64, P]
        L.csa2_quantize_swa_fp8.restype = i32
        L.csa2_sparse_attn_swa.argtypes = [i32, P, i32, i32, i32, P, P, P, P, i32, P, P, P, P, P, i32, i64, P,
                                           ctypes.c_float, P, i32, P, P, sz, P]
        L.csa2_sparse_attn_swa.restype = i32
        L.csa2_sparse_attn_swa_workspace_size.argtypes = [i32, i32, i32, i32]
        L.csa2_sparse_attn_swa_workspace_size.restype = sz
        L.csa2_visible_entries.argtypes = [P, i32, i32, P, P]
        L.csa2_visible_entries.restype = i32
        L.csa2_last_error.argtypes = []
        L.csa2_last_error.restype = ctypes.c_char_p
        L.csa2_profile_kernel_events.argtypes = [i32, P, P]
        L.csa2_profile_kernel_events.restype = i32
        _LIB = L
    return _LIB


def _check(code: int):
    if code != 0:
        raise CSA2Error(code, lib().csa2_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("expected float32 or bfloat16, got %s" % t.dtype)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def quantize_kv_fp4(x: torch.Tensor, kv_codes: torch.Tensor, kv_scales: torch.Tensor,
                    dst_rows: Optional[torch.Tensor] = None, stream=None) -> None:
    """x [n, 512(+)] fp32/bf16 -> FP4 rows of kv_codes [cap, 256] u8 / kv_scales [cap, 32] u8."""
    _contig(kv_codes, kv_scales, dst_rows)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [n, C] with unit channel stride")
    _check(lib().csa2_quantize_kv_fp4(_ptr(x), _dt(x), x.shape[0], x.stride(0), _ptr(dst_rows),
                                      _ptr(kv_codes), _ptr(kv_scales), kv_codes.shape[0], _stream(stream)))


def index_topk_workspace_size(mode: int, n_rows: int, n_heads: int, max_visible: int, pool_stride: int,
                              top_k: int, pool_size: int) -> int:
    return int(lib().csa2_index_topk_workspace_size(mode, n_rows, n_heads, max_visible, pool_stride, top_k,
                                                    pool_size))


def index_topk(mode: int, idx_q: torch.Tensor, idx_k: torch.Tensor, row_kv_start: torch.Tensor,
               row_visible: torch.Tensor, max_visible: int, top_k: int, out_idx: torch.Tensor,
               workspace: torch.Tensor, pool: Optional[torch.Tensor] = None,
               pool_len: Optional[torch.Tensor] = None, pool_size: int = 0,
               out_pool: Optional[torch.Tensor] = None, out_pool_len: Optional[torch.Tensor] = None,
               stream=None) -> None:
    """Indexer scores + exact top-K (and the HSI pool in Full mode)."""
    _contig(idx_q, idx_k, row_kv_start, row_visible, out_idx, workspace, pool, pool_len, out_pool, out_pool_len)
    R, H, Dk = idx_q.shape
    pool_stride = pool.shape[1] if pool is not None else 0
    _check(lib().csa2_index_topk(
        mode, R, _ptr(idx_q), _dt(idx_q), H, Dk, _ptr(idx_k), _dt(idx_k), 1, _ptr(row_kv_start), _ptr(row_visible),
        int(max_visible), _ptr(pool), _ptr(pool_len), pool_stride, top_k, _ptr(out_idx), pool_size,
        8 if pool_size else 0, _ptr(out_pool), _ptr(out_pool_len), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def quantize_idx_mxfp4(x: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor,
                       dst_rows: Optional[torch.Tensor] = None, stream=None) -> None:
    """Indexer keys x [n, 64(+)] fp32/bf16 -> OCP MXFP4 rows of k_codes [cap, 32] u8 / k_scales [cap, 2] u8."""
    _contig(k_codes, k_scales, dst_rows)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [n, C] with unit channel stride")
    _check(lib().csa2_quantize_idx_mxfp4(_ptr(x), _dt(x), x.shape[0], x.stride(0), _ptr(dst_rows), _ptr(k_codes),
                                         _ptr(k_scales), k_codes.shape[0], _stream(stream)))


def index_topk_mxfp4(mode: int, idx_q: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor,
                     row_kv_start: torch.Tensor, row_visible: torch.Tensor, max_visible: int, top_k: int,
                     out_idx: torch.Tensor, workspace: torch.Tensor, pool: Optional[torch.Tensor] = None,
                     pool_len: Optional[torch.Tensor] = None, pool_size: int = 0,
                     out_pool: Optional[torch.Tensor] = None, out_pool_len: Optional[torch.Tensor] = None,
                     stream=None) -> None:
    """index_topk over MXFP4 indexer keys (k_codes [rows, 32], k_scales [rows, 2])."""
    _contig(idx_q, k_codes, k_scales, row_kv_start, row_visible, out_idx, workspace, pool, pool_len, out_pool,
            out_pool_len)
    R, H, Dk = idx_q.shape
    pool_stride = pool.shape[1] if pool is not None else 0
    _check(lib().csa2_index_topk_mxfp4(
        mode, R, _ptr(idx_q), _dt(idx_q), H, Dk, _ptr(k_codes), _ptr(k_scales), 1, _ptr(row_kv_start),
        _ptr(row_visible), int(max_visible), _ptr(pool), _ptr(pool_len), pool_stride, top_k, _ptr(out_idx),
        pool_size, 8 if pool_size else 0, _ptr(out_pool), _ptr(out_pool_len), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def sparse_attn_workspace_size(n_rows: int, n_heads: int, q_dtype: int, top_k: int) -> int:
    return int(lib().csa2_sparse_attn_workspace_size(n_rows, n_heads, q_dtype, top_k))


def sparse_attn(q: torch.Tensor, kv_codes: torch.Tensor, kv_scales: torch.Tensor, row_kv_start: torch.Tensor,
                idx: torch.Tensor, out: torch.Tensor, softmax_scale: float,
                row_visible: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Gather + dequant + softmax attention over the selected entries."""
    _contig(q, kv_codes, kv_scales, row_kv_start, idx, out, row_visible, lse, workspace)
    R, Hq, D = q.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().csa2_sparse_attn(
        R, _ptr(q), _dt(q), Hq, D, _ptr(kv_codes), _ptr(kv_scales), _ptr(row_kv_start), _ptr(idx),
        idx.shape[1], _ptr(row_visible), float(softmax_scale), _ptr(out), _dt(out), _ptr(lse), _ptr(workspace),
        ws_bytes, _stream(stream)))


def sparse_attn_noalloc(q: torch.Tensor, kv_codes: torch.Tensor, kv_scales: torch.Tensor, row_kv_start: torch.Tensor,
                        idx: torch.Tensor, out: torch.Tensor, softmax_scale: float,
                        row_visible: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                        stream=None) -> None:
    """sparse_attn with the library's own scratch instead of a workspace (nothing is allocated;
    calls on one device share that scratch and must not overlap)."""
    _contig(q, kv_codes, kv_scales, row_kv_start, idx, out, row_visible, lse)
    R, Hq, D = q.shape
    _check(lib().csa2_sparse_attn_noalloc(
        R, _ptr(q), _dt(q), Hq, D, _ptr(kv_codes), _ptr(kv_scales), _ptr(row_kv_start), _ptr(idx),
        idx.shape[1], _ptr(row_visible), float(softmax_scale), _ptr(out), _dt(out), _ptr(lse), _stream(stream)))


def quantize_swa_fp8(x: torch.Tensor, win_codes: torch.Tensor, dst_rows: Optional[torch.Tensor] = None,
                    stream=None) -> None:
    """x [n, 512(+)] fp32/bf16 -> signed E4M3 rows of win_codes [cap, 512] u8."""
    _contig(win_codes, dst_rows)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [n, C] with unit channel stride")
    _check(lib().csa2_quantize_swa_fp8(_ptr(x), _dt(x), x.shape[0], x.stride(0), _ptr(dst_rows), _ptr(win_codes),
                                       win_codes.shape[0], _stream(stream)))


def sparse_attn_swa_workspace_size(n_rows: int, n_heads: int, q_dtype: int, top_k: int) -> int:
    return int(lib().csa2_sparse_attn_swa_workspace_size(n_rows, n_heads, q_dtype, top_k))


def sparse_attn_swa(q: torch.Tensor, win_codes: torch.Tensor, row_win_start: torch.Tensor,
                    row_win_len: torch.Tensor, out: torch.Tensor, softmax_scale: float,
                    kv_codes: Optional[torch.Tensor] = None, kv_scales: Optional[torch.Tensor] = None,
                    row_kv_start: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                    row_visible: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, new_x: Optional[torch.Tensor] = None,
                    new_rows: Optional[torch.Tensor] = None, stream=None) -> None:
    """Selected FP4 entries (idx; None = window only) joined with each row's FP8 window in one softmax;
    new_x [R, 512(+)] / new_rows [R]: each row's newest token, written into its window by the same call."""
    _contig(q, win_codes, row_win_start, row_win_len, out, kv_codes, kv_scales, row_kv_start, idx, row_visible, lse,
            workspace, new_rows)
    if new_x is not None and (new_x.dim() != 2 or new_x.stride(1) != 1):
        raise ValueError("new_x must be [R, C] with unit channel stride")
    R, Hq, D = q.shape
    top_k = 0 if idx is None else idx.shape[1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().csa2_sparse_attn_swa(
        R, _ptr(q), _dt(q), Hq, D, _ptr(kv_codes), _ptr(kv_scales), _ptr(row_kv_start), _ptr(idx), top_k,
        _ptr(row_visible), _ptr(win_codes), _ptr(row_win_start), _ptr(row_win_len), _ptr(new_x),
        _dt(new_x) if new_x is not None else 0, new_x.stride(0) if new_x is not None else 0, _ptr(new_rows),
        float(softmax_scale), _ptr(out),
        _dt(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def visible_entries(token_pos: torch.Tensor, tokens_per_entry: int, row_visible: torch.Tensor,
                    stream=None) -> None:
    """row_visible [R] int32 <- entries visible at token positions token_pos [R] int64 when each
    entry folds tokens_per_entry tokens (computed by the library on the device)."""
    _contig(token_pos, row_visible)
    if token_pos.dtype != torch.int64 or row_visible.dtype != torch.int32 or token_pos.shape != row_visible.shape:
        raise ValueError("token_pos must be int64 and row_visible int32 of the same shape")
    _check(lib().csa2_visible_entries(_ptr(token_pos), int(tokens_per_entry), token_pos.numel(), _ptr(row_visible),
                                      _stream(stream)))


def profile_kernel_events(kernel_id: int, start=None, stop=None) -> None:
    """Record torch.cuda.Event pairs around every launch of one kernel (None stops)."""
    s = None if start is None else ctypes.c_void_p(start.cuda_event)
    e = None if stop is None else ctypes.c_void_p(stop.cuda_event)
    _check(lib().csa2_profile_kernel_events(kernel_id, s, e))
