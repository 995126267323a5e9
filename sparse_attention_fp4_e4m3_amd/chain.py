"""Static layer-mode chains over one FP4 cache.

Each CSA2 layer is statically Full, Reindex or Reuse (course brief
"DeepSeek-V4.1-Flash", "CSA2: most layers don't keep their own cache": the
mode table and the released layer layout; talk write-up "DeepSeek V4.1
Flash: pushing the limits", "The Paper": the first global layer has to be
Full because there is nothing to reuse yet).  Rules enforced here:

* the first layer of a chain is Full;
* Reindex re-scores the candidate pool of the most recent Full layer with
  its own indexer query, so that Full layer must emit a pool;
* Reuse takes the selection of the most recent Full or Reindex layer;
* every layer attends with its own query;
* with local windows, every layer also attends over its own FP8 window of
  the most recent tokens, joined to its selected entries in one softmax
  ("The Paper" in the talk write-up; "Two attention paths in every layer"
  in the course brief).

The driver only sequences the three library calls on one stream; all
arithmetic happens in libcsa2.so.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

from . import csa2


@dataclass
class Cache:
    """A packed FP4 cache and its indexer keys (device tensors)."""
    kv_codes: torch.Tensor      # [rows, 256] uint8
    kv_scales: torch.Tensor     # [rows, 32] uint8
    idx_k: torch.Tensor         # [rows, 64] bf16 / fp32, or MXFP4 codes [rows, 32] uint8
    row_kv_start: torch.Tensor  # [R] int64
    row_visible: torch.Tensor   # [R] int32
    max_visible: int
    shared_segment: bool = False  # every row reads the segment at row_kv_start[0] (a prefill chunk)
    idx_k_scales: Optional[torch.Tensor] = None  # [rows, 2] uint8 E8M0: the indexer keys are MXFP4


@dataclass
class Window:
    """One layer's local window cache (device tensors): FP8 entries and each row's window."""
    codes: torch.Tensor         # [rows, 512] uint8, signed E4M3 per channel
    row_start: torch.Tensor     # [R] int64 first window entry of each query row
    row_len: torch.Tensor       # [R] int32 window entries of each query row (<= 128)


@dataclass(frozen=True)
class LayerSpec:
    mode: str                   # "full" | "reindex" | "reuse"
    pool_size: int = 0          # Full only


def compressed_visible(token_pos: torch.Tensor, m: int, stream=None) -> torch.Tensor:
    """row_visible for query rows at token positions token_pos ([R] int64, device) when each cache
    entry folds m consecutive tokens: the library counts the complete blocks on the device."""
    out = torch.empty(token_pos.shape, dtype=torch.int32, device=token_pos.device)
    csa2.visible_entries(token_pos, m, out, stream=stream)
    return out


def validate_modes(layers: Sequence[LayerSpec]) -> None:
    have_full = have_pool = have_sel = False
    for i, L in enumerate(layers):
        if L.mode == "full":
            have_full, have_sel = True, True
            have_pool = L.pool_size > 0
        elif L.mode == "reindex":
            if not have_full:
                raise ValueError("layer %d: Reindex before any Full layer" % i)
            if not have_pool:
                raise ValueError("layer %d: Reindex needs the most recent Full layer to emit a pool" % i)
            have_sel = True
        elif L.mode == "reuse":
            if not have_sel:
                raise ValueError("layer %d: Reuse before any Full/Reindex selection" % i)
        else:
            raise ValueError("layer %d: unknown mode %r" % (i, L.mode))
        if L.mode != "full" and L.pool_size:
            raise ValueError("layer %d: only Full layers emit a pool" % i)
    if layers and layers[0].mode != "full":
        raise ValueError("the first layer must be Full")


class LayerChain:
    """Runs a fixed mode sequence for R query rows over one cache."""

    def __init__(self, layers: Sequence[LayerSpec], n_rows: int, n_heads: int, idx_heads: int, top_k: int,
                 max_visible: int, q_dtype: torch.dtype, device="cuda", out_dtype=torch.float32,
                 shared_segment: bool = False, swa: bool = False):
        validate_modes(layers)
        self.swa = swa
        self.layers = list(layers)
        self.full_mode = csa2.FULL_SHARED if shared_segment else csa2.FULL
        self.R, self.Hq, self.H, self.K = n_rows, n_heads, idx_heads, top_k
        self.max_visible = max_visible
        dev = torch.device(device)
        self.idx = [torch.empty(n_rows, top_k, dtype=torch.int32, device=dev) if L.mode != "reuse" else None
                    for L in self.layers]
        self.pool = {}
        ws = 0
        last_pool = 0
        for i, L in enumerate(self.layers):
            if L.mode == "full":
                ws = max(ws, csa2.index_topk_workspace_size(self.full_mode, n_rows, idx_heads, max_visible, 0,
                                                            top_k, L.pool_size))
                last_pool = L.pool_size
                if L.pool_size:
                    self.pool[i] = (torch.empty(n_rows, L.pool_size, dtype=torch.int32, device=dev),
                                    torch.empty(n_rows, dtype=torch.int32, device=dev))
            elif L.mode == "reindex":
                ws = max(ws, csa2.index_topk_workspace_size(csa2.REINDEX, n_rows, idx_heads, max_visible,
                                                            last_pool, top_k, 0))
        qdt = csa2.F32 if q_dtype == torch.float32 else csa2.BF16
        aws = (csa2.sparse_attn_swa_workspace_size if swa else csa2.sparse_attn_workspace_size)(n_rows, n_heads, qdt,
                                                                                                top_k)
        self.ws_index = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.ws_attn = torch.zeros(max(aws, 256), dtype=torch.uint8, device=dev)  # split-merge counters start at 0
        self.out = [torch.empty(n_rows, n_heads, 512, dtype=out_dtype, device=dev) for _ in self.layers]
        self.lse = [torch.empty(n_rows, n_heads, dtype=torch.float32, device=dev) for _ in self.layers]

    def step(self, cache: Cache, q: List[torch.Tensor], idx_q: List[Optional[torch.Tensor]], softmax_scale: float,
             new_kv: Optional[torch.Tensor] = None, new_kv_rows: Optional[torch.Tensor] = None,
             windows: Optional[List[Window]] = None, new_win: Optional[List[torch.Tensor]] = None,
             new_win_rows: Optional[torch.Tensor] = None, stream=None):
        """One pass of every layer.  q[l]: [R, Hq, 512]; idx_q[l]: [R, H, 64] for Full/Reindex layers.
        new_kv/new_kv_rows: tokens the first Full layer writes into the cache before indexing.
        windows[l] (chains built with swa=True): layer l's window; new_win[l]/new_win_rows: the
        tokens layer l writes into its window before attending."""
        if self.swa != (windows is not None):
            raise ValueError("windows must be given exactly when the chain was built with swa=True")
        last_full_pool = None
        last_sel = None
        if cache.idx_k_scales is not None:
            def topk(mode, iq, out, **kw):
                csa2.index_topk_mxfp4(mode, iq, cache.idx_k, cache.idx_k_scales, cache.row_kv_start,
                                      cache.row_visible, cache.max_visible, self.K, out, self.ws_index,
                                      stream=stream, **kw)
        else:
            def topk(mode, iq, out, **kw):
                csa2.index_topk(mode, iq, cache.idx_k, cache.row_kv_start, cache.row_visible, cache.max_visible,
                                self.K, out, self.ws_index, stream=stream, **kw)
        for i, L in enumerate(self.layers):
            if L.mode == "full":
                if new_kv is not None and i == 0:
                    csa2.quantize_kv_fp4(new_kv, cache.kv_codes, cache.kv_scales, new_kv_rows, stream=stream)
                pool, plen = self.pool.get(i, (None, None))
                topk(self.full_mode, idx_q[i], self.idx[i], pool_size=L.pool_size, out_pool=pool, out_pool_len=plen)
                last_full_pool = (pool, plen)
                last_sel = self.idx[i]
            elif L.mode == "reindex":
                pool, plen = last_full_pool
                topk(csa2.REINDEX, idx_q[i], self.idx[i], pool=pool, pool_len=plen)
                last_sel = self.idx[i]
            if windows is None:
                csa2.sparse_attn(q[i], cache.kv_codes, cache.kv_scales, cache.row_kv_start, last_sel, self.out[i],
                                 softmax_scale, row_visible=cache.row_visible, lse=self.lse[i],
                                 workspace=self.ws_attn, stream=stream)
                continue
            win = windows[i]
            # one window per row (decode): the attention call writes each row's token itself; a
            # chunk's rows share overlapping windows, so its tokens are written first
            fused = new_win is not None and not cache.shared_segment
            if new_win is not None and not fused:
                csa2.quantize_swa_fp8(new_win[i], win.codes, new_win_rows, stream=stream)
            csa2.sparse_attn_swa(q[i], win.codes, win.row_start, win.row_len, self.out[i], softmax_scale,
                                 kv_codes=cache.kv_codes, kv_scales=cache.kv_scales, row_kv_start=cache.row_kv_start,
                                 idx=last_sel, row_visible=cache.row_visible, lse=self.lse[i],
                                 workspace=self.ws_attn, new_x=new_win[i] if fused else None,
                                 new_rows=new_win_rows if fused else None, stream=stream)
        return self.out
