"""Workload descriptions and chunk-addressable seeded generators.

Every array is drawn from numpy's PCG64 (``default_rng``) keyed by a
``SeedSequence`` of ``(seed, stream tag, sequence, chunk)``.  Because each
chunk of ``CHUNK`` tokens has its own key, any token range of any sequence
can be regenerated on its own and always yields the same bytes, whatever
range or thread order asked for it.  That lets the GPU side stream a cache
into device memory chunk by chunk while the CPU oracle regenerates only the
rows it checks.

The five workloads follow the configurations the method is measured on:

* ``c1`` tiny decode, Full mode: batch 1 over 4,096 cached tokens, fp32.
* ``c2`` decode, Full mode: batch 32, per-sequence context uniform on
  [32,768, 65,536], 1 % of KV channels scaled x20, bf16.
* ``c3`` six-layer chain over 128K tokens, batch 16: Full (with an 8,192
  candidate pool), two Reindex layers, three Reuse layers.
* ``c4`` prefill chunk: 4,096 new tokens appended causally to 262,144 cached
  tokens, per-query top-2,048.
* ``c5`` long-context decode: batch 4 at 1,048,576 tokens, keys drifting as
  a random walk (sigma 0.01 per token); Full (pool 16,384), Reindex, Reuse.

Readings taken where the configuration text is silent are listed in the
design notes (seeds 1, 2, 4 for c2/c3/c5; q ~ N(0,1) in bf16 for c2-c5;
5 = floor(1 % of 512) outlier channels drawn once per seed; the random walk
applies independently per sequence and channel to both the KV latent and
the indexer keys).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import List, Optional, Sequence

import numpy as np

D = 512  # channels of the shared KV latent
D_I = 64  # indexer head dimension
CHUNK = 4096  # tokens per generator chunk

# stream tags of the seed sequence
_T_KV, _T_IK, _T_WTOT_KV, _T_WTOT_IK, _T_WKV, _T_WIK = 1, 2, 3, 4, 5, 6
_T_LEN, _T_OUTLIER = 7, 8
_T_Q, _T_IQ, _T_WIN = 100, 200, 300

_POOL = None


def _pool() -> ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        import os

        _POOL = ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1)))
    return _POOL


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bfloat16, returned as fp32."""
    return (bf16_bits(x).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Layer:
    mode: str  # "full" | "reindex" | "reuse"
    pool_size: int = 0  # Full only: HSI candidate pool size (0 = none)


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    B: int  # sequences (decode) or 1 (prefill)
    n: int  # cached tokens per sequence (upper bound when lens vary)
    Hq: int  # attention query heads
    q_dtype: str  # "f32" | "bf16"
    q_std: float
    H: int  # indexer heads
    idx_dtype: str  # "f32" | "bf16"
    K: int  # top-K
    seed: int
    layers: Sequence[Layer]
    len_range: Optional[tuple] = None  # (lo, hi) inclusive, uniform per sequence
    outlier_channels: int = 0
    outlier_gain: float = 1.0
    drift_sigma: float = 0.0
    prefill_tokens: int = 0  # >0: prefill chunk of this many new tokens at the end
    verify: int = 1  # decode query rows per sequence: the last `verify` cached tokens are drafts, checked in one pass
    block: int = 8  # HSI block size

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(D)

    @property
    def is_prefill(self) -> bool:
        return self.prefill_tokens > 0

    @property
    def rows(self) -> int:
        """Query rows per layer: sequences (x draft rows) for decode, chunk tokens for prefill."""
        return self.prefill_tokens if self.is_prefill else self.B * self.verify

    def scaled(self, **kw) -> "Workload":
        """The same distributions at other sizes (for oracle-sized parity runs)."""
        return replace(self, **kw)


WORKLOADS = {
    "c1": Workload(
        name="c1", description="tiny decode, Full: B=1, n=4096, 16 fp32 heads, indexer 4x64 fp32, K=256",
        B=1, n=4096, Hq=16, q_dtype="f32", q_std=1.0 / math.sqrt(D), H=4, idx_dtype="f32",
        K=256, seed=0, layers=(Layer("full"),)),
    "c2": Workload(
        name="c2", description="decode, Full: B=32, n~U[32K,64K], 64 bf16 heads, indexer 8x64 bf16, K=2048, 1% channels x20",
        B=32, n=65536, Hq=64, q_dtype="bf16", q_std=1.0, H=8, idx_dtype="bf16",
        K=2048, seed=1, layers=(Layer("full"),), len_range=(32768, 65536),
        outlier_channels=5, outlier_gain=20.0),
    "c3": Workload(
        name="c3", description="6-layer chain at 128K, B=16: Full(pool 8192), 2x Reindex, 3x Reuse",
        B=16, n=131072, Hq=64, q_dtype="bf16", q_std=1.0, H=8, idx_dtype="bf16",
        K=2048, seed=2,
        layers=(Layer("full", 8192), Layer("reindex"), Layer("reindex"),
                Layer("reuse"), Layer("reuse"), Layer("reuse"))),
    "c4": Workload(
        name="c4", description="prefill 4096 tokens onto 256K cached (n=266240), causal top-2048",
        B=1, n=262144 + 4096, Hq=64, q_dtype="bf16", q_std=1.0, H=8, idx_dtype="bf16",
        K=2048, seed=3, layers=(Layer("full"),), prefill_tokens=4096),
    "c3v": Workload(
        name="c3v", description="the 128K chain checking 5 draft tokens per sequence in one pass: 80 query rows",
        B=16, n=131072, Hq=64, q_dtype="bf16", q_std=1.0, H=8, idx_dtype="bf16",
        K=2048, seed=2, verify=5,
        layers=(Layer("full", 8192), Layer("reindex"), Layer("reindex"),
                Layer("reuse"), Layer("reuse"), Layer("reuse"))),
    "c5": Workload(
        name="c5", description="long decode at 1M, B=4, drifting keys: Full(pool 16384), Reindex, Reuse",
        B=4, n=1048576, Hq=64, q_dtype="bf16", q_std=1.0, H=8, idx_dtype="bf16",
        K=2048, seed=4,
        layers=(Layer("full", 16384), Layer("reindex"), Layer("reuse")),
        drift_sigma=0.01),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def seq_lens(w: Workload) -> np.ndarray:
    """Cached tokens per sequence (int64 [B])."""
    if w.len_range is None:
        return np.full(w.B, w.n, dtype=np.int64)
    lo, hi = w.len_range
    return _rng(w.seed, _T_LEN).integers(lo, hi + 1, size=w.B, dtype=np.int64)


def _outlier_channels(w: Workload) -> np.ndarray:
    return np.sort(_rng(w.seed, _T_OUTLIER).choice(D, w.outlier_channels, replace=False))


def _walk_chunk(w: Workload, tag_tot: int, tag_inc: int, b: int, chunk: int, ch: int) -> np.ndarray:
    """Random-walk means of the CHUNK tokens of one chunk (float64 [CHUNK, ch]).

    The chunk totals are drawn first (one normal per chunk and channel with
    variance sigma^2 * CHUNK); inside a chunk the per-token increments are
    drawn and conditioned on that total (subtract their mean, add
    total / CHUNK), which is an exact draw of Gaussian increments given
    their sum.  Any chunk can thus be generated without its predecessors.
    """
    n_chunks = (w.n + CHUNK - 1) // CHUNK
    tot = _rng(w.seed, tag_tot, b).standard_normal((n_chunks, ch)) * (w.drift_sigma * math.sqrt(CHUNK))
    start = tot[:chunk].sum(axis=0)
    inc = _rng(w.seed, tag_inc, b, chunk).standard_normal((CHUNK, ch)) * w.drift_sigma
    inc = inc - inc.mean(axis=0, keepdims=True) + tot[chunk] / CHUNK
    return start + np.cumsum(inc, axis=0)


def _kv_chunk(w: Workload, b: int, chunk: int) -> np.ndarray:
    x = _rng(w.seed, _T_KV, b, chunk).standard_normal((CHUNK, D), dtype=np.float32)
    if w.outlier_channels:
        x[:, _outlier_channels(w)] *= np.float32(w.outlier_gain)
    if w.drift_sigma:
        x = (x + _walk_chunk(w, _T_WTOT_KV, _T_WKV, b, chunk, D)).astype(np.float32)
    return x


def _ik_chunk(w: Workload, b: int, chunk: int) -> np.ndarray:
    x = _rng(w.seed, _T_IK, b, chunk).standard_normal((CHUNK, D_I), dtype=np.float32)
    if w.drift_sigma:
        x = (x + _walk_chunk(w, _T_WTOT_IK, _T_WIK, b, chunk, D_I)).astype(np.float32)
    if w.idx_dtype == "bf16":
        x = bf16_round(x)
    return x


def _rows(w: Workload, fn, b: int, t0: int, t1: int, ch: int, threads: bool) -> np.ndarray:
    out = np.empty((t1 - t0, ch), dtype=np.float32)
    if t1 <= t0:
        return out
    chunks = range(t0 // CHUNK, (t1 - 1) // CHUNK + 1)

    def fill(c):
        blk = fn(w, b, c)
        lo, hi = max(t0, c * CHUNK), min(t1, (c + 1) * CHUNK)
        out[lo - t0:hi - t0] = blk[lo - c * CHUNK:hi - c * CHUNK]

    if threads and len(chunks) > 1:
        list(_pool().map(fill, chunks))
    else:
        for c in chunks:
            fill(c)
    return out


def kv_rows(w: Workload, b: int, t0: int, t1: int, threads: bool = True) -> np.ndarray:
    """Raw (unquantized) KV latents of tokens [t0, t1) of sequence b: fp32 [t1-t0, 512]."""
    return _rows(w, _kv_chunk, b, t0, t1, D, threads)


def idx_k_rows(w: Workload, b: int, t0: int, t1: int, threads: bool = True) -> np.ndarray:
    """Indexer keys of tokens [t0, t1) of sequence b: fp32 [t1-t0, 64] (bf16-exact if bf16)."""
    return _rows(w, _ik_chunk, b, t0, t1, D_I, threads)


def _win_chunk(w: Workload, layer: int, b: int, chunk: int) -> np.ndarray:
    x = _rng(w.seed, _T_WIN + layer, b, chunk).standard_normal((CHUNK, D), dtype=np.float32)
    if w.outlier_channels:
        x[:, _outlier_channels(w)] *= np.float32(w.outlier_gain)
    return x


def window_rows(w: Workload, layer: int, b: int, t0: int, t1: int, threads: bool = True) -> np.ndarray:
    """Local sliding-window latents of one layer, tokens [t0, t1) of sequence b: fp32 [t1-t0, 512].

    Each layer has its own window (its own hidden state), drawn like the
    KV latents (N(0, 1), the same outlier channels) from its own stream.
    """
    return _rows(w, lambda w_, b_, c: _win_chunk(w_, layer, b_, c), b, t0, t1, D, threads)


def attn_q(w: Workload, layer: int, r0: int = 0, r1: Optional[int] = None) -> np.ndarray:
    """Attention queries of one layer for rows [r0, r1): fp32 [rows, Hq, 512].

    Row r's values depend only on (seed, layer, r), so any row range can be
    regenerated on its own.
    """
    r1 = w.rows if r1 is None else r1
    out = np.empty((r1 - r0, w.Hq, D), dtype=np.float32)
    for r in range(r0, r1):
        out[r - r0] = _rng(w.seed, _T_Q + layer, r).standard_normal((w.Hq, D), dtype=np.float32) * np.float32(w.q_std)
    if w.q_dtype == "bf16":
        out = bf16_round(out)
    return out


def index_q(w: Workload, layer: int, r0: int = 0, r1: Optional[int] = None) -> np.ndarray:
    """Indexer queries of one layer for rows [r0, r1): fp32 [rows, H, 64]."""
    r1 = w.rows if r1 is None else r1
    out = np.empty((r1 - r0, w.H, D_I), dtype=np.float32)
    for r in range(r0, r1):
        out[r - r0] = _rng(w.seed, _T_IQ + layer, r).standard_normal((w.H, D_I), dtype=np.float32)
    if w.idx_dtype == "bf16":
        out = bf16_round(out)
    return out
