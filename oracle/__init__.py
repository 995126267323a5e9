"""CPU oracle for CSA2 sparse attention over an FP4 (E2M1 + per-16 E4M3) KV cache.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the benchmark's ``cpu_baseline`` leg may import this package.  The
product path (``sparse_attention_fp4_e4m3_amd``) never imports it and shares
no code with it.

The arithmetic lives in ``csa2_oracle.c`` (plain C, built with gcc, fp32
operations fixed by ``-ffp-contract=off``; attention in double).  This module
is argument marshalling plus the per-mode compositions, which follow the
mode table of the course brief "DeepSeek-V4.1-Flash", section "CSA2: most
layers don't keep their own cache", and the three-mode description of the
metallab.ai article:

* Full: quantize the written rows, score every visible entry, keep the
  top-K (and, for the first Full layer, the hierarchical candidate pool),
  attend.
* Reindex: score only the pool entries with this layer's indexer query,
  keep the top-K, attend.
* Reuse: attend over the indices handed down.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libcsa2_oracle.so")
_LIB = None

D = 512
NG = 32

CFLAGS = ["-O2", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c99"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (the checker, not the product)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _lib():
    global _LIB
    if _LIB is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        sig = {
            "oracle_e2m1_value": (f64, [ctypes.c_uint8]),
            "oracle_e4m3_value": (f64, [ctypes.c_uint8]),
            "oracle_e4m3_encode": (ctypes.c_uint8, [ctypes.c_float]),
            "oracle_e2m1_encode": (ctypes.c_uint8, [ctypes.c_float]),
            "oracle_e4m3_encode_array": (None, [P, i64, P]),
            "oracle_e2m1_encode_array": (None, [P, i64, P]),
            "oracle_quantize_rows": (None, [P, i64, i64, P, P]),
            "oracle_dequant_rows": (None, [P, P, i64, P]),
            "oracle_index_scores": (None, [P, i32, i32, P, i64, i64, P]),
            "oracle_topk": (i64, [P, P, i64, i32, P]),
            "oracle_hsi_pool": (i64, [P, i64, i32, i32, P]),
            "oracle_attention_row": (None, [P, i32, P, P, P, i32, i64, f64, P, P]),
            "oracle_attention_rows": (None, [i32, P, i32, P, P, P, P, i32, P, f64, P, P]),
            "oracle_e4m3_encode_signed": (ctypes.c_uint8, [ctypes.c_float]),
            "oracle_e8m0_value": (f64, [ctypes.c_uint8]),
            "oracle_mxfp4_quantize_rows": (None, [P, i64, i64, i32, P, P]),
            "oracle_mxfp4_dequant_rows": (None, [P, P, i64, i32, P]),
            "oracle_e4m3_encode_signed_array": (None, [P, i64, P]),
            "oracle_attention_row_swa": (None, [P, i32, P, P, P, i32, i64, P, i64, i32, f64, P, P]),
            "oracle_attention_rows_swa": (None, [i32, P, i32, P, P, P, P, i32, P, P, P, P, f64, P, P]),
            "oracle_num_threads": (i32, []),
            "oracle_set_num_threads": (None, [i32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (timing only)."""
    _lib().oracle_set_num_threads(int(n))


# ------------------------------------------------------------------ codecs

def e2m1_value(code: int) -> float:
    return float(_lib().oracle_e2m1_value(code))


def e4m3_value(b: int) -> float:
    return float(_lib().oracle_e4m3_value(b))


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    _lib().oracle_e4m3_encode_array(_p(v), v.size, _p(out))
    return out


def e4m3_encode_signed(v: np.ndarray) -> np.ndarray:
    """Signed E4M3 byte per element (the FP8 local-window cache format)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    _lib().oracle_e4m3_encode_signed_array(_p(v), v.size, _p(out))
    return out


def fp8_dequant(codes: np.ndarray) -> np.ndarray:
    """Signed E4M3 bytes -> float64 values (the format definition, per byte)."""
    table = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    _lib().oracle_e2m1_encode_array(_p(v), v.size, _p(out))
    return out


def quantize(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """fp32 [n, 512] -> (codes uint8 [n, 256], scales uint8 [n, 32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    n = x.shape[0]
    codes = np.empty((n, D // 2), dtype=np.uint8)
    scales = np.empty((n, NG), dtype=np.uint8)
    _lib().oracle_quantize_rows(_p(x), n, D, _p(codes), _p(scales))
    return codes, scales


def dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    n = codes.shape[0]
    out = np.empty((n, D), dtype=np.float64)
    _lib().oracle_dequant_rows(_p(codes), _p(scales), n, _p(out))
    return out


# ----------------------------------------------------------------- indexer

def mxfp4_quantize(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """fp32 [n, dim] (dim a multiple of 32) -> OCP MXFP4 (codes u8 [n, dim/2], E8M0 scales u8 [n, dim/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    n, dim = x.shape
    codes = np.empty((n, dim // 2), dtype=np.uint8)
    scales = np.empty((n, dim // 32), dtype=np.uint8)
    _lib().oracle_mxfp4_quantize_rows(_p(x), n, dim, dim, _p(codes), _p(scales))
    return codes, scales


def mxfp4_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 rows -> fp32 [n, dim] (exact)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    n, dim = codes.shape[0], codes.shape[1] * 2
    out = np.empty((n, dim), dtype=np.float32)
    _lib().oracle_mxfp4_dequant_rows(_p(codes), _p(scales), n, dim, _p(out))
    return out


def e8m0_value(b: int) -> float:
    return float(_lib().oracle_e8m0_value(b))


def index_scores(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """q fp32 [H, Dk], k fp32 [n, Dk] -> scores fp32 [n] (fixed fmaf order)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    H, Dk = q.shape
    out = np.empty(k.shape[0], dtype=np.float32)
    _lib().oracle_index_scores(_p(q), H, Dk, _p(k), k.shape[0], Dk, _p(out))
    return out


def topk(scores: np.ndarray, K: int, pos: Optional[np.ndarray] = None) -> np.ndarray:
    """Top-K positions by (score desc, position asc), ascending, -1 padded."""
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    if pos is not None:
        pos = np.ascontiguousarray(pos, dtype=np.int64)
    out = np.empty(K, dtype=np.int32)
    _lib().oracle_topk(_p(scores), _p(pos), scores.shape[0], K, _p(out))
    return out


def hsi_pool(scores: np.ndarray, P: int, block: int = 8) -> Tuple[np.ndarray, int]:
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    out = np.empty(P, dtype=np.int32)
    n = int(_lib().oracle_hsi_pool(_p(scores), scores.shape[0], block, P, _p(out)))
    return out, n


# --------------------------------------------------------------- attention

def attention(q: np.ndarray, codes: np.ndarray, scales: np.ndarray, idx: np.ndarray,
              visible: int, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """One row: q fp32 [Hq, 512] over one cache segment -> (o fp32 [Hq,512], lse fp32 [Hq])."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    Hq = q.shape[0]
    o = np.empty((Hq, D), dtype=np.float32)
    lse = np.empty(Hq, dtype=np.float32)
    _lib().oracle_attention_row(_p(q), Hq, _p(codes), _p(scales), _p(idx), idx.shape[0],
                                int(visible), float(scale), _p(o), _p(lse))
    return o, lse


def attention_rows(q: np.ndarray, codes: np.ndarray, scales: np.ndarray, row_start: np.ndarray,
                   idx: np.ndarray, visible: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """R rows at once: q [R, Hq, 512], idx [R, K], packed cache with per-row segment starts."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    row_start = np.ascontiguousarray(row_start, dtype=np.int64)
    visible = np.ascontiguousarray(visible, dtype=np.int64)
    R, Hq, _ = q.shape
    o = np.empty((R, Hq, D), dtype=np.float32)
    lse = np.empty((R, Hq), dtype=np.float32)
    _lib().oracle_attention_rows(R, _p(q), Hq, _p(codes), _p(scales), _p(row_start), _p(idx),
                                 idx.shape[1], _p(visible), float(scale), _p(o), _p(lse))
    return o, lse


def attention_rows_swa(q: np.ndarray, codes: np.ndarray, scales: np.ndarray, row_start: np.ndarray,
                       idx: np.ndarray, visible: np.ndarray, win_codes: np.ndarray, win_start: np.ndarray,
                       win_len: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """R rows, each attending over its selected FP4 entries joined with its
    FP8 window (rows win_start[r] .. + min(win_len[r], 128) of win_codes
    [*, 512]) in one softmax."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    row_start = np.ascontiguousarray(row_start, dtype=np.int64)
    visible = np.ascontiguousarray(visible, dtype=np.int64)
    win_codes = np.ascontiguousarray(win_codes, dtype=np.uint8)
    win_start = np.ascontiguousarray(win_start, dtype=np.int64)
    win_len = np.ascontiguousarray(win_len, dtype=np.int32)
    R, Hq, _ = q.shape
    o = np.empty((R, Hq, D), dtype=np.float32)
    lse = np.empty((R, Hq), dtype=np.float32)
    _lib().oracle_attention_rows_swa(R, _p(q), Hq, _p(codes), _p(scales), _p(row_start), _p(idx), idx.shape[1],
                                     _p(visible), _p(win_codes), _p(win_start), _p(win_len), float(scale),
                                     _p(o), _p(lse))
    return o, lse


def visible_entries(t: int, m: int) -> int:
    """Cache entries a query at token position t sees when each entry folds m tokens: the entries
    whose whole block of m tokens lies at or before t (the brief's encoder layers compress m = 2
    tokens per entry, "The global branch" / mode layout).  Counted one block at a time."""
    n = 0
    e = 0
    while m * e + (m - 1) <= t:
        n += 1
        e += 1
    return n


# ------------------------------------------------------------------- modes

def full_select(idx_q: np.ndarray, idx_k: np.ndarray, visible: int, K: int,
                pool_size: int = 0, block: int = 8):
    """Full-mode selection for one row: (idx [K], pool [P] or None, pool_len)."""
    s = index_scores(idx_q, idx_k[:visible])
    sel = topk(s, K)
    if pool_size > 0:
        pool, n = hsi_pool(s, pool_size, block)
        return sel, pool, n
    return sel, None, 0


def reindex_select(idx_q: np.ndarray, idx_k: np.ndarray, pool: np.ndarray, visible: int, K: int) -> np.ndarray:
    """Reindex-mode selection for one row: score pool entries (skipping -1 and
    entries >= visible) with this layer's indexer query, keep the top-K."""
    pool = np.asarray(pool, dtype=np.int64)
    ok = (pool >= 0) & (pool < visible)
    cand = pool[ok]
    s = index_scores(idx_q, idx_k[cand]) if cand.size else np.empty(0, np.float32)
    return topk(s, K, cand)
