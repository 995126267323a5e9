"""CSA2 decode benchmark on one MI355X.

Default workload: the six-layer chain at 128K context, batch 16 (Full with
an 8,192-entry candidate pool, two Reindex layers, three Reuse layers), one
decode step per timed step: the first Full layer quantizes each sequence's
newest token into the FP4 cache, every selecting layer runs the indexer and
exact top-K, every layer runs sparse attention with its own query.  Inputs
are seeded synthetic data (gen/) resident in HBM before timing starts.

Prints one JSON line: tokens/s over the timed steps, the roofline of the
dominant kernel (HIP events on the launch stream via the library's
measurement hook), and the CPU oracle timed on a bounded sample (all host
threads, and one thread on a smaller sample).  The timed steps replay back to
back (warm caches); `cold_cache` repeats the per-kernel event pass with a
1 GiB write before every step, so that nothing of the step stays in the
256 MB MALL or the L2s.  `dtype` names the arithmetic: fp16 MFMA with fp32
accumulation in the attention, fp32 fused multiply-adds in the indexer.

    python bench.py [--steps K] [--warmup W] [--workload c3|c2|c5|c4] [--gpus 1]

The prefill workload (c4) times one 4,096-token chunk appended causally to a
262,144-token cache: quantize-on-write of the chunk, the Full indexer and
exact top-K for each of its rows, and sparse attention for each row.

--idx-mxfp4 stores the indexer keys in OCP MXFP4 (34 B per 64-channel key
instead of 128 B of bf16), quantized on the GPU from the same generated keys.

--workload c3v checks 5 draft tokens per sequence of the 128K chain in one pass
(speculative verification): the 5 drafts are the last 5 cached tokens, written
by the step, and draft i of a sequence sees the cache up to itself (80 rows).

--swa adds the local branch to every layer: each layer keeps its own FP8
window of the 128 most recent tokens (a ring of 128 rows per sequence in
decode, the chunk's band in prefill), writes the step's tokens into it and
attends over it joined with its selected entries in one softmax.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import gen  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
VALU_F32_PEAK_TFLOPS = 157.3
METRIC = "CSA2 decode tokens/s + achieved HBM GB/s (FP4 KV) at 128K ctx, 1 GPU"
KV_ROW_BYTES = 288


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ setup

def build_cache(w, lens, device, chunk=65536, mxfp4=False):
    """Quantize every sequence's KV into one packed FP4 cache on the GPU (indexer keys in MXFP4 if asked)."""
    import torch

    from sparse_attention_fp4_e4m3_amd import Cache, csa2

    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    rows = int(lens.sum())
    codes = torch.empty(rows, 256, dtype=torch.uint8, device=device)
    scales = torch.empty(rows, 32, dtype=torch.uint8, device=device)
    kdt = torch.bfloat16 if w.idx_dtype == "bf16" else torch.float32
    idx_k = torch.empty(rows, 64, dtype=kdt, device=device)
    ik_codes = torch.empty(rows, 32, dtype=torch.uint8, device=device) if mxfp4 else None
    ik_scales = torch.empty(rows, 2, dtype=torch.uint8, device=device) if mxfp4 else None
    for b in range(len(lens)):
        for t0 in range(0, int(lens[b]), chunk):
            t1 = min(int(lens[b]), t0 + chunk)
            x = torch.from_numpy(gen.kv_rows(w, b, t0, t1)).to(device)
            r0 = int(starts[b]) + t0
            csa2.quantize_kv_fp4(x, codes[r0:r0 + (t1 - t0)], scales[r0:r0 + (t1 - t0)])
            ik = gen.idx_k_rows(w, b, t0, t1)
            if kdt == torch.bfloat16:
                ik = torch.from_numpy(gen.bf16_bits(ik).view(np.int16)).view(torch.bfloat16)
            else:
                ik = torch.from_numpy(ik)
            idx_k[r0:r0 + (t1 - t0)] = ik.to(device)
            if mxfp4:
                csa2.quantize_idx_mxfp4(idx_k[r0:r0 + (t1 - t0)], ik_codes[r0:r0 + (t1 - t0)],
                                        ik_scales[r0:r0 + (t1 - t0)])
        torch.cuda.synchronize()
    if mxfp4:
        del idx_k
        return Cache(codes, scales, ik_codes, torch.from_numpy(starts).to(device),
                     torch.from_numpy(lens.astype(np.int32)).to(device), int(lens.max()),
                     idx_k_scales=ik_scales), starts
    return Cache(codes, scales, idx_k, torch.from_numpy(starts).to(device),
                 torch.from_numpy(lens.astype(np.int32)).to(device), int(lens.max())), starts


def build_prefill(w, device, chunk=65536, mxfp4=False):
    """The prefill workload: a cache of n - T tokens plus the chunk's own T rows.

    Row r of the chunk sits at cache position P0 + r and sees positions
    [0, P0 + r].  Indexer keys of every position are resident up front; the
    chunk's KV rows are (re)written by the timed step's quantize-on-write.
    Returns (cache, q per layer, idx_q per layer, new_kv, new_kv_rows, lens)."""
    import torch

    from sparse_attention_fp4_e4m3_amd import Cache, csa2

    T = w.prefill_tokens
    P0 = w.n - T
    codes = torch.empty(w.n, 256, dtype=torch.uint8, device=device)
    scales = torch.empty(w.n, 32, dtype=torch.uint8, device=device)
    kdt = torch.bfloat16 if w.idx_dtype == "bf16" else torch.float32
    idx_k = torch.empty(w.n, 64, dtype=kdt, device=device)
    for t0 in range(0, w.n, chunk):
        t1 = min(w.n, t0 + chunk)
        csa2.quantize_kv_fp4(torch.from_numpy(gen.kv_rows(w, 0, t0, t1)).to(device), codes[t0:t1], scales[t0:t1])
        idx_k[t0:t1] = to_dev(gen.idx_k_rows(w, 0, t0, t1), w.idx_dtype, device)
    torch.cuda.synchronize()
    starts = torch.zeros(T, dtype=torch.int64, device=device)
    vis = torch.from_numpy((P0 + 1 + np.arange(T)).astype(np.int32)).to(device)
    cache = Cache(codes, scales, idx_k, starts, vis, w.n, shared_segment=True)
    if mxfp4:
        kc = torch.empty(w.n, 32, dtype=torch.uint8, device=device)
        ks = torch.empty(w.n, 2, dtype=torch.uint8, device=device)
        csa2.quantize_idx_mxfp4(idx_k, kc, ks)
        torch.cuda.synchronize()
        cache = Cache(codes, scales, kc, starts, vis, w.n, shared_segment=True, idx_k_scales=ks)
        del idx_k
    qs = [to_dev(gen.attn_q(w, 0), w.q_dtype, device)]
    iqs = [to_dev(gen.index_q(w, 0), w.idx_dtype, device)]
    new_kv = torch.from_numpy(gen.kv_rows(w, 0, P0, w.n)).to(device)
    new_rows = torch.from_numpy(np.arange(P0, w.n, dtype=np.int64)).to(device)
    return cache, qs, iqs, new_kv, new_rows, (P0 + 1 + np.arange(T)).astype(np.int64)


def build_windows(w, lens, device):
    """Each layer's FP8 window, filled with the 128 tokens before the timed step's own.

    Decode: a ring of 128 rows per sequence (row = position mod 128); the step
    writes each sequence's newest token.  Prefill: rows i <-> positions
    P0 - 127 + i; the step writes the chunk's T tokens at rows 127.., and
    chunk row r attends over rows r .. r + 127.
    Returns (windows, new_win per layer, new_win_rows)."""
    import torch

    from sparse_attention_fp4_e4m3_amd import Window, csa2

    W = 128
    wins, new = [], []
    if w.is_prefill:
        T = w.prefill_tokens
        P0 = w.n - T
        rows = torch.from_numpy(np.arange(W - 1, W - 1 + T, dtype=np.int64)).to(device)
        for li in range(len(w.layers)):
            codes = torch.empty(W - 1 + T, 512, dtype=torch.uint8, device=device)
            csa2.quantize_swa_fp8(torch.from_numpy(gen.window_rows(w, li, 0, P0 - (W - 1), P0)).to(device),
                                  codes[:W - 1])
            wins.append(Window(codes, torch.arange(T, dtype=torch.int64, device=device),
                               torch.full((T,), W, dtype=torch.int32, device=device)))
            new.append(torch.from_numpy(gen.window_rows(w, li, 0, P0, w.n)).to(device))
        torch.cuda.synchronize()
        return wins, new, rows
    B = len(lens)
    ring = lambda b, t: b * W + t % W  # noqa: E731
    rows = torch.from_numpy(np.array([ring(b, int(lens[b]) - 1) for b in range(B)], np.int64)).to(device)
    for li in range(len(w.layers)):
        codes = torch.zeros(B * W, 512, dtype=torch.uint8, device=device)
        for b in range(B):
            n = int(lens[b])
            t0 = max(0, n - W)
            dst = torch.from_numpy(np.array([ring(b, t) for t in range(t0, n)], np.int64)).to(device)
            csa2.quantize_swa_fp8(torch.from_numpy(gen.window_rows(w, li, b, t0, n)).to(device), codes, dst)
        wins.append(Window(codes, torch.from_numpy(np.arange(B, dtype=np.int64) * W).to(device),
                           torch.from_numpy(np.minimum(lens, W).astype(np.int32)).to(device)))
        new.append(torch.from_numpy(np.concatenate([gen.window_rows(w, li, b, int(lens[b]) - 1, int(lens[b]))
                                                    for b in range(B)])).to(device))
    torch.cuda.synchronize()
    return wins, new, rows


def to_dev(a, kind, device):
    import torch

    if kind == "bf16":
        return torch.from_numpy(gen.bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def layer_inputs(w, device):
    qs, iqs = [], []
    for li, L in enumerate(w.layers):
        qs.append(to_dev(gen.attn_q(w, li), w.q_dtype, device))
        iqs.append(to_dev(gen.index_q(w, li), w.idx_dtype, device) if L.mode != "reuse" else None)
    return qs, iqs


# ------------------------------------------------------------------ accounting

def algorithmic_bytes(w, lens, mxfp4=False):
    """Bytes the method must move per step (one decode token per sequence, or one prefill chunk), by kernel family."""
    R, K = w.rows, w.K
    qb = 2 if w.q_dtype == "bf16" else 4
    kb = 2 if w.idx_dtype == "bf16" else 4
    if mxfp4:
        kb = 34 / 64  # 32 code bytes + 2 E8M0 scale bytes per 64-channel key
    out = {"quantize": R * (512 * 4 + KV_ROW_BYTES)}
    if w.is_prefill:
        # the chunk's rows share one key segment: each key and each query is read once
        out["index_scan"] = int(lens.max()) * 64 * kb + R * w.H * 64 * qb
    else:
        out["index_scan"] = int(int(lens.sum()) * 64 * kb)
    pool = 0
    reindex = 0
    for L in w.layers:
        if L.mode == "full":
            pool = L.pool_size
        elif L.mode == "reindex":
            reindex += int(R * pool * 64 * kb)
    out["reindex_score"] = reindex
    per_attn = R * (K * KV_ROW_BYTES + K * 4 + w.Hq * 512 * qb + w.Hq * 512 * 4)
    out["attention_per_layer"] = per_attn
    out["attention"] = per_attn * len(w.layers)
    out["total"] = out["quantize"] + out["index_scan"] + out["reindex_score"] + out["attention"]
    return out


def attention_kernel_name(w):
    """Name and source file of the attention kernel the library's launch plan picks for this
    workload (a label for the report).  bf16 queries without a window: 64-head workgroups when
    rows x 64-head groups fill 256 workgroups, else 32-head decode workgroups (k_attn_dec, whose
    key splits are merged by workgroups of the same launch) for up to 256 row x 32-head pairs."""
    if w.q_dtype == "bf16" and w.Hq % 32 == 0:
        if (w.Hq // 16) % 4 == 0 and w.rows * (w.Hq // 64) >= 256:
            return "k_sparse_attn_wide", "k_attn.hip"
        if w.rows * (w.Hq // 32) <= 256:
            return "k_attn_dec<%s>" % ("true" if dec_keys_per_split(w) > 256 else "false"), "k_attn_dec.hip"
    return "k_sparse_attn", "k_attn.hip"


def dec_keys_per_split(w):
    """Keys per workgroup of the decode attention: splits so that about 256 workgroups run, at most
    one per 256-key chunk and at most 8."""
    pairs = w.rows * (w.Hq // 32)
    chunks = -(-w.K // 256)
    s = min(chunks, 8, max(1, -(-256 // pairs)))
    return -(-(-(-w.K // s)) // 256) * 256


def attention_flops(w):
    return 4.0 * w.rows * w.Hq * w.K * 512


def index_flops(w, lens):
    """fp32 multiply-adds of the indexer scan: every visible entry, every indexer head, 64 channels."""
    return 2.0 * float(np.sum(lens)) * w.H * 64 * w.verify


def oracle_window(w, li, b, t_end):
    """Signed E4M3 codes of layer li's window ending before position t_end (at most 128 tokens)."""
    import oracle

    return oracle.e4m3_encode_signed(gen.window_rows(w, li, b, max(0, t_end - 128), t_end, threads=False))


def oracle_attend(w, q, codes, scales, sel, nvis, win):
    """The oracle's attention of one row, joined with its window when one is given."""
    import oracle

    if win is None:
        return oracle.attention(q, codes, scales, sel, nvis, w.softmax_scale)
    z = np.zeros(1, np.int64)
    return oracle.attention_rows_swa(q[None], codes, scales, z, sel[None], np.array([nvis]), win, z,
                                     np.array([win.shape[0]], np.int32), w.softmax_scale)


def cpu_baseline_prefill(w, sample_rows, swa=False, mxfp4=False):
    """The CPU oracle on `sample_rows` rows of the prefill chunk: indexer scan over the row's visible
    entries, exact top-K and attention (joined with the row's window under swa)."""
    import oracle

    T = w.prefill_tokens
    P0 = w.n - T
    rows = [int(r) for r in np.linspace(0, T - 1, sample_rows)]
    log("cpu baseline: preparing the oracle cache (%d entries)" % w.n)
    codes, scales = oracle.quantize(gen.kv_rows(w, 0, 0, w.n))
    ik = gen.idx_k_rows(w, 0, 0, w.n)
    if mxfp4:  # the keys the GPU scores: MXFP4, dequantized exactly
        ik = oracle.mxfp4_dequant(*oracle.mxfp4_quantize(ik))
    iq = gen.index_q(w, 0)
    q = gen.attn_q(w, 0)
    wins = {r: oracle_window(w, 0, 0, P0 + r + 1) for r in rows} if swa else {}
    def run(rs):
        t0 = time.perf_counter()
        for r in rs:
            nvis = P0 + r + 1
            sel = oracle.topk(oracle.index_scores(iq[r], ik[:nvis]), w.K)
            oracle_attend(w, q[r], codes, scales, sel, nvis, wins.get(r))
        return time.perf_counter() - t0

    cores = oracle.num_threads()
    dt = run(rows)
    res = {"value": len(rows) / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": "%d of %d chunk rows (indexer scan over ~%d entries, top-K, attention each); %.1f s wall"
                     % (len(rows), T, P0, dt)}
    one = rows[::max(1, len(rows) // 8)][:8]
    oracle.set_num_threads(1)
    try:
        dt1 = run(one)
    finally:
        oracle.set_num_threads(cores)
    res["single_thread"] = {"value": len(one) / dt1, "unit": "tokens/s", "cores": 1,
                            "sample": "%d of the same chunk rows; %.1f s wall" % (len(one), dt1)}
    res["cpu_model"] = cpu_model()
    return res


def traffic_from_profiles(workload, kernel_file):
    """HBM bytes per launch measured with rocprofv3 counters on this workload, if taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic_counters.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        src = os.path.join(ROOT, "sparse_attention_fp4_e4m3_amd", "csrc", kernel_file)
        h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        ent = rec.get("workloads", {}).get(workload, {}).get(kernel_file)
        if ent and ent.get("source_sha256_16") == h:
            return ent.get("bytes_per_launch")
    except Exception:
        return None
    return None


# ------------------------------------------------------------------ CPU oracle baseline

def cpu_baseline(w, lens, sample_rows, reps, swa=False, mxfp4=False):
    """`reps` decode steps of the same chain for `sample_rows` sequences, run by the CPU oracle
    (every layer joined with its window under swa)."""
    import oracle

    rows = list(range(min(sample_rows, w.B)))
    V = w.verify
    reps = max(1, reps // V)  # V query rows per sequence multiply the work of a step: keep the sample's CPU time bounded
    log("cpu baseline: preparing oracle cache for %d sequences" % len(rows))
    caches = {}
    for b in rows:
        x = gen.kv_rows(w, b, 0, int(lens[b]))
        ik = gen.idx_k_rows(w, b, 0, int(lens[b]))
        if mxfp4:  # the keys the GPU scores: MXFP4, dequantized exactly
            ik = oracle.mxfp4_dequant(*oracle.mxfp4_quantize(ik))
        caches[b] = (oracle.quantize(x), ik)
        del x
    qs = [gen.attn_q(w, li, 0, len(rows) * V) for li in range(len(w.layers))]
    iqs = [gen.index_q(w, li, 0, len(rows) * V) if L.mode != "reuse" else None for li, L in enumerate(w.layers)]
    new_kv = [gen.kv_rows(w, b, int(lens[b]) - V, int(lens[b])) for b in rows]
    wins = {(li, b): oracle_window(w, li, b, int(lens[b])) for li in range(len(w.layers)) for b in rows} if swa else {}
    def run(seqs, nrep):
        t0 = time.perf_counter()
        for b in [b for _ in range(nrep) for b in seqs]:
            (codes, scales), ik = caches[b]
            c1, s1 = oracle.quantize(new_kv[b])  # the newest token(s), written by the first Full layer
            codes[int(lens[b]) - V:int(lens[b])], scales[int(lens[b]) - V:int(lens[b])] = c1, s1
            for i in range(V):  # query row (b, i) sees the cache up to its own token
                n = int(lens[b]) - V + 1 + i
                r = b * V + i
                pool = None
                sel = None
                for li, L in enumerate(w.layers):
                    if L.mode == "full":
                        sel, pool, _ = oracle.full_select(iqs[li][r], ik, n, w.K, L.pool_size)
                    elif L.mode == "reindex":
                        sel = oracle.reindex_select(iqs[li][r], ik, pool, n, w.K)
                    oracle_attend(w, qs[li][r], codes, scales, sel, n, wins.get((li, b)))
        return time.perf_counter() - t0

    what = ("one full decode step of the %d-layer chain (quantize newest token(s), indexer scan over %d tokens, "
            "top-K, pool, Reindex, attention per layer)" % (len(w.layers), int(lens[0])))
    cores = oracle.num_threads()
    dt = run(rows, reps)
    res = {"value": reps * len(rows) * V / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": "%d of %d sequences x %d query rows x %d repetitions of %s; %.1f s wall"
                     % (len(rows), w.B, V, reps, what, dt)}
    # the same oracle on one thread, over a smaller sample of the same steps
    one = rows[:min(2, len(rows))]
    oracle.set_num_threads(1)
    try:
        dt1 = run(one, 1)
    finally:
        oracle.set_num_threads(cores)
    res["single_thread"] = {"value": len(one) * V / dt1, "unit": "tokens/s", "cores": 1,
                            "sample": "%d of %d sequences x %d query rows x 1 repetition of the same step; %.1f s wall"
                                      % (len(one), w.B, V, dt1)}
    res["cpu_model"] = cpu_model()
    return res


def cpu_model():
    """The host CPU: lscpu's model name and counts, else /proc/cpuinfo's model name."""
    import subprocess

    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        f = dict(line.split(":", 1) for line in out.splitlines() if ":" in line)
        f = {k.strip(): v.strip() for k, v in f.items()}
        if "Model name" in f:
            return "%s; %s CPUs, %s threads per core, %s sockets" % (
                f["Model name"], f.get("CPU(s)", "?"), f.get("Thread(s) per core", "?"), f.get("Socket(s)", "?"))
    except Exception:
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return None


# ------------------------------------------------------------------ HIP events without a system fence

_HIP = None


def _hip_runtime():
    """The HIP runtime library already loaded into this process (the one torch uses)."""
    global _HIP
    if _HIP is None:
        import ctypes

        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        _HIP = ctypes.CDLL(path or "libamdhip64.so")
        P = ctypes.c_void_p
        _HIP.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(P), ctypes.c_uint]
        _HIP.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
        _HIP.hipEventDestroy.argtypes = [P]
        _HIP.hipEventRecord.argtypes = [P, P]
    return _HIP


class HipEvent:
    """A timing event created with hipEventDisableSystemFence, so that recording it
    around a kernel does not add a system-scope cache flush to the measured span."""

    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        import ctypes

        self._h = ctypes.c_void_p()
        rc = _hip_runtime().hipEventCreateWithFlags(ctypes.byref(self._h), self.FLAGS)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)
        self.cuda_event = self._h.value
        # recorded once up front, so that a kernel a step never launches reads as 0
        import torch

        _hip_runtime().hipEventRecord(self._h, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))

    def elapsed_time(self, other) -> float:
        import ctypes

        ms = ctypes.c_float()
        rc = _hip_runtime().hipEventElapsedTime(ctypes.byref(ms), self._h, other._h)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return ms.value

    def __del__(self):
        try:
            _hip_runtime().hipEventDestroy(self._h)
        except Exception:
            pass


# ------------------------------------------------------------------ main

def attn_row_sweep(rows_list, steps, warmup):
    """The decode attention call alone at the 128K chain's shape (64 bf16 query heads of 512, top-2048
    over 131,072 cached FP4 entries per row, each row its own segment) for several row counts: one JSON
    line with microseconds per launch (a HIP graph of `steps` back-to-back launches, warm caches) and the
    launch's algorithmic bytes and flops against the HBM and fp16 MFMA peaks.  Cache bytes are random
    codes and finite scales: only the timing is of interest here."""
    import torch

    from sparse_attention_fp4_e4m3_amd import csa2

    device = torch.device("cuda:0")
    ctx, Hq, K = 131072, 64, 2048
    per_row = K * 288 + K * 4 + Hq * 512 * 2 + Hq * 512 * 4
    out = []
    rmax = max(rows_list)
    gen_t = torch.Generator(device=device)
    gen_t.manual_seed(7)
    codes = torch.randint(0, 256, (rmax * ctx, 256), dtype=torch.uint8, device=device, generator=gen_t)
    scales = torch.randint(0x28, 0x50, (rmax * ctx, 32), dtype=torch.uint8, device=device, generator=gen_t)
    for R in rows_list:
        q = (torch.randn(R, Hq, 512, device=device, generator=gen_t)).to(torch.bfloat16)
        idx = torch.stack([torch.randperm(ctx, device=device, generator=gen_t)[:K] for _ in range(R)]).to(torch.int32)
        idx, _ = torch.sort(idx, dim=1)
        starts = torch.arange(R, dtype=torch.int64, device=device) * ctx
        vis = torch.full((R,), ctx, dtype=torch.int32, device=device)
        o = torch.empty(R, Hq, 512, dtype=torch.float32, device=device)
        ws = torch.zeros(max(256, csa2.sparse_attn_workspace_size(R, Hq, csa2.BF16, K)), dtype=torch.uint8,
                         device=device)

        def call():
            csa2.sparse_attn(q, codes, scales, starts, idx, o, 1.0 / 512 ** 0.5, row_visible=vis, workspace=ws)

        for _ in range(max(1, warmup)):
            call()
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for _ in range(steps):
                    call()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = float("inf")
        for _ in range(5):
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3 / steps)
        nbytes, flops = R * per_row, 4.0 * R * Hq * K * 512
        out.append({"rows": R, "us_per_launch": best, "bytes": nbytes, "GBps": nbytes / best * 1e-3,
                    "hbm_frac": nbytes / best * 1e-3 / 8000.0, "TFLOPs": flops / best * 1e-6,
                    "mfma_frac": flops / best * 1e-6 / 2500.0})
        log("attention alone, %d rows: %.2f us per launch, %.3f of HBM" % (R, best, out[-1]["hbm_frac"]))
        del q, idx, o, ws, g
    print(json.dumps({"attn_rows_sweep": out, "shape": {"ctx_per_row": ctx, "q_heads": Hq, "top_k": K,
                                                         "q_dtype": "bf16", "kv": "fp4 e2m1 + e4m3 per 16"},
                      "timing": "hip graph of %d back-to-back launches, best of 5 replays, warm caches" % steps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3", choices=["c2", "c3", "c5", "c4", "c3v"])
    ap.add_argument("--cpu-rows", type=int, default=16)
    ap.add_argument("--cpu-reps", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--idx-mxfp4", action="store_true",
                    help="indexer keys stored in OCP MXFP4 (decode workloads)")
    ap.add_argument("--swa", action="store_true",
                    help="every layer also attends over its own 128-token FP8 window (local branch)")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a HIP graph replay")
    ap.add_argument("--event-kind", default="nofence", choices=["nofence", "torch"],
                    help="per-kernel timing events: created without a system fence, or torch's default")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    ap.add_argument("--attn-rows", default="",
                    help="comma-separated row counts: time the decode attention call alone at the 128K chain's "
                         "shape for each (one JSON line), instead of a workload step")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU per process and box; --gpus %d is not supported "
              "(multi-GPU sharding is a design note only)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.attn_rows:
        attn_row_sweep([int(x) for x in args.attn_rows.split(",")], max(1, min(args.steps, 50)), args.warmup)
        return

    import torch

    from sparse_attention_fp4_e4m3_amd import LayerChain, LayerSpec, csa2

    device = torch.device("cuda:0")
    w = gen.get(args.workload)
    if args.swa and w.verify > 1:
        print("bench.py: --swa is built for one query row per sequence", file=sys.stderr)
        sys.exit(2)
    log("workload %s: %s" % (w.name, w.description))
    t = time.time()
    if w.is_prefill:
        cache, qs, iqs, new_kv, new_rows_t, lens = build_prefill(w, device, mxfp4=args.idx_mxfp4)
    else:
        lens = gen.seq_lens(w)
        cache, _ = build_cache(w, lens, device, mxfp4=args.idx_mxfp4)
        qs, iqs = layer_inputs(w, device)
        V = w.verify  # the last V tokens of each sequence are (re)written by the step; row (b, i) sees up to draft i
        starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
        new_rows = np.concatenate([starts[b] + np.arange(int(lens[b]) - V, int(lens[b])) for b in range(w.B)])
        new_kv = torch.from_numpy(np.concatenate([gen.kv_rows(w, b, int(lens[b]) - V, int(lens[b]))
                                                  for b in range(w.B)])).to(device)
        new_rows_t = torch.from_numpy(new_rows.astype(np.int64)).to(device)
        if V > 1:
            cache.row_kv_start = torch.from_numpy(np.repeat(starts, V).astype(np.int64)).to(device)
            cache.row_visible = torch.from_numpy(np.concatenate([int(lens[b]) - V + 1 + np.arange(V)
                                                                 for b in range(w.B)]).astype(np.int32)).to(device)
    log("inputs built in %.1f s (%d cache rows)" % (time.time() - t, int(cache.kv_codes.shape[0])))
    wins = new_win = new_win_rows = None
    if args.swa:
        wins, new_win, new_win_rows = build_windows(w, lens, device)
        log("windows built: %d layers x %d rows" % (len(wins), int(wins[0].codes.shape[0])))
    chain = LayerChain([LayerSpec(L.mode, L.pool_size) for L in w.layers], w.rows, w.Hq, w.H, w.K, cache.max_visible,
                       qs[0].dtype, device, shared_segment=cache.shared_segment, swa=args.swa)

    def step():
        chain.step(cache, qs, iqs, w.softmax_scale, new_kv=new_kv, new_kv_rows=new_rows_t, windows=wins,
                   new_win=new_win, new_win_rows=new_win_rows)

    if args.calib_copy_mib:
        a = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=device)
        b_ = torch.empty_like(a)
        b_.copy_(a)
        torch.cuda.synchronize()

    # eager warm-up (also configures the kernels), then capture one decode step as a HIP graph
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    graph = None
    if not args.eager:
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            step()
        torch.cuda.current_stream().wait_stream(s_cap)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()

    run = graph.replay if graph is not None else step
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        run()
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_step = total_ms / args.steps

    # per-kernel durations: HIP events recorded by the library on the launch stream around
    # each kernel, over an eager pass of the same number of steps (a kernel launched several
    # times per step is timed on its last launch of the step)
    kernels = {"index_scan": csa2.KERNEL_INDEX_SCAN, "reindex_score": csa2.KERNEL_REINDEX_SCORE,
               "attention": csa2.KERNEL_ATTN, "attention_combine": csa2.KERNEL_ATTN_COMBINE,
               "quantize": csa2.KERNEL_QUANT}
    n_launch = {"index_scan": 1, "quantize": 1,
                "reindex_score": sum(L.mode == "reindex" for L in w.layers),
                "attention": len(w.layers), "attention_combine": len(w.layers)}
    if args.swa:
        # decode writes each row's window token inside the attention call; a prefill chunk writes first
        kernels["swa_attention"] = csa2.KERNEL_SWA_ATTN
        n_launch["swa_attention"] = len(w.layers)
        if w.is_prefill:
            kernels["quantize_fp8"] = csa2.KERNEL_QUANT_FP8
            n_launch["quantize_fp8"] = len(w.layers)

    def arm(kid):
        if args.event_kind == "torch":
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            e.record()  # materialize the handles
        else:
            s, e = HipEvent(), HipEvent()
        csa2.profile_kernel_events(kid, s, e)
        return s, e

    def mark():
        if args.event_kind == "torch":
            m = torch.cuda.Event(enable_timing=True)
            m.record()
            return m
        return HipEvent()  # recorded on creation

    def event_pass(flush=None):
        """Eager steps with every kernel bracketed by events; flush: a tensor written by a fill kernel
        before each step (cold caches).  Returns per-kernel mean us (None: never launched)."""
        pairs = []
        torch.cuda.synchronize()
        for i in range(args.steps):
            if flush is not None:
                flush.fill_(1 + (i % 250))
            armed = {k: arm(kid) for k, kid in kernels.items()}
            begin = mark()  # a kernel whose stop event precedes this one was not launched in the step
            step()
            pairs.append((begin, armed))
        torch.cuda.synchronize()
        us = {}
        for k in kernels:
            vals = [a[k][0].elapsed_time(a[k][1]) * 1e3 for b, a in pairs if b.elapsed_time(a[k][1]) > 0]
            us[k] = float(np.mean(vals)) if vals else None
        return us

    def step_times(flush=None):
        """Mean time of one step (a graph replay, else eager) between events around it, each step
        after a fill kernel over `flush` when given; the fill gives the host time to queue the step."""
        spans = []
        torch.cuda.synchronize()
        for i in range(args.steps):
            if flush is not None:
                flush.fill_(1 + (i % 250))
            b = mark()
            run()
            spans.append((b, mark()))
        torch.cuda.synchronize()
        return float(np.mean([b.elapsed_time(e) for b, e in spans]))

    per_kernel_us = event_pass()
    # cold caches: a 1 GiB write before every step evicts the 256 MB MALL and the L2s, so the step's
    # cache, queries and indices come from HBM
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=device)
    cold_us = event_pass(flush)
    for kid in kernels.values():
        csa2.profile_kernel_events(kid, None, None)
    cold_ms = step_times(flush)
    del flush
    warm_ms = step_times(torch.empty(1 << 20, dtype=torch.uint8, device=device))  # same spacing, no eviction

    wname = w.name + ("+swa" if args.swa else "") + ("+mxfp4idx" if args.idx_mxfp4 else "")
    byt = algorithmic_bytes(w, lens, args.idx_mxfp4)
    attn_flops = attention_flops(w)
    kern = {
        "index_scan": {"avg_us": per_kernel_us["index_scan"], "bytes": byt["index_scan"], "flops": index_flops(w, lens)},
        "reindex_score": {"avg_us": per_kernel_us["reindex_score"], "bytes": byt["reindex_score"] //
                          max(1, n_launch["reindex_score"])},
        "attention": {"avg_us": per_kernel_us["attention"], "bytes": byt["attention_per_layer"],
                      "flops": attn_flops},
        "attention_combine": {"avg_us": per_kernel_us["attention_combine"]},
        "quantize": {"avg_us": per_kernel_us["quantize"], "bytes": byt["quantize"]},
    }
    if per_kernel_us["attention_combine"] is None:
        del kern["attention_combine"]  # the split merge runs inside the attention launch
    if n_launch["reindex_score"] == 0:
        del kern["reindex_score"]  # a chain without Reindex layers
    if args.swa:
        # the window: 128 entries x 512 B per row; QK^T and PV over them for every head
        win_bytes, win_flops = w.rows * 128 * 512, 4.0 * w.rows * w.Hq * 128 * 512
        if per_kernel_us["swa_attention"] is None:
            # the 64-head plan joins the window to the selection as one more step of the attention launch
            kern["attention"]["bytes"] += win_bytes
            kern["attention"]["flops"] += win_flops
        else:
            kern["swa_attention"] = {"avg_us": per_kernel_us["swa_attention"], "bytes": win_bytes, "flops": win_flops}
        if w.is_prefill:
            kern["quantize_fp8"] = {"avg_us": per_kernel_us["quantize_fp8"], "bytes": w.prefill_tokens * (512 * 4 + 512)}
    for k, v in kern.items():
        if v["avg_us"] is None:
            raise RuntimeError("kernel %s was not launched by the step" % k)
        if "bytes" in v and v["avg_us"] > 0:
            v["GBps"] = v["bytes"] / (v["avg_us"] * 1e3)
            v["hbm_frac"] = v["GBps"] / HBM_PEAK_GBS
        if "flops" in v and v["avg_us"] > 0:
            v["TFLOPs"] = v["flops"] / (v["avg_us"] * 1e6)
            if k in ("attention", "swa_attention"):
                v["mfma_frac"] = v["TFLOPs"] / MFMA_F16_PEAK_TFLOPS
            else:
                v["valu_fp32_frac"] = v["TFLOPs"] / VALU_F32_PEAK_TFLOPS
        v["per_step_us"] = v["avg_us"] * n_launch.get(k, 1)
    dominant = max([k for k in ("index_scan", "attention", "reindex_score") if k in kern],
                   key=lambda k: kern[k]["per_step_us"])
    dk = kern[dominant]
    if dominant == "attention":
        kname, ksrc = attention_kernel_name(w)
        roof = {"kernel": kname, "bound": "mfma", "achieved": dk["TFLOPs"],
                "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": dk["mfma_frac"],
                "traffic": traffic_from_profiles(wname, ksrc)}
    elif dominant == "index_scan" and w.is_prefill:
        # the chunk's rows share one key segment: the scores are a bf16 MFMA product (two passes)
        roof = {"kernel": "k_pf_pass", "bound": "mfma", "achieved": dk["TFLOPs"], "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": dk["TFLOPs"] / MFMA_F16_PEAK_TFLOPS,
                "traffic": traffic_from_profiles(wname, "k_index.hip")}
    else:
        # the Full scan: k_scan_even (decode batches of up to 256 rows share the tiles evenly), else k_score
        scan_name = "k_scan_even" if w.rows <= 256 else "k_score (Full)"
        roof = {"kernel": scan_name if dominant == "index_scan" else "k_score (Reindex)", "bound": "hbm",
                "achieved": dk["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dk["hbm_frac"],
                "traffic": traffic_from_profiles(wname, "k_index.hip")}

    tokens_s = w.rows / (ms_step * 1e-3)
    res = {
        "metric": METRIC if not w.is_prefill else "CSA2 prefill tokens/s (FP4 KV), 4096-token chunk at 262K ctx, 1 GPU",
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16-mfma+f32",
        "data": "synthetic",
        "config": {"workload": "%s: %s" % (wname, w.description + (" + local 128-token FP8 window" if args.swa else "")
                                                        + (" + MXFP4 indexer keys" if args.idx_mxfp4 else "")), "batch": w.B, "rows": w.rows,
                   "ctx": int(lens.max()),
                   "layers": [L.mode for L in w.layers], "top_k": w.K, "q_heads": w.Hq, "indexer_heads": w.H,
                   "kv": "fp4 e2m1 + e4m3 scale per 16 ch (288 B/entry)",
                   "compute": "indexer fp32 fmaf; attention f16 MFMA, f32 accumulate", "parallelism": "single GPU",
                   "launch": "eager" if graph is None else "hip graph replay of one step",
                   "local_window": "128-token FP8 (E4M3) window per layer, joined in one softmax" if args.swa
                   else "none"},
        "roofline": roof,
        "kernels": kern,
    }
    res["chain_hbm_GBps"] = byt["total"] / (ms_step * 1e-3) / 1e9
    res["cold_cache"] = {
        "flush": "1 GiB written by a fill kernel before each step (warm: 1 MiB)",
        "ms_per_step": cold_ms, "warm_ms_per_step": warm_ms, "tokens_per_s": w.rows / (cold_ms * 1e-3),
        "kernels_avg_us": {k: v for k, v in cold_us.items() if v is not None},
        "warm_kernels_avg_us": {k: v for k, v in per_kernel_us.items() if v is not None}}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = (cpu_baseline_prefill(w, max(args.cpu_rows, 128), args.swa, args.idx_mxfp4) if w.is_prefill
                               else cpu_baseline(w, lens, args.cpu_rows, args.cpu_reps, args.swa, args.idx_mxfp4))
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
