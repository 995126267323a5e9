"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This package holds random-number plumbing only: it draws the raw values the
method consumes (KV latents, local-window latents, indexer keys and queries, attention queries,
sequence lengths) and rounds them to the storage dtype a workload names.  It
contains none of the method's arithmetic (no quantization, scoring,
selection or attention).
"""
from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    Layer,
    get,
    bf16_round,
    bf16_bits,
    kv_rows,
    window_rows,
    idx_k_rows,
    attn_q,
    index_q,
    seq_lens,
    CHUNK,
)
