"""CSA2 sparse attention over an FP4 (E2M1 + per-16 E4M3 scale) KV cache, gfx950.

The compute lives in libcsa2.so (hand-written HIP kernels behind the C ABI
of include/csa2.h); this package is its ctypes binding plus the static
layer-mode driver.  Importing it does not require a GPU; calling the
kernels does, and fails loudly when the library is missing.
"""
from . import csa2  # noqa: F401
from .csa2 import (  # noqa: F401
    BF16,
    F32,
    FULL,
    REINDEX,
    CSA2Error,
    index_topk,
    index_topk_mxfp4,
    index_topk_workspace_size,
    quantize_idx_mxfp4,
    quantize_kv_fp4,
    quantize_swa_fp8,
    sparse_attn,
    sparse_attn_noalloc,
    sparse_attn_swa,
    sparse_attn_swa_workspace_size,
    sparse_attn_workspace_size,
)
from .chain import Cache, LayerChain, LayerSpec, Window, compressed_visible, validate_modes  # noqa: F401
