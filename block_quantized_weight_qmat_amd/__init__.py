"""Block-quantized weight matmul (Q4_0, Q8_0, Q4_K-style, Q6_K-style) for
MI355X.

The compute lives in the HIP library ``libqmat.so`` (C ABI in
``include/qmat.h``); ``binding`` marshals torch device tensors into it.
``inputs`` draws the seeded synthetic workloads.
"""
from __future__ import annotations

__all__ = ["quantize", "gemv", "gemv_batch", "gemv_jobs", "gemm", "gemm_ws", "gemm_workspace_bytes", "prefill", "prefill_noalloc", "kv_write",
           "block_elems", "block_bytes", "row_bytes", "noalloc_scratch_bytes",
           "Q4_0", "Q8_0", "Q4_K", "Q6_K", "FORMATS", "QmatError", "library_path"]

Q4_0, Q8_0, Q4_K, Q6_K = 0, 1, 2, 3


def __getattr__(name):
    # The binding imports torch; load it only when an entry point is used.
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
