"""ctypes binding of libqmat.so (C ABI in include/qmat.h).

Argument marshalling only: torch device tensors supply the memory and
torch's current HIP stream orders the work; every step of the computation
runs in the library's kernels. There is no CPU fallback: without the built
library, or with a tensor that is not on a GPU, the calls raise.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch already loaded (both name it libamdhip64.so.7).
"""
from __future__ import annotations

import ctypes
import os

import torch

Q4_0, Q8_0, Q4_K, Q6_K = 0, 1, 2, 3
FORMATS = {"q4_0": Q4_0, "q8_0": Q8_0, "q4_k": Q4_K, "q6_k": Q6_K}
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqmat.so")
_lib = None


class QmatError(RuntimeError):
    """A non-zero status returned by the C ABI."""

    def __init__(self, func: str, status: int, message: str):
        super().__init__(f"{func}: {message} (status {status})")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libqmat.so once (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m block_quantized_weight_qmat_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.qmat_block_elems.argtypes = [i32]
    lib.qmat_block_elems.restype = i64
    lib.qmat_block_bytes.argtypes = [i32]
    lib.qmat_block_bytes.restype = i64
    lib.qmat_row_bytes.argtypes = [i32, i64]
    lib.qmat_row_bytes.restype = i64
    lib.qmat_strerror.argtypes = [i32]
    lib.qmat_strerror.restype = ctypes.c_char_p
    lib.qmat_quantize.argtypes = [i32, p, p, i64, i64, p]
    lib.qmat_quantize.restype = i32
    lib.qmat_gemv.argtypes = [i32, p, p, p, i64, i64, p]
    lib.qmat_gemv.restype = i32
    lib.qmat_gemm.argtypes = [i32, p, p, p, i64, i64, i64, p]
    lib.qmat_gemm.restype = i32
    lib.qmat_gemm_workspace_bytes.argtypes = [i32, i64, i64, i64]
    lib.qmat_gemm_workspace_bytes.restype = i64
    lib.qmat_gemm_ws.argtypes = [i32, p, p, p, i64, i64, i64, p, i64, p]
    lib.qmat_gemm_ws.restype = i32
    lib.qmat_prefill.argtypes = [i32, p, p, p, p, i64, i64, i64, p]
    lib.qmat_prefill.restype = i32
    lib.qmat_kv_write.argtypes = [i32, p, p, p, i64, i64, i64, i64, p]
    lib.qmat_kv_write.restype = i32
    lib.qmat_gemv_batch.argtypes = [i32, p, i64, p]
    lib.qmat_gemv_batch.restype = i32
    lib.qmat_prefill_noalloc.argtypes = [i32, p, p, p, i64, i64, i64, p]
    lib.qmat_prefill_noalloc.restype = i32
    lib.qmat_noalloc_scratch_bytes.argtypes = []
    lib.qmat_noalloc_scratch_bytes.restype = i64
    _lib = lib
    return lib


def _fmt(fmt) -> int:
    f = FORMATS[fmt.lower()] if isinstance(fmt, str) else int(fmt)
    if f not in (Q4_0, Q8_0, Q4_K, Q6_K):
        raise ValueError(f"unknown format {fmt!r}")
    return f


def _check(func: str, status: int):
    if status != 0:
        msg = load_library().qmat_strerror(status).decode()
        raise QmatError(func, status, msg)


def block_elems(fmt) -> int:
    return int(load_library().qmat_block_elems(_fmt(fmt)))


def block_bytes(fmt) -> int:
    return int(load_library().qmat_block_bytes(_fmt(fmt)))


def row_bytes(fmt, K: int) -> int:
    rb = int(load_library().qmat_row_bytes(_fmt(fmt), int(K)))
    if rb < 0:
        raise ValueError(f"K={K} is not a multiple of the block size of format {fmt!r}")
    return rb


def _gpu(t: torch.Tensor, name: str, dtype: torch.dtype):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor (no CPU path exists)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def quantize(fmt, W: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 [rows, K] -> uint8 [rows, row_bytes(fmt, K)] packed blocks."""
    f = _fmt(fmt)
    _gpu(W, "W", torch.float32)
    if W.dim() != 2:
        raise ValueError("W must be 2-D [rows, K]")
    rows, K = W.shape
    rb = row_bytes(f, K)
    if out is None:
        out = torch.empty((rows, rb), dtype=torch.uint8, device=W.device)
    _gpu(out, "out", torch.uint8)
    if out.numel() != rows * rb:
        raise ValueError("out has the wrong size")
    _check("qmat_quantize", load_library().qmat_quantize(
        f, W.data_ptr(), out.data_ptr(), rows, K, _stream(W)))
    return out


def gemv(fmt, blocks: torch.Tensor, x: torch.Tensor, M: int, K: int,
         out: torch.Tensor | None = None) -> torch.Tensor:
    """y[M] = dequant(W) @ x, W given as packed blocks of M rows of K."""
    f = _fmt(fmt)
    _gpu(blocks, "blocks", torch.uint8)
    _gpu(x, "x", torch.float32)
    if blocks.numel() != M * row_bytes(f, K) or x.numel() != K:
        raise ValueError("blocks or x does not match M, K")
    if out is None:
        out = torch.empty(M, dtype=torch.float32, device=x.device)
    _gpu(out, "out", torch.float32)
    if out.numel() != M:
        raise ValueError("out must hold M values")
    _check("qmat_gemv", load_library().qmat_gemv(
        f, blocks.data_ptr(), x.data_ptr(), out.data_ptr(), M, K, _stream(x)))
    return out


class GemvJob(ctypes.Structure):
    """One job of gemv_batch (the C struct qmat_gemv_job)."""
    _fields_ = [("blocks", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("K", ctypes.c_int64)]


def gemv_jobs(fmt, items) -> ctypes.Array:
    """A job array for gemv_batch from (blocks, x, y, M, K) tuples of GPU
    tensors; it keeps raw pointers, so the tensors must outlive its use."""
    f = _fmt(fmt)
    arr = (GemvJob * len(items))()
    for i, (blocks, x, y, M, K) in enumerate(items):
        _gpu(blocks, "blocks", torch.uint8)
        _gpu(x, "x", torch.float32)
        _gpu(y, "y", torch.float32)
        if blocks.numel() != M * row_bytes(f, K) or x.numel() != K or y.numel() != M:
            raise ValueError(f"job {i}: blocks, x or y does not match M, K")
        arr[i] = GemvJob(blocks.data_ptr(), x.data_ptr(), y.data_ptr(), M, K)
    return arr


def gemv_batch(fmt, jobs, stream_of: torch.Tensor | None = None):
    """Run many GEMVs (a gemv_jobs array, or (blocks, x, y, M, K) tuples) in
    as few launches as possible, on torch's current stream."""
    f = _fmt(fmt)
    arr = jobs if isinstance(jobs, ctypes.Array) else gemv_jobs(f, jobs)
    dev = stream_of.device if stream_of is not None else torch.device("cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    _check("qmat_gemv_batch", load_library().qmat_gemv_batch(
        f, ctypes.cast(arr, ctypes.c_void_p), len(arr), st))


def gemm(fmt, blocks: torch.Tensor, Xq: torch.Tensor, M: int, K: int, N: int,
         out: torch.Tensor | None = None) -> torch.Tensor:
    """Y[N, M] = dequant(Xq) @ dequant(W)^T; Xq are Q8_0 activation blocks."""
    f = _fmt(fmt)
    _gpu(blocks, "blocks", torch.uint8)
    _gpu(Xq, "Xq", torch.uint8)
    if blocks.numel() != M * row_bytes(f, K) or Xq.numel() != N * row_bytes(Q8_0, K):
        raise ValueError("blocks or Xq does not match M, K, N")
    if out is None:
        out = torch.empty((N, M), dtype=torch.float32, device=Xq.device)
    _gpu(out, "out", torch.float32)
    if out.numel() != N * M:
        raise ValueError("out must hold N*M values")
    _check("qmat_gemm", load_library().qmat_gemm(
        f, blocks.data_ptr(), Xq.data_ptr(), out.data_ptr(), M, K, N, _stream(Xq)))
    return out


def gemm_workspace_bytes(fmt, M: int, K: int, N: int) -> int:
    """Workspace bytes gemm_ws needs for this product (0: none)."""
    n = int(load_library().qmat_gemm_workspace_bytes(_fmt(fmt), M, K, N))
    if n < 0:
        raise ValueError(f"invalid gemm shape M={M} K={K} N={N} for format {fmt}")
    return n


def gemm_ws(fmt, blocks: torch.Tensor, Xq: torch.Tensor, M: int, K: int, N: int,
            out: torch.Tensor | None = None,
            workspace: torch.Tensor | None = None) -> torch.Tensor:
    """gemm with a workspace, so that a product of few tiles is also split
    along K; a workspace of gemm_workspace_bytes() bytes is allocated when
    none is given."""
    f = _fmt(fmt)
    _gpu(blocks, "blocks", torch.uint8)
    _gpu(Xq, "Xq", torch.uint8)
    if blocks.numel() != M * row_bytes(f, K) or Xq.numel() != N * row_bytes(Q8_0, K):
        raise ValueError("blocks or Xq does not match M, K, N")
    if out is None:
        out = torch.empty((N, M), dtype=torch.float32, device=Xq.device)
    _gpu(out, "out", torch.float32)
    if out.numel() != N * M:
        raise ValueError("out must hold N*M values")
    need = gemm_workspace_bytes(f, M, K, N)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=Xq.device)
    if workspace is not None:
        _gpu(workspace, "workspace", torch.uint8)
    wp = workspace.data_ptr() if workspace is not None else None
    wn = workspace.numel() if workspace is not None else 0
    _check("qmat_gemm_ws", load_library().qmat_gemm_ws(
        f, blocks.data_ptr(), Xq.data_ptr(), out.data_ptr(), M, K, N, wp, wn, _stream(Xq)))
    return out


def prefill(fmt, blocks: torch.Tensor, X: torch.Tensor, M: int,
            out: torch.Tensor | None = None,
            xq: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Y[N, M] = dequant(Q8_0(X)) @ dequant(W)^T from fp32 X [N, K] in one
    call; returns (Y, xq), xq being the Q8_0 activation blocks it wrote."""
    f = _fmt(fmt)
    _gpu(blocks, "blocks", torch.uint8)
    _gpu(X, "X", torch.float32)
    if X.dim() != 2:
        raise ValueError("X must be 2-D [N, K]")
    N, K = X.shape
    if blocks.numel() != M * row_bytes(f, K):
        raise ValueError("blocks do not match M, K")
    if xq is None:
        xq = torch.empty((N, row_bytes(Q8_0, K)), dtype=torch.uint8, device=X.device)
    _gpu(xq, "xq", torch.uint8)
    if xq.numel() != N * row_bytes(Q8_0, K):
        raise ValueError("xq has the wrong size")
    if out is None:
        out = torch.empty((N, M), dtype=torch.float32, device=X.device)
    _gpu(out, "out", torch.float32)
    if out.numel() != N * M:
        raise ValueError("out must hold N*M values")
    _check("qmat_prefill", load_library().qmat_prefill(
        f, blocks.data_ptr(), X.data_ptr(), xq.data_ptr(), out.data_ptr(), M, K, N, _stream(X)))
    return out, xq


def noalloc_scratch_bytes() -> int:
    """Size of the static device workspace of prefill_noalloc."""
    return int(load_library().qmat_noalloc_scratch_bytes())


def prefill_noalloc(fmt, blocks: torch.Tensor, X: torch.Tensor, M: int,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """prefill() with the Q8_0 activation workspace in the library's static
    device array instead of a caller buffer (nothing is allocated when out
    is given); calls that overlap on one device race on that workspace."""
    f = _fmt(fmt)
    _gpu(blocks, "blocks", torch.uint8)
    _gpu(X, "X", torch.float32)
    if X.dim() != 2:
        raise ValueError("X must be 2-D [N, K]")
    N, K = X.shape
    if blocks.numel() != M * row_bytes(f, K):
        raise ValueError("blocks do not match M, K")
    if out is None:
        out = torch.empty((N, M), dtype=torch.float32, device=X.device)
    _gpu(out, "out", torch.float32)
    if out.numel() != N * M:
        raise ValueError("out must hold N*M values")
    _check("qmat_prefill_noalloc", load_library().qmat_prefill_noalloc(
        f, blocks.data_ptr(), X.data_ptr(), out.data_ptr(), M, K, N, _stream(X)))
    return out


def kv_write(fmt, rows: torch.Tensor, cache: torch.Tensor, cell0: int,
             bias: torch.Tensor | None = None) -> torch.Tensor:
    """Quantize rows [n, dim] (minus bias [dim] if given) into cache rows
    cell0 .. cell0 + n - 1 (cache: uint8 [cells, row_bytes(fmt, dim)])."""
    f = _fmt(fmt)
    _gpu(rows, "rows", torch.float32)
    _gpu(cache, "cache", torch.uint8)
    if rows.dim() != 2 or cache.dim() != 2:
        raise ValueError("rows and cache must be 2-D")
    n, dim = rows.shape
    if cache.shape[1] != row_bytes(f, dim):
        raise ValueError("cache rows do not match fmt and dim")
    bp = 0
    if bias is not None:
        _gpu(bias, "bias", torch.float32)
        if bias.numel() != dim:
            raise ValueError("bias must hold dim values")
        bp = bias.data_ptr()
    _check("qmat_kv_write", load_library().qmat_kv_write(
        f, rows.data_ptr(), bp or None, cache.data_ptr(), int(cell0), n, cache.shape[0], dim,
        _stream(rows)))
    return cache
