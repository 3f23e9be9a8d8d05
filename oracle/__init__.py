"""CPU oracle of the block-quantized weight matmul (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package; the product path
(the ``block_quantized_weight_qmat_amd`` package and its HIP library) never
does, and this package never imports the product path.

The arithmetic lives in ``qmat_oracle.c`` (plain C, fp64 accumulation,
IEEE fp32 quantizers); this file only marshals numpy arrays. Every function
cites its source passage in the C file. Format ids: 0 = Q4_0, 1 = Q8_0,
2 = Q4_K-style, 3 = Q6_K-style.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qmat_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

Q4_0, Q8_0, Q4_K, Q6_K = 0, 1, 2, 3
FORMATS = {"q4_0": Q4_0, "q8_0": Q8_0, "q4_k": Q4_K, "q6_k": Q6_K}

CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-fexcess-precision=standard", "-Wall", "-Wextra"]


def compile_c(src: str, out: str) -> str:
    """gcc-compile an oracle source file into a shared library."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle (IEEE fp32: no contraction, no fast-math)."""
    if not force and os.path.exists(LIB):
        return LIB
    return compile_c(SRC, LIB)


def _fmt(fmt) -> int:
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """One loaded copy of the oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_f16.restype = ctypes.c_uint16
        lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f32.restype = ctypes.c_float
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_f32_to_f16_array.argtypes = [p, p, i64]
        lib.oracle_f32_to_f16_array.restype = None
        lib.oracle_f16_to_f64_array.argtypes = [p, p, i64]
        lib.oracle_f16_to_f64_array.restype = None
        lib.oracle_block_elems.argtypes = [ctypes.c_int]
        lib.oracle_block_elems.restype = i64
        lib.oracle_block_bytes.argtypes = [ctypes.c_int]
        lib.oracle_block_bytes.restype = i64
        lib.oracle_quantize.argtypes = [ctypes.c_int, p, p, i64, i64]
        lib.oracle_quantize.restype = ctypes.c_int
        lib.oracle_dequant.argtypes = [ctypes.c_int, p, p, i64, i64]
        lib.oracle_dequant.restype = ctypes.c_int
        lib.oracle_gemv.argtypes = [ctypes.c_int, p, p, p, i64, i64]
        lib.oracle_gemv.restype = ctypes.c_int
        lib.oracle_gemm.argtypes = [ctypes.c_int, p, p, p, i64, i64, i64]
        lib.oracle_gemm.restype = ctypes.c_int
        lib.oracle_kv_write.argtypes = [ctypes.c_int, p, p, p, i64, i64, i64, i64]
        lib.oracle_kv_write.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    # sizes -----------------------------------------------------------------
    def block_elems(self, fmt) -> int:
        return int(self.lib.oracle_block_elems(_fmt(fmt)))

    def block_bytes(self, fmt) -> int:
        return int(self.lib.oracle_block_bytes(_fmt(fmt)))

    def row_bytes(self, fmt, K: int) -> int:
        be = self.block_elems(fmt)
        assert be > 0 and K % be == 0
        return K // be * self.block_bytes(fmt)

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def set_threads(self, n: int) -> int:
        """OpenMP threads for later calls; returns the number in effect."""
        return int(self.lib.oracle_set_threads(int(n)))

    # fp16 ------------------------------------------------------------------
    def f32_to_f16_bits(self, v: float) -> int:
        return int(self.lib.oracle_f32_to_f16(ctypes.c_float(v)))

    def f16_bits_to_f64(self, h: int) -> float:
        return float(self.lib.oracle_f16_to_f64(ctypes.c_uint16(h)))

    def f32_to_f16_array(self, v: np.ndarray) -> np.ndarray:
        """binary16 bit patterns (uint16) of float32 values."""
        v = np.ascontiguousarray(v, dtype=np.float32).reshape(-1)
        out = np.empty(v.size, dtype=np.uint16)
        self.lib.oracle_f32_to_f16_array(_ptr(v), _ptr(out), v.size)
        return out

    def f16_to_f64_array(self, h: np.ndarray) -> np.ndarray:
        """float64 values of binary16 bit patterns (uint16)."""
        h = np.ascontiguousarray(h, dtype=np.uint16).reshape(-1)
        out = np.empty(h.size, dtype=np.float64)
        self.lib.oracle_f16_to_f64_array(_ptr(h), _ptr(out), h.size)
        return out

    # method ----------------------------------------------------------------
    def quantize(self, fmt, W: np.ndarray) -> np.ndarray:
        """fp32 [rows][K] -> uint8 [rows][row_bytes]."""
        f = _fmt(fmt)
        W = np.ascontiguousarray(W, dtype=np.float32)
        assert W.ndim == 2
        rows, K = W.shape
        out = np.empty((rows, self.row_bytes(f, K)), dtype=np.uint8)
        rc = self.lib.oracle_quantize(f, _ptr(W), _ptr(out), rows, K)
        if rc != 0:
            raise ValueError(f"oracle_quantize failed ({rc})")
        return out

    def dequant(self, fmt, blocks: np.ndarray, rows: int, K: int) -> np.ndarray:
        """uint8 blocks -> fp64 [rows][K] (exact)."""
        f = _fmt(fmt)
        blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
        assert blocks.size == rows * self.row_bytes(f, K)
        out = np.empty((rows, K), dtype=np.float64)
        rc = self.lib.oracle_dequant(f, _ptr(blocks), _ptr(out), rows, K)
        if rc != 0:
            raise ValueError(f"oracle_dequant failed ({rc})")
        return out

    def gemv(self, fmt, blocks: np.ndarray, x: np.ndarray, M: int, K: int) -> np.ndarray:
        """fp64 y[M] = dequant(W) @ x."""
        f = _fmt(fmt)
        blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
        x = np.ascontiguousarray(x, dtype=np.float32)
        assert blocks.size == M * self.row_bytes(f, K) and x.size == K
        y = np.empty(M, dtype=np.float64)
        rc = self.lib.oracle_gemv(f, _ptr(blocks), _ptr(x), _ptr(y), M, K)
        if rc != 0:
            raise ValueError(f"oracle_gemv failed ({rc})")
        return y

    def gemm(self, fmt, blocks: np.ndarray, Xq8: np.ndarray, M: int, K: int, N: int) -> np.ndarray:
        """fp64 Y[N][M] = dequant(Xq8) @ dequant(W)^T."""
        f = _fmt(fmt)
        blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
        Xq8 = np.ascontiguousarray(Xq8, dtype=np.uint8)
        assert blocks.size == M * self.row_bytes(f, K)
        assert Xq8.size == N * self.row_bytes(Q8_0, K)
        Y = np.empty((N, M), dtype=np.float64)
        rc = self.lib.oracle_gemm(f, _ptr(blocks), _ptr(Xq8), _ptr(Y), M, K, N)
        if rc != 0:
            raise ValueError(f"oracle_gemm failed ({rc})")
        return Y


    def kv_write(self, fmt, rows: np.ndarray, bias, cache: np.ndarray, cell0: int) -> np.ndarray:
        """Quantize rows [n][dim] (minus bias [dim] if given) into a copy of
        cache (uint8 [cells][row_bytes]) at rows cell0..; returns the copy."""
        f = _fmt(fmt)
        rows = np.ascontiguousarray(rows, dtype=np.float32)
        n, dim = rows.shape
        out = np.array(cache, dtype=np.uint8, copy=True, order="C")
        cells = out.shape[0]
        assert out.shape[1] == self.row_bytes(f, dim)
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        rc = self.lib.oracle_kv_write(f, _ptr(rows), None if b is None else _ptr(b), _ptr(out),
                                      cell0, n, cells, dim)
        if rc != 0:
            raise ValueError(f"oracle_kv_write failed ({rc})")
        return out


_default = None


def default() -> Oracle:
    """The oracle built from qmat_oracle.c (compiled on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB):
            build()
        _default = Oracle(LIB)
    return _default


def __getattr__(name):
    # Module-level shortcuts: oracle.quantize(...), oracle.gemv(...), ...
    if not name.startswith("_") and hasattr(Oracle, name):
        return getattr(default(), name)
    raise AttributeError(name)
