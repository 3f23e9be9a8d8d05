"""The C-ABI library: loads, exports every symbol include/qmat.h declares, and
rejects bad arguments on the host, before anything is enqueued (no GPU is
needed for any of these: every case returns before the first HIP call)."""
import ctypes
import os
import re

import pytest

import oracle
from block_quantized_weight_qmat_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmat.h")

OK, E_FMT, E_SHAPE, E_NULL, E_HIP, E_ALIGN, E_SCRATCH, E_WORKSPACE = 0, 1, 2, 3, 4, 5, 6, 7


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        pytest.skip("libqmat.so not built")
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmat_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("qmat_quantize", "qmat_gemv", "qmat_gemm", "qmat_block_elems",
              "qmat_block_bytes", "qmat_row_bytes", "qmat_strerror"):
        assert n in names


def test_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_enum_values_match_header():
    text = open(HEADER).read()
    vals = dict(re.findall(r"\b(QMAT_[A-Z0-9_]+)\s*=\s*(\d+)", text))
    assert vals["QMAT_Q4_0"] == "0" and vals["QMAT_Q8_0"] == "1" and vals["QMAT_Q4_K"] == "2"
    assert vals["QMAT_Q6_K"] == "3"
    assert binding.Q4_0 == 0 and binding.Q8_0 == 1 and binding.Q4_K == 2 and binding.Q6_K == 3
    assert [vals[k] for k in ("QMAT_OK", "QMAT_E_FMT", "QMAT_E_SHAPE", "QMAT_E_NULL",
                              "QMAT_E_HIP", "QMAT_E_ALIGN", "QMAT_E_SCRATCH",
                              "QMAT_E_WORKSPACE")] == \
        ["0", "1", "2", "3", "4", "5", "6", "7"]


def test_sizes_agree_with_oracle(lib):
    for f in (0, 1, 2, 3):
        assert lib.qmat_block_elems(f) == oracle.block_elems(f)
        assert lib.qmat_block_bytes(f) == oracle.block_bytes(f)
        for K in (0, 256, 11008 if f < 2 else 4096, 2 ** 20):
            assert lib.qmat_row_bytes(f, K) == oracle.row_bytes(f, K)
    assert lib.qmat_block_elems(7) == 0 and lib.qmat_block_bytes(-1) == 0
    assert lib.qmat_row_bytes(0, 33) == -1 and lib.qmat_row_bytes(2, 32) == -1
    assert lib.qmat_row_bytes(0, -32) == -1 and lib.qmat_row_bytes(9, 32) == -1


def test_strerror(lib):
    for s in range(8):
        assert len(lib.qmat_strerror(s)) > 3
    assert lib.qmat_strerror(99) == b"unknown status"


A = 0x10000  # a 16-byte aligned fake address: never dereferenced (rejected first)


def test_bad_format(lib):
    assert lib.qmat_quantize(4, A, A, 1, 32, None) == E_FMT
    assert lib.qmat_gemv(-1, A, A, A, 1, 32, None) == E_FMT
    assert lib.qmat_gemm(5, A, A, A, 1, 32, 1, None) == E_FMT


def test_bad_shapes(lib):
    assert lib.qmat_quantize(0, A, A, 1, 48, None) == E_SHAPE      # K % 32
    assert lib.qmat_quantize(2, A, A, 1, 288, None) == E_SHAPE     # K % 256
    assert lib.qmat_quantize(3, A, A, 1, 288, None) == E_SHAPE     # K % 256
    assert lib.qmat_quantize(1, A, A, -1, 32, None) == E_SHAPE
    assert lib.qmat_gemv(0, A, A, A, -5, 32, None) == E_SHAPE
    assert lib.qmat_gemv(0, A, A, A, 1, -32, None) == E_SHAPE
    assert lib.qmat_gemv(0, A, A, A, 2 ** 31, 32, None) == E_SHAPE  # M beyond 2^31-1
    assert lib.qmat_gemv(0, A, A, A, 1, 2 ** 31 + 32, None) == E_SHAPE
    assert lib.qmat_gemm(0, A, A, A, 1, 32, -1, None) == E_SHAPE
    assert lib.qmat_gemm(2, A, A, A, 1, 32, 1, None) == E_SHAPE    # Q4_K needs K % 256
    assert lib.qmat_gemm(0, A, A, A, 1, 2 ** 24 + 32, 1, None) == E_SHAPE  # GEMM K limit


def test_null_and_alignment(lib):
    assert lib.qmat_quantize(0, None, A, 1, 32, None) == E_NULL
    assert lib.qmat_quantize(0, A, None, 1, 32, None) == E_NULL
    assert lib.qmat_gemv(0, A, None, A, 1, 32, None) == E_NULL
    assert lib.qmat_gemv(0, A, A, None, 1, 32, None) == E_NULL
    assert lib.qmat_gemm(0, A, A, None, 1, 32, 1, None) == E_NULL
    assert lib.qmat_gemm(0, A, None, A, 1, 32, 1, None) == E_NULL
    assert lib.qmat_quantize(0, A + 4, A, 1, 32, None) == E_ALIGN
    assert lib.qmat_gemv(0, A + 2, A, A, 1, 32, None) == E_ALIGN
    assert lib.qmat_gemm(1, A, A + 8, A, 1, 32, 1, None) == E_ALIGN


def test_empty_work_is_ok_with_null_pointers(lib):
    # nothing to read or write: nothing is enqueued, no pointer is needed
    assert lib.qmat_quantize(0, None, None, 0, 32, None) == OK
    assert lib.qmat_quantize(2, None, None, 5, 0, None) == OK
    assert lib.qmat_gemv(1, None, None, None, 0, 64, None) == OK
    assert lib.qmat_gemm(0, None, None, None, 0, 64, 3, None) == OK
    assert lib.qmat_gemm(0, None, None, None, 3, 64, 0, None) == OK


def test_binding_refuses_cpu_tensors():
    import torch
    W = torch.zeros(2, 32)
    with pytest.raises(TypeError):
        binding.quantize("q4_0", W)


def test_product_path_does_not_use_the_oracle():
    pkg = os.path.join(ROOT, "block_quantized_weight_qmat_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text and "qmat_oracle" not in text, f


def test_kv_write_arguments(lib):
    f = lib.qmat_kv_write
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    f.restype = ctypes.c_int
    assert f(2, A, None, A, 0, 1, 4, 256, None) == E_FMT           # Q4_K is not a cache type
    assert f(3, A, None, A, 0, 1, 4, 256, None) == E_FMT
    assert f(0, A, None, A, 0, 1, 4, 48, None) == E_SHAPE          # dim % 32
    assert f(0, A, None, A, 3, 2, 4, 256, None) == E_SHAPE         # past the last cell
    assert f(0, A, None, A, -1, 1, 4, 256, None) == E_SHAPE
    assert f(1, A, None, A, 0, -1, 4, 256, None) == E_SHAPE
    assert f(0, None, None, A, 0, 0, 4, 256, None) == 0            # nothing to do
    assert f(0, None, None, A, 0, 1, 4, 256, None) == E_NULL
    assert f(0, A, None, None, 0, 1, 4, 256, None) == E_NULL
    assert f(0, A, A + 4, A, 0, 1, 4, 256, None) == E_ALIGN        # bias
    assert f(0, A, None, A, 1, 1, 4, 64, None) == E_ALIGN          # cell 1 of 36-byte rows


def test_prefill_arguments(lib):
    f = lib.qmat_prefill
    assert f(7, A, A, A, A, 1, 32, 1, None) == E_FMT
    assert f(0, A, A, A, A, 1, 48, 1, None) == E_SHAPE             # K % 32
    assert f(2, A, A, A, A, 1, 32, 1, None) == E_SHAPE             # Q4_K needs K % 256
    assert f(0, A, A, A, A, 1, 32, -1, None) == E_SHAPE
    assert f(0, A, A, A, A, 1, 2 ** 24 + 32, 1, None) == E_SHAPE   # GEMM K limit
    assert f(0, A, None, A, A, 1, 32, 1, None) == E_NULL           # X
    assert f(0, A, A, None, A, 1, 32, 1, None) == E_NULL           # workspace
    assert f(0, A, A, A, None, 1, 32, 1, None) == E_NULL           # Y
    assert f(0, A, A + 4, A, A, 1, 32, 1, None) == E_ALIGN
    assert f(0, A, A, A + 2, A, 1, 32, 1, None) == E_ALIGN
    assert f(0, None, None, None, None, 0, 64, 3, None) == OK      # nothing to do
    assert f(0, None, None, None, None, 3, 64, 0, None) == OK


def test_measured_peak_library():
    """libqmat_micro.so (the benchmark's measured-peak kernels) exports its
    four entry points, and each refuses bad arguments before any HIP call."""
    path = os.path.join(os.path.dirname(binding.library_path()), "libqmat_micro.so")
    if not os.path.exists(path):
        pytest.skip("libqmat_micro.so not built")
    m = ctypes.CDLL(path)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    m.qmat_micro_read.argtypes = [P, i64, P, i32, P]
    for f in (m.qmat_micro_mfma_i8, m.qmat_micro_fma_f32, m.qmat_micro_mix):
        f.argtypes = [i32, P, i32, P]
    assert m.qmat_micro_read(None, 64, A, 1, None) == 1
    assert m.qmat_micro_read(A, 40, A, 1, None) == 1       # not a multiple of 16 bytes
    assert m.qmat_micro_read(A, 64, A, 0, None) == 1
    assert m.qmat_micro_mfma_i8(0, A, 1, None) == 1
    assert m.qmat_micro_fma_f32(1, None, 1, None) == 1
    assert m.qmat_micro_mix(8, A, 1, None) == 1            # fewer than 16 iterations


def test_prefill_noalloc_arguments(lib):
    """The allocation-free prefill checks its arguments as qmat_prefill does,
    then its workspace limit, all before any HIP call."""
    f = lib.qmat_prefill_noalloc
    assert lib.qmat_noalloc_scratch_bytes() == 16 << 20
    K = 11008
    n_over = (16 << 20) // oracle.row_bytes(1, K) + 1
    assert f(4, A, A, A, 1, K, 1, None) == E_FMT
    assert f(0, A, A, A, 1, 48, 1, None) == E_SHAPE
    assert f(0, A, A, A, 1, 2 ** 24 + 32, 1, None) == E_SHAPE
    assert f(0, A, A, A, 4, K, n_over, None) == E_SCRATCH
    assert f(0, None, None, None, 0, K, n_over, None) == OK   # M == 0: nothing to do
    assert f(0, A, None, A, 4, K, 2, None) == E_NULL
    assert f(0, A, A + 4, A, 4, K, 2, None) == E_ALIGN


def test_documented_departures_from_the_planned_header(lib):
    """The boundary's documented departures, each as documented: an int
    format (out-of-range values are ordinary arguments), signed size helpers
    that report errors, the 16-byte alignment rule, the GEMM's K limit, and
    Python calls that take the shape."""
    import inspect
    assert lib.qmat_block_elems(2 ** 31 - 1) == 0 and lib.qmat_row_bytes(-7, 32) == -1
    assert lib.qmat_gemv(2 ** 31 - 1, A, A, A, 1, 32, None) == E_FMT
    assert lib.qmat_row_bytes(0, 31) == -1 and lib.qmat_row_bytes(0, 2 ** 40) == 2 ** 35 * 18
    for off in (1, 2, 4, 8):
        assert lib.qmat_gemv(0, A, A, A + off, 1, 32, None) == E_ALIGN
    assert lib.qmat_gemm(0, A, A, A, 1, 2 ** 24 + 32, 1, None) == E_SHAPE
    assert lib.qmat_prefill(0, A, A, A, A, 1, 2 ** 24 + 32, 1, None) == E_SHAPE
    assert list(inspect.signature(binding.gemv).parameters)[:5] == ["fmt", "blocks", "x", "M", "K"]
    assert list(inspect.signature(binding.gemm).parameters)[:6] == ["fmt", "blocks", "Xq", "M", "K", "N"]
    import block_quantized_weight_qmat_amd as pkg
    for name in pkg.__all__:
        assert getattr(pkg, name) is not None, name


def test_gemv_batch_arguments(lib):
    """Every job is checked before anything is enqueued; a bad one anywhere
    fails the whole call with its status."""
    J = binding.GemvJob
    good = J(A, A, A, 64, 1024)
    arr = (J * 3)(good, good, good)
    f = lib.qmat_gemv_batch
    p = ctypes.cast(arr, ctypes.c_void_p)
    assert f(9, p, 3, None) == E_FMT
    assert f(0, p, -1, None) == E_SHAPE
    assert f(0, None, 2, None) == E_NULL
    assert f(0, None, 0, None) == OK
    arr[2] = J(A, A, A, 64, 48)
    assert f(0, p, 3, None) == E_SHAPE
    arr[2] = J(A, A, A + 8, 64, 1024)
    assert f(0, p, 3, None) == E_ALIGN
    arr[2] = J(A, None, A, 64, 1024)
    assert f(0, p, 3, None) == E_NULL
    assert ctypes.sizeof(J) == 40


def test_gemm_ws_arguments(lib):
    """The workspace size is a function of the shape (0 when the product is
    not split, (splits - 1) * N * M * 4 otherwise); qmat_gemm_ws checks
    qmat_gemm's arguments, then the workspace, all before any HIP call."""
    wb, f = lib.qmat_gemm_workspace_bytes, lib.qmat_gemm_ws
    M, K = 4096, 11008
    assert wb(0, M, K, 16) == 0 and wb(0, M, K, 512) == 0 and wb(0, 0, K, 64) == 0
    need = wb(0, M, K, 64)
    assert need == 7 * 64 * M * 4                      # eight K ranges
    assert wb(1, M, K, 64) == need and wb(3, M, K, 64) == need
    assert wb(0, 11008, 4096, 64) == 1 * 64 * 11008 * 4
    assert wb(5, M, K, 64) == -1 and wb(2, M, 32, 64) == -1
    assert wb(0, M, 2 ** 24 + 32, 64) == -1 and wb(0, -1, K, 64) == -1
    assert f(7, A, A, A, M, K, 64, A, need, None) == E_FMT
    assert f(0, A, A, A, M, K, -1, A, need, None) == E_SHAPE
    assert f(0, A, A, None, M, K, 64, A, need, None) == E_NULL
    assert f(0, A, A + 4, A, M, K, 64, A, need, None) == E_ALIGN
    assert f(0, A, A, A, M, K, 64, A, -1, None) == E_SHAPE
    assert f(0, A, A, A, M, K, 64, None, need, None) == E_WORKSPACE
    assert f(0, A, A, A, M, K, 64, A, need - 1, None) == E_WORKSPACE
    assert f(0, A, A, A, M, K, 64, A + 8, need, None) == E_ALIGN
    assert f(0, None, None, None, 0, K, 64, None, 0, None) == OK   # nothing to do
    assert b"workspace" in lib.qmat_strerror(E_WORKSPACE)


def test_gemm_split_policy_properties(lib):
    """The K-split policy on seeded random shapes (host code only): the
    workspace holds whole partial products, at most 16 ranges of at least
    two stages each (Q6_K-style: whole pairs of stages), none below 17
    tokens, and the tiles of all ranges stay within 2^24."""
    import numpy as np
    rng = np.random.default_rng(7)
    wb = lib.qmat_gemm_workspace_bytes
    for _ in range(3000):
        f = int(rng.integers(0, 4))
        be = 256 if f >= 2 else 32
        M = int(rng.integers(1, 40000))
        K = be * int(rng.integers(1, 2 ** 24 // be // 64))
        N = int(rng.integers(1, 4000))
        b = wb(f, M, K, N)
        assert b >= 0 and b % (4 * N * M) == 0, (f, M, K, N, b)
        splits = b // (4 * N * M) + 1
        nst = -(-(K // 32) // 8)
        unit = 2 if f == 3 else 1
        assert splits <= 16
        if N < 17:
            assert splits == 1
        if splits > 1:
            units = -(-nst // unit)
            assert -(-units // splits) * unit >= 2          # stages of the longest range
            assert splits <= units
            tiles = -(-M // 128) * -(-N // 64)
            assert tiles * splits <= 2 ** 24
