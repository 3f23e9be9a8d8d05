"""qmat_prefill_noalloc against qmat_prefill, through the C ABI.

Two calls in a row on one device, the second with a smaller input than the
first (the static workspace keeps the first call's activations), each
compared bit for bit with qmat_prefill's output on the same inputs and
within the GEMM bound of the oracle; outputs are NaN-filled before the call
and carry a guard tail. The size limit and the empty case return without
touching the device.
"""
import sys

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

GEMM_TOL = 2e-3
GUARD = 1024
E_SCRATCH = 6


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def q():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_quantized_weight_qmat_amd import binding
    binding.load_library()
    return binding


def nan_out(N, M):
    """A NaN-filled [N, M] view with a guard tail behind it."""
    import torch
    buf = torch.full((N * M + GUARD,), float("nan"), dtype=torch.float32, device="cuda")
    buf[N * M:] = 7.0
    return buf, buf[:N * M].view(N, M)


def tail_intact(buf, n):
    import torch
    torch.cuda.synchronize()
    return bool(torch.all(buf[n:] == 7.0).item())


def test_noalloc_matches_prefill_two_calls(q):
    import torch
    rng = np.random.default_rng(1234)
    # (fmt, M, K, N): the first call fills most of the 16 MiB workspace
    # (1200 x 11008 activations = 14.0 MB), the second is smaller and
    # leaves the first one's bytes behind it, the third a decode batch
    cases = [(0, 512, 11008, 1200), (1, 130, 2048, 70), (2, 97, 256 * 9, 4)]
    assert cases[0][3] * oracle.row_bytes(1, cases[0][2]) <= q.noalloc_scratch_bytes()
    for fmt, M, K, N in cases:
        say(f"prefill_noalloc fmt={fmt} M={M} K={K} N={N}")
        W = rng.normal(0, 0.02, (M, K)).astype(np.float32)
        X = rng.normal(0, 1, (N, K)).astype(np.float32)
        B = oracle.quantize(fmt, W)
        dB = torch.from_numpy(B).cuda()
        dX = torch.from_numpy(X).cuda()
        bufa, ya = nan_out(N, M)
        q.prefill_noalloc(fmt, dB, dX, M, out=ya)
        bufb, yb = nan_out(N, M)
        q.prefill(fmt, dB, dX, M, out=yb)
        torch.cuda.synchronize()
        assert tail_intact(bufa, N * M) and tail_intact(bufb, N * M)
        a, b = ya.cpu().numpy(), yb.cpu().numpy()
        assert np.all(np.isfinite(a))
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "differs from qmat_prefill"
        ref = oracle.gemm(fmt, B, oracle.quantize(1, X), M, K, N)
        e = np.linalg.norm(a - ref) / np.linalg.norm(ref)
        say(f"  rel_l2 {e:.3e}")
        assert e <= GEMM_TOL


def test_noalloc_limits(q):
    import torch
    lib = q.load_library()
    K = 11008
    too_many = q.noalloc_scratch_bytes() // oracle.row_bytes(1, K) + 1
    A = 0x10000  # never dereferenced: the size check comes first
    assert lib.qmat_prefill_noalloc(0, A, A, A, 4, K, too_many, None) == E_SCRATCH
    assert lib.qmat_prefill_noalloc(0, None, None, None, 0, K, too_many - 1, None) == 0
    # the largest N that fits still runs (K = 256: one Q8_0 block row is 272 B)
    n_max = q.noalloc_scratch_bytes() // oracle.row_bytes(1, 256)
    say(f"prefill_noalloc at the limit N={n_max} K=256")
    rng = np.random.default_rng(5)
    W = rng.normal(0, 0.02, (64, 256)).astype(np.float32)
    X = rng.normal(0, 1, (n_max, 256)).astype(np.float32)
    B = oracle.quantize(0, W)
    dB, dX = torch.from_numpy(B).cuda(), torch.from_numpy(X).cuda()
    bufa, ya = nan_out(n_max, 64)
    q.prefill_noalloc(0, dB, dX, 64, out=ya)
    bufb, yb = nan_out(n_max, 64)
    q.prefill(0, dB, dX, 64, out=yb)
    torch.cuda.synchronize()
    assert tail_intact(bufa, n_max * 64)
    assert np.array_equal(ya.cpu().numpy().view(np.uint32), yb.cpu().numpy().view(np.uint32))
