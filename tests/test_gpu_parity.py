"""Parity of the HIP library (through the C ABI) with the CPU oracle.

Bar: quantized bytes (codes and scales, weights and activations) identical;
GEMV relative L2 error <= 1e-3 and GEMM <= 2e-3 against the fp64 oracle,
with no NaN or Inf. GEMV/GEMM inputs are the oracle's own quantized bytes, so
the products are checked independently of the GPU quantizer. Sizes span
several tiles with ragged tails; the full workload sizes are checked in
full (quantizers, GEMV) or on sampled outputs (GEMM).
"""
import sys

import numpy as np
import pytest

import oracle
from block_quantized_weight_qmat_amd import inputs

pytestmark = pytest.mark.gpu

GEMV_TOL = 1e-3
GEMM_TOL = 2e-3


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


def dev_tensor(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def rel_l2(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(a)), "non-finite output"
    den = np.linalg.norm(ref)
    num = np.linalg.norm(a - ref)
    return num / den if den > 0 else num


def mixed_matrix(rng, rows, K):
    """Rows drawn from several populations: N(0,0.02) with outliers, N(0,1),
    heavy tails, tiny (fp16-subnormal scales), zero rows, all-negative and
    all-positive rows, and values that sit exactly on rounding ties."""
    W = rng.normal(0, 0.02, (rows, K))
    kinds = rng.integers(0, 8, rows)
    for r in range(rows):
        k = kinds[r]
        if k == 1:
            W[r] = rng.normal(0, 1.0, K)
        elif k == 2:
            W[r] = rng.standard_t(2, K) * 0.01
        elif k == 3:
            W[r] = rng.normal(0, 1e-6, K)
        elif k == 4:
            W[r] = 0.0
        elif k == 5:
            W[r] = -np.abs(rng.normal(0, 0.5, K))
        elif k == 6:
            W[r] = np.abs(rng.normal(0, 0.5, K))
        elif k == 7:
            # 3.5 sets a Q4_0 scale of exactly 0.5; multiples of 0.25 then
            # land on ties of the rounding (x/D = k + 0.5)
            W[r] = rng.integers(-14, 15, K) * 0.25
            W[r, ::32] = 3.5
    nout = max(1, rows * K // 3200)
    W.reshape(-1)[rng.choice(rows * K, nout, replace=False)] = 0.2 * rng.choice([-1, 1], nout)
    return W.astype(np.float32)


# ------------------------------------------------------------- quantizers --

SMALL_SHAPES = {
    0: [(1, 32), (3, 32 * 37), (5, 256), (64, 1024), (33, 2048), (7, 32 * 345)],
    1: [(1, 32), (3, 32 * 37), (5, 256), (64, 1024), (33, 2048), (7, 32 * 345)],
    2: [(1, 256), (3, 768), (17, 4096), (5, 11008)],
    3: [(1, 256), (3, 768), (17, 4096), (5, 11008), (9, 256 * 9)],
}


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_quantize_bytes_identical_small(q, fmt):
    rng = np.random.default_rng(100 + fmt)
    for rows, K in SMALL_SHAPES[fmt]:
        say(f"quantize fmt={fmt} rows={rows} K={K}")
        W = mixed_matrix(rng, rows, K)
        got = host(q.quantize(fmt, dev_tensor(W)))
        ref = oracle.quantize(fmt, W)
        assert got.shape == ref.shape
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"fmt {fmt} {rows}x{K}: {len(bad)} bytes differ, first {bad[:4]}"


def test_quantize_edge_values(q):
    say("quantize edge values")
    # exact ties, fp16-subnormal and fp16-overflow-adjacent scales, +-0
    rows = []
    base = np.zeros(32, np.float32)
    t = base.copy(); t[0] = 3.5; t[1:9] = [1.25, -1.25, 0.25, -0.25, 2.75, -2.75, 0.75, -0.75]; rows.append(t)
    t = base.copy(); t[0] = 7 * 65504.0; t[1] = -1000.0; rows.append(t)           # d = 65504
    t = np.full(32, 6.1e-5 * 7, np.float32); rows.append(t)                        # d at the fp16 normal edge
    t = (np.arange(32) - 16).astype(np.float32) * 1e-7; rows.append(t)            # subnormal scale
    t = np.full(32, -0.0, np.float32); rows.append(t)
    t = np.full(32, 1e-30, np.float32); rows.append(t)                            # d rounds to 0
    t = base.copy(); t[5] = 127 * 0.25; t[6] = 0.125; t[7] = -0.375; rows.append(t)
    t = np.linspace(-1, 1, 32).astype(np.float32); rows.append(t)
    W = np.stack(rows)
    for fmt in (0, 1):
        got = host(q.quantize(fmt, dev_tensor(W)))
        assert np.array_equal(got, oracle.quantize(fmt, W)), fmt
    Wk = np.tile(W.reshape(1, -1), (3, 1))  # 3 superblocks of 256
    for fmt in (2, 3):
        got = host(q.quantize(fmt, dev_tensor(Wk)))
        assert np.array_equal(got, oracle.quantize(fmt, Wk)), fmt


def test_quantize_bytes_identical_full_sizes(q):
    for orient in (0, 1):
        W, _ = inputs.llama7b_layer(orient)
        for fmt in (0, 1, 2, 3):
            say(f"quantize full llama7b_layer orient={orient} fmt={fmt} {W.shape}")
            got = host(q.quantize(fmt, dev_tensor(W)))
            assert np.array_equal(got, oracle.quantize(fmt, W))
    say("quantize full prefill activations 512x11008 q8_0")
    _, X = inputs.prefill()
    assert np.array_equal(host(q.quantize(1, dev_tensor(X))), oracle.quantize(1, X))
    for shape in (0, 1):
        W, _ = inputs.q4k_rows(shape)
        say(f"quantize full q4k_rows {W.shape}")
        assert np.array_equal(host(q.quantize(2, dev_tensor(W))), oracle.quantize(2, W))


def test_kv_write_bytes(q):
    """KV-cache writes (with and without the per-channel bias) give the
    oracle's bytes in the written cells and leave every other byte alone."""
    import torch
    rng = np.random.default_rng(900)
    for fmt in (0, 1):
        for dim, cells, cell0, n, centred in (
                (256, 40, 0, 1, False), (256, 40, 7, 5, True), (1024, 64, 31, 33, True),
                (4096, 12, 1, 11, False), (1024, 16, 16, 0, True), (2048, 9, 0, 9, True),
                (32, 12, 8, 4, True), (96, 5, 0, 5, False),  # one and three blocks per row
                (1024, 16384, 16383, 1, True),  # a decode write into the last cell
                (1024, 16384, 512, 512, True),  # the 512-token prefill write
                (1024, 4096, 100, 2048, fmt == 0)):  # >= 1024 waves: 256-thread workgroups
            say(f"kv write fmt={fmt} dim={dim} cells={cells} cell0={cell0} n={n} bias={centred}")
            rb = oracle.row_bytes(fmt, dim)
            cache = rng.integers(0, 256, (cells, rb), dtype=np.uint8)
            mean = rng.normal(0, 3, dim).astype(np.float32)
            rows = (mean + rng.normal(0, 0.5, (n, dim))).astype(np.float32)
            rows[:, ::37] = 0.0
            bias = mean if centred else None
            dc = dev_tensor(cache)
            q.kv_write(fmt, dev_tensor(rows), dc, cell0, None if bias is None else dev_tensor(bias))
            want = oracle.kv_write(fmt, rows, bias, cache, cell0)
            assert np.array_equal(host(dc), want), (fmt, dim, cell0, n, centred)
    torch.cuda.synchronize()


# ------------------------------------------------------------------ GEMV --

def gemv_case(q, fmt, W, x):
    M, K = W.shape
    B = oracle.quantize(fmt, W)
    y = host(q.gemv(fmt, dev_tensor(B), dev_tensor(x), M, K))
    ref = oracle.gemv(fmt, B, x, M, K)
    return y, ref, B


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemv_small_and_ragged(q, fmt):
    rng = np.random.default_rng(200 + fmt)
    shapes = [(1, 256), (3, 512), (17, 2048), (31, 11008 if fmt >= 2 else 32 * 345), (70, 4096),
              (129, 1024), (9, 256 * 40), (6, 256 * 72), (64, 256 * 9), (200, 256 * 43),
              # rows of 256..512 slices take the row-per-wave kernel: its first
              # and last sizes, an odd strip count, and just past its limit
              (33, 8192), (20, 16384), (18, 256 * 33), (7, 256 * 65)]
    if fmt < 2:
        shapes += [(1, 32), (5, 32 * 37), (2, 64), (40, 32 * 1001), (100, 32 * 345),
                   (65, 32 * 1001), (130, 32 * 65), (19, 32 * 257), (21, 32 * 511),
                   (7, 32 * 513)]
    for M, K in shapes:
        say(f"gemv fmt={fmt} M={M} K={K}")
        W = mixed_matrix(rng, M, K) if M > 2 else rng.normal(0, 0.02, (M, K)).astype(np.float32)
        x = rng.normal(0, 1, K).astype(np.float32)
        y, ref, _ = gemv_case(q, fmt, W, x)
        assert rel_l2(y, ref) <= GEMV_TOL, (M, K, rel_l2(y, ref))


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemv_one_hot_gives_the_column(q, fmt):
    rng = np.random.default_rng(300)
    for M, K, k in [(40, 2048, k) for k in (0, 15, 16, 31, 32, 1000, 2047)] + \
                   [(70, 4096, k) for k in (0, 2047, 2048, 4095)] + \
                   [(35, 11008, k) for k in (0, 4100, 11007)]:
        W = rng.normal(0, 0.02, (M, K)).astype(np.float32)
        B = oracle.quantize(fmt, W)
        Wd = oracle.dequant(fmt, B, M, K)
        dB = dev_tensor(B)
        say(f"gemv one-hot fmt={fmt} M={M} K={K} k={k}")
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        y = host(q.gemv(fmt, dB, dev_tensor(x), M, K)).astype(np.float64)
        if fmt == 2:
            # S*q - O may round once in fp32
            assert np.allclose(y, Wd[:, k], rtol=2 ** -23, atol=0)
        else:
            assert np.array_equal(y, Wd[:, k])
        x[k] = -3.0
        y = host(q.gemv(fmt, dB, dev_tensor(x), M, K)).astype(np.float64)
        assert np.allclose(y, -3.0 * Wd[:, k], rtol=2 ** -22, atol=0)


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemv_activation_range(q, fmt):
    """Per-32 power-of-two prescaling keeps any finite x in fp16 range."""
    rng = np.random.default_rng(400)
    # K = 4096 and K = 11008 take the two GEMV kernels (rows of fewer or more
    # than 256 slices)
    cases = [(M, K, name, scale) for M, K in ((24, 4096), (70, 4096), (37, 11008))
             for name, scale in (("tiny", 1e-30), ("huge", 1e30), ("subnormal", 1e-40),
                                 ("mixed", None), ("binade-top", "top"))]
    for M, K, name, scale in cases:
        say(f"gemv x-range fmt={fmt} M={M} K={K} {name}")
        W = rng.normal(0, 0.02, (M, K)).astype(np.float32)
        x = rng.normal(0, 1, K)
        if scale == "top":
            # every slice's maximum is positive and just below a power of two
            # (the top of the fixed-point digit range after prescaling)
            x = rng.uniform(-0.9, 0.9, K)
            x[::32] = 1.0 - 2.0 ** -rng.integers(9, 24, K // 32)
            x *= np.repeat(2.0 ** rng.integers(-8, 8, K // 32), 32)
        elif scale is None:
            x *= np.repeat(10.0 ** rng.integers(-20, 20, K // 32), 32)
        else:
            x *= scale
        x = x.astype(np.float32)
        y, ref, _ = gemv_case(q, fmt, W, x)
        assert rel_l2(y, ref) <= GEMV_TOL, (name, rel_l2(y, ref))


def test_gemv_k_zero_and_tall(q):
    import torch
    say("gemv K=0")
    y = q.gemv(0, torch.empty(0, dtype=torch.uint8, device="cuda"),
               torch.empty(0, dtype=torch.float32, device="cuda"), 37, 0)
    assert np.array_equal(host(y), np.zeros(37, np.float32))
    say("gemv tall M=70000 K=64")
    rng = np.random.default_rng(5)
    W = rng.normal(0, 0.02, (70000, 64)).astype(np.float32)
    x = rng.normal(0, 1, 64).astype(np.float32)
    for fmt in (0, 1):
        y, ref, _ = gemv_case(q, fmt, W, x)
        assert rel_l2(y, ref) <= GEMV_TOL


def test_gemv_workloads_full(q):
    """Every matrix of the decode workloads, every output row."""
    W, x = inputs.gemv_1024()
    say("gemv gemv_1024 q4_0")
    y, ref, _ = gemv_case(q, 0, W, x)
    assert rel_l2(y, ref) <= GEMV_TOL
    for orient in (0, 1):
        W, x = inputs.llama7b_layer(orient)
        for fmt in (0, 1):
            say(f"gemv llama7b_layer orient={orient} fmt={fmt}")
            y, ref, _ = gemv_case(q, fmt, W, x)
            assert rel_l2(y, ref) <= GEMV_TOL
    for shape in (0, 1):
        W, x = inputs.q4k_rows(shape)
        for fmt in (2, 3):
            say(f"gemv q4k_rows {W.shape} fmt={fmt}")
            y, ref, _ = gemv_case(q, fmt, W, x)
            assert rel_l2(y, ref) <= GEMV_TOL
    for orient in (0, 1):
        W, x = inputs.llama7b_layer(orient)
        say(f"gemv llama7b_layer orient={orient} fmt=3")
        y, ref, _ = gemv_case(q, 3, W, x)
        assert rel_l2(y, ref) <= GEMV_TOL


def test_gemv_qwen3_decode_set(q):
    worst = {0: 0.0, 1: 0.0}
    for i in range(len(inputs.qwen3_shapes())):
        name, W, x = inputs.qwen3_matrix(i)
        if i % 28 == 0:
            say(f"gemv qwen3 set matrix {i} {name} {W.shape}")
        for fmt in (0, 1):
            y, ref, _ = gemv_case(q, fmt, W, x)
            e = rel_l2(y, ref)
            worst[fmt] = max(worst[fmt], e)
            assert e <= GEMV_TOL, (name, fmt, e)
    say(f"gemv qwen3 worst rel_l2 {worst}")


def test_gemv_deterministic(q):
    W, x = inputs.llama7b_layer(0)
    B = dev_tensor(oracle.quantize(0, W))
    dx = dev_tensor(x)
    a = host(q.gemv(0, B, dx, 4096, 11008))
    b = host(q.gemv(0, B, dx, 4096, 11008))
    assert np.array_equal(a, b)


def test_gemv_two_streams(q):
    """Calls in flight on two streams at once."""
    import torch
    rng = np.random.default_rng(6)
    cases = []
    for M, K in ((4096, 11008), (300, 32 * 345)):
        W = rng.normal(0, 0.02, (M, K)).astype(np.float32)
        x = rng.normal(0, 1, K).astype(np.float32)
        B = oracle.quantize(0, W)
        cases.append((dev_tensor(B), dev_tensor(x), M, K, oracle.gemv(0, B, x, M, K)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = []
    for rep in range(4):
        say(f"gemv two streams rep {rep}")
        for (dB, dx, M, K, _), st in zip(cases, streams):
            with torch.cuda.stream(st):
                outs.append((q.gemv(0, dB, dx, M, K), M, K))
    torch.cuda.synchronize()
    for i, (y, M, K) in enumerate(outs):
        ref = cases[i % 2][4]
        assert rel_l2(host(y), ref) <= GEMV_TOL, (i, M, K)
        assert np.array_equal(host(y), host(outs[i % 2][0]))


# ------------------------------------------------------------------ GEMM --

def gemm_case(q, fmt, W, X):
    M, K = W.shape
    N = X.shape[0]
    B = oracle.quantize(fmt, W)
    Xq = oracle.quantize(1, X)
    Y = host(q.gemm(fmt, dev_tensor(B), dev_tensor(Xq), M, K, N))
    ref = oracle.gemm(fmt, B, Xq, M, K, N)
    return Y, ref


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemm_small_and_ragged(q, fmt):
    rng = np.random.default_rng(500 + fmt)
    shapes = [(96, 1024, 40), (130, 2048, 3), (257, 768, 17), (128, 4096, 64), (1, 256, 1),
              (200, 256 * 9, 130)]
    if fmt < 2:
        shapes += [(1, 32, 1), (33, 32 * 37, 5), (65, 32 * 5, 66)]
        # last stages of 3, 4 and 7 blocks: the two compute waves of a tile
        # split a stage's 8 blocks 4 + 4, so these leave the second share
        # short or empty and the first one full or short
        shapes += [(130, 32 * 11, 64), (129, 32 * 12, 65), (128, 32 * 23, 70)]
    for M, K, N in shapes:
        say(f"gemm fmt={fmt} M={M} K={K} N={N}")
        W = mixed_matrix(rng, M, K) if M > 2 else rng.normal(0, 0.02, (M, K)).astype(np.float32)
        X = rng.normal(0, 1, (N, K)).astype(np.float32)
        Y, ref = gemm_case(q, fmt, W, X)
        assert Y.shape == (N, M)
        assert rel_l2(Y, ref) <= GEMM_TOL, (M, K, N, rel_l2(Y, ref))


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemm_decode_small_n(q, fmt):
    """Few-token products (the decode batch path, up to 48 tokens, in chunks
    of 16): every token count around the chunk sizes, odd row strides,
    ragged row counts, and the switch to the MFMA path after 48 tokens."""
    rng = np.random.default_rng(700 + fmt)
    K1 = 256 * 9 if fmt >= 2 else 32 * 345  # odd block count per row
    cases = [(97, K1, n) for n in (1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 33, 48, 49)]
    cases += [(1, 256, 3), (2, 512, 16), (1000, 1024, 4), (33, 2048, 12)]
    if fmt < 2:
        cases += [(5, 32, 2), (64, 32 * 37, 6)]
    for M, K, N in cases:
        say(f"gemm decode fmt={fmt} M={M} K={K} N={N}")
        W = mixed_matrix(rng, M, K) if M > 2 else rng.normal(0, 0.02, (M, K)).astype(np.float32)
        X = rng.normal(0, 1, (N, K)).astype(np.float32)
        Y, ref = gemm_case(q, fmt, W, X)
        assert Y.shape == (N, M)
        assert rel_l2(Y, ref) <= GEMM_TOL, (M, K, N, rel_l2(Y, ref))


def test_gemm_decode_full_size_sampled(q):
    """The 4096 x 11008 layer with 4, 16 and 48 tokens (the decode batch
    path), checked on sampled rows against the oracle, and deterministic."""
    import torch
    W, X = inputs.llama7b_layer(0)
    M, K = W.shape
    rng = np.random.default_rng(11)
    Xs = rng.normal(0, 1, (48, K)).astype(np.float32)
    for fmt in (0, 1, 2, 3):
        dW = q.quantize(fmt, dev_tensor(W))
        Bh = host(dW)
        rb = oracle.row_bytes(fmt, K)
        for N in (4, 16, 48):
            say(f"gemm decode full fmt={fmt} N={N}")
            dXq = q.quantize(1, dev_tensor(Xs[:N]))
            Xq = host(dXq)
            Y = host(q.gemm(fmt, dW, dXq, M, K, N))
            assert np.all(np.isfinite(Y))
            rows = np.sort(rng.choice(M, 40, replace=False))
            ref = oracle.gemm(fmt, Bh.reshape(M, rb)[rows], Xq, len(rows), K, N)
            assert rel_l2(Y[:, rows], ref) <= GEMM_TOL, (fmt, N, rel_l2(Y[:, rows], ref))
            if N == 16:
                assert np.array_equal(Y, host(q.gemm(fmt, dW, dXq, M, K, N)))
        del dW
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemm_k_zero(q, fmt):
    """Empty sums: both the decode-batch path (7 tokens) and the MFMA tiles
    (70 tokens, ragged in M and N) write zeros over whatever Y held."""
    import torch
    e = torch.empty(0, dtype=torch.uint8, device="cuda")
    for N in (7, 70):
        say(f"gemm K=0 fmt={fmt} N={N}")
        Y = torch.full((N, 133), 3.0, dtype=torch.float32, device="cuda")
        q.gemm(fmt, e, e, 133, 0, N, out=Y)
        assert np.array_equal(host(Y), np.zeros((N, 133), np.float32))


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_prefill_one_call(q, fmt):
    """qmat_prefill: its workspace holds the oracle's Q8_0 activation bytes,
    and its product is qmat_gemm's on them (same bits) and within the GEMM
    bound of the oracle; a decode batch, an MFMA-sized batch and a ragged one."""
    import torch
    rng = np.random.default_rng(800 + fmt)
    for M, K, N in ((97, 256 * 9, 4), (130, 2048, 70), (64, 256 * 3, 1)):
        say(f"prefill one call fmt={fmt} M={M} K={K} N={N}")
        W = mixed_matrix(rng, M, K)
        X = rng.normal(0, 1, (N, K)).astype(np.float32)
        dB = dev_tensor(oracle.quantize(fmt, W))
        Y, xq = q.prefill(fmt, dB, dev_tensor(X), M)
        Xq = oracle.quantize(1, X)
        assert np.array_equal(host(xq), Xq)
        assert np.array_equal(host(Y), host(q.gemm(fmt, dB, xq, M, K, N)))
        ref = oracle.gemm(fmt, oracle.quantize(fmt, W), Xq, M, K, N)
        assert rel_l2(host(Y), ref) <= GEMM_TOL
    # K = 0: nothing to quantize, and every output is an empty sum
    say(f"prefill one call fmt={fmt} K=0")
    Y0 = torch.full((5, 7), 3.0, dtype=torch.float32, device="cuda")
    q.prefill(fmt, torch.empty((7, 0), dtype=torch.uint8, device="cuda"),
              torch.empty((5, 0), dtype=torch.float32, device="cuda"), 7, out=Y0)
    assert np.array_equal(host(Y0), np.zeros((5, 7), np.float32))
    torch.cuda.synchronize()


def test_prefill_full_size_sampled(q):
    """The prefill workload at full size, quantized on the GPU (bytes checked
    against the oracle), GEMM checked on sampled rows and tokens."""
    import torch
    M, K, N = inputs.PREFILL_SHAPE
    W, X = inputs.prefill()
    say("prefill full: quantize W and X on GPU")
    dB = q.quantize(0, dev_tensor(W))
    dXq = q.quantize(1, dev_tensor(X))
    B, Xq = host(dB), host(dXq)
    assert np.array_equal(B, oracle.quantize(0, W))
    assert np.array_equal(Xq, oracle.quantize(1, X))
    for fmt in (0, 1, 2, 3):
        say(f"prefill full gemm fmt={fmt}")
        if fmt == 0:
            dW = dB
            Bh = B
        else:
            dW = q.quantize(fmt, dev_tensor(W))
            Bh = host(dW)
        Y = host(q.gemm(fmt, dW, dXq, M, K, N))
        assert np.all(np.isfinite(Y))
        rng = np.random.default_rng(7 + fmt)
        rows = np.sort(rng.choice(M, 48, replace=False))
        toks = np.sort(rng.choice(N, 24, replace=False))
        rb = oracle.row_bytes(fmt, K)
        xb = oracle.row_bytes(1, K)
        ref = oracle.gemm(fmt, Bh.reshape(M, rb)[rows], Xq.reshape(N, xb)[toks], len(rows), K, len(toks))
        got = Y[np.ix_(toks, rows)]
        assert rel_l2(got, ref) <= GEMM_TOL, rel_l2(got, ref)
        if fmt == 0:
            Y2 = host(q.gemm(fmt, dW, dXq, M, K, N))
            assert np.array_equal(Y, Y2), "GEMM not deterministic"
    del dB, dXq
    torch.cuda.empty_cache()
