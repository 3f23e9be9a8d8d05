"""Parity of the HIP library (through the C ABI) with the CPU oracle.

Bar: quantized bytes (codes and scales, weights and activations) identical;
GEMV relative L2 error <= 1e-3 and GEMM <= 2e-3 against the fp64 oracle,
with no NaN or Inf. GEMV/GEMM inputs are the oracle's own quantized bytes, so
the products are checked independently of the GPU quantizer. Sizes span
several tiles with ragged tails; the full workload sizes are checked in
full, every output element against the oracle.

Every output buffer is filled with a sentinel before the call (NaN for the
float outputs, so an element the kernel skips fails the finiteness check)
and carries a guard tail past its end that must come back unchanged.
"""
import sys

import numpy as np
import pytest

import oracle
from block_quantized_weight_qmat_amd import inputs

pytestmark = pytest.mark.gpu

GEMV_TOL = 1e-3
GEMM_TOL = 2e-3
GUARD = 4096  # elements (bytes for uint8 outputs) past the end of each output
F32_GUARD = -1.2345e-38  # a float no kernel writes
U8_FILL, U8_GUARD = 0xA5, 0x5A


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


class Guarded:
    """An output buffer of `shape` prefilled with a sentinel (NaN for float32,
    0xA5 for bytes), followed by GUARD elements of a second sentinel; `out`
    is the view the library writes, `check()` asserts the tail is intact."""

    def __init__(self, shape, dtype="f32"):
        import torch
        self.n = int(np.prod(shape))
        if dtype == "f32":
            buf = torch.full((self.n + GUARD,), float("nan"), dtype=torch.float32, device="cuda")
            buf[self.n:] = F32_GUARD
        else:
            buf = torch.full((self.n + GUARD,), U8_FILL, dtype=torch.uint8, device="cuda")
            buf[self.n:] = U8_GUARD
        self.buf = buf
        self.out = buf[:self.n].view(*shape) if len(shape) else buf[:self.n]

    def check(self):
        tail = host(self.buf[self.n:])
        if tail.dtype == np.float32:
            ok = np.array_equal(tail.view(np.uint32),
                                np.full(GUARD, F32_GUARD, np.float32).view(np.uint32))
        else:
            ok = np.all(tail == U8_GUARD)
        assert ok, "the kernel wrote past the end of its output"

    def get(self):
        v = host(self.out)
        self.check()
        return v


def rel_l2(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(a)), f"{np.count_nonzero(~np.isfinite(a))} non-finite outputs"
    den = np.linalg.norm(ref)
    num = np.linalg.norm(a - ref)
    return num / den if den > 0 else num


def check_close(a, ref, tol, what):
    """rel-L2 within tol; also reports the worst element (its absolute error
    relative to the largest reference value) so a single bad tile shows."""
    e = rel_l2(a, ref)
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = np.abs(a - ref)
    i = np.unravel_index(int(np.argmax(diff)), diff.shape) if diff.size else ()
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    worst = float(diff[i]) / scale if diff.size and scale > 0 else 0.0
    say(f"{what}: rel_l2 {e:.3e}, worst element {i} |err|/max|ref| {worst:.3e}")
    assert e <= tol, (what, e)
    return e


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


def gpu_quantize(q, fmt, W):
    """The GPU quantizer's bytes for W, written into a guarded buffer."""
    rows, K = W.shape
    g = Guarded((rows, oracle.row_bytes(fmt, K)), "u8")
    q.quantize(fmt, dev_tensor(W), out=g.out)
    return g.get()


def assert_bytes(got, ref, what):
    assert got.shape == ref.shape, what
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{what}: {len(bad)} bytes differ, first {bad[:4]}"


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_quantize_bytes_identical_small(q, fmt):
    rng = np.random.default_rng(100 + fmt)
    for rows, K in SMALL_SHAPES[fmt]:
        say(f"quantize fmt={fmt} rows={rows} K={K}")
        W = mixed_matrix(rng, rows, K)
        assert_bytes(gpu_quantize(q, fmt, W), oracle.quantize(fmt, W), f"fmt {fmt} {rows}x{K}")



def random_shape(rng, be, max_elems, max_rows=20000, max_k=32768):
    """A seeded (rows, K) pair: rows log-uniform in [1, max_rows], K a
    log-uniform multiple of the block size be, rows * K <= max_elems."""
    K = be * int(np.exp(rng.uniform(0, np.log(max_k // be))))
    rows = int(np.exp(rng.uniform(0, np.log(min(max_rows, max(1, max_elems // K))))))
    return max(1, rows), max(be, K)


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_quantize_random_shapes(q, fmt):
    """Seeded random shapes: the quantizer's launch shape (lanes per block,
    blocks per wave, workgroups) follows rows and K."""
    rng = np.random.default_rng(150 + fmt)
    be = 256 if fmt >= 2 else 32
    for i in range(10):
        rows, K = random_shape(rng, be, 3_000_000)
        say(f"quantize random fmt={fmt} case {i}: rows={rows} K={K}")
        W = mixed_matrix(rng, rows, K)
        assert_bytes(gpu_quantize(q, fmt, W), oracle.quantize(fmt, W), f"fmt {fmt} {rows}x{K}")

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
        assert_bytes(gpu_quantize(q, fmt, W), oracle.quantize(fmt, W), f"edge fmt {fmt}")
    Wk = np.tile(W.reshape(1, -1), (3, 1))  # 3 superblocks of 256
    for fmt in (2, 3):
        assert_bytes(gpu_quantize(q, fmt, Wk), oracle.quantize(fmt, Wk), f"edge fmt {fmt}")


def test_quantize_bytes_identical_full_sizes(q):
    for orient in (0, 1):
        W, _ = inputs.llama7b_layer(orient)
        for fmt in (0, 1, 2, 3):
            say(f"quantize full llama7b_layer orient={orient} fmt={fmt} {W.shape}")
            assert_bytes(gpu_quantize(q, fmt, W), oracle.quantize(fmt, W), f"llama7b {orient} {fmt}")
    say("quantize full prefill activations 512x11008 q8_0")
    _, X = inputs.prefill()
    assert_bytes(gpu_quantize(q, 1, X), oracle.quantize(1, X), "activations")
    for shape in (0, 1):
        W, _ = inputs.q4k_rows(shape)
        for fmt in (2, 3):
            say(f"quantize full q4k_rows {W.shape} fmt={fmt}")
            assert_bytes(gpu_quantize(q, fmt, W), oracle.quantize(fmt, W), f"q4k_rows {shape}")
    W, _ = inputs.gemv_1024()
    say("quantize full gemv_1024 q4_0")
    assert_bytes(gpu_quantize(q, 0, W), oracle.quantize(0, W), "gemv_1024")


def test_quantize_qwen3_decode_set(q):
    """The GPU quantizer on all 196 matrices of the Qwen3-0.6B-like set (with
    their 1% outlier blocks), Q4_0 and Q8_0, bytes against the oracle."""
    for i in range(len(inputs.qwen3_shapes())):
        name, W, _ = inputs.qwen3_matrix(i)
        if i % 28 == 0:
            say(f"quantize qwen3 set matrix {i} {name} {W.shape}")
        for fmt in (0, 1):
            assert_bytes(gpu_quantize(q, fmt, W), oracle.quantize(fmt, W), f"{name} fmt {fmt}")


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
            g = Guarded((cells, rb), "u8")
            g.out.copy_(dev_tensor(cache))
            q.kv_write(fmt, dev_tensor(rows), g.out, cell0,
                       None if bias is None else dev_tensor(bias))
            want = oracle.kv_write(fmt, rows, bias, cache, cell0)
            assert np.array_equal(g.get(), want), (fmt, dim, cell0, n, centred)
    torch.cuda.synchronize()


# ------------------------------------------------------------------ GEMV --

def gpu_gemv(q, fmt, dB, dx, M, K):
    g = Guarded((M,))
    q.gemv(fmt, dB, dx, M, K, out=g.out)
    return g.get()


def gemv_case(q, fmt, W, x):
    M, K = W.shape
    B = oracle.quantize(fmt, W)
    y = gpu_gemv(q, fmt, dev_tensor(B), dev_tensor(x), M, K)
    ref = oracle.gemv(fmt, B, x, M, K)
    return y, ref, B


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemv_small_and_ragged(q, fmt):
    rng = np.random.default_rng(200 + fmt)
    shapes = [(1, 256), (3, 512), (17, 2048), (31, 11008 if fmt >= 2 else 32 * 345), (70, 4096),
              (129, 1024), (9, 256 * 40), (6, 256 * 72), (64, 256 * 9), (200, 256 * 43),
              # rows of 256..512 slices take the row-per-wave kernel: its first
              # and last sizes, an odd strip count, and just past its limit
              (33, 8192), (20, 16384), (18, 256 * 33), (7, 256 * 65),
              # rows of at most 32 slices: both halves of a wave take rows
              (40, 256), (33, 768), (16, 1024), (2, 1024), (100, 512),
              # a million elements per row: many passes of the strip kernel
              (3, 1 << 20), (70, 1 << 17)]
    if fmt < 2:
        shapes += [(1, 32), (5, 32 * 37), (2, 64), (40, 32 * 1001), (100, 32 * 345),
                   (65, 32 * 1001), (130, 32 * 65), (19, 32 * 257), (21, 32 * 511),
                   (7, 32 * 513),
                   # pair mode with odd row strides (an odd slice count)
                   (17, 32), (2, 32), (3, 32 * 3), (37, 32 * 31), (50, 32 * 17), (33, 32 * 5),
                   (16, 32 * 33)]
    for M, K in shapes:
        say(f"gemv fmt={fmt} M={M} K={K}")
        W = mixed_matrix(rng, M, K) if M > 2 else rng.normal(0, 0.02, (M, K)).astype(np.float32)
        x = rng.normal(0, 1, K).astype(np.float32)
        y, ref, _ = gemv_case(q, fmt, W, x)
        assert rel_l2(y, ref) <= GEMV_TOL, (M, K, rel_l2(y, ref))



@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemv_random_shapes(q, fmt):
    """Seeded random shapes across the GEMV's routes, which depend on rows
    and K: the strip kernel in its row-group shapes, the row-per-wave kernel
    with one or two rows per wave (tall matrices), ragged strips and tails."""
    rng = np.random.default_rng(250 + fmt)
    be = 256 if fmt >= 2 else 32
    for i in range(16):
        M, K = random_shape(rng, be, 24_000_000)
        say(f"gemv random fmt={fmt} case {i}: M={M} K={K}")
        W = rng.normal(0, 0.02, (M, K)).astype(np.float32)
        x = rng.normal(0, 1, K).astype(np.float32)
        y, ref, _ = gemv_case(q, fmt, W, x)
        check_close(y, ref, GEMV_TOL, f"gemv random fmt={fmt} M={M} K={K}")

@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemv_one_hot_gives_the_column(q, fmt):
    rng = np.random.default_rng(300)
    for M, K, k in [(40, 2048, k) for k in (0, 15, 16, 31, 32, 1000, 2047)] + \
                   [(40, 1024, k) for k in (0, 31, 32, 1023)] + \
                   ([(9, 32 * 31, k) for k in (0, 500, 991)] if fmt < 2 else []) + \
                   [(70, 4096, k) for k in (0, 2047, 2048, 4095)] + \
                   [(35, 11008, k) for k in (0, 4100, 11007)]:
        W = rng.normal(0, 0.02, (M, K)).astype(np.float32)
        B = oracle.quantize(fmt, W)
        Wd = oracle.dequant(fmt, B, M, K)
        dB = dev_tensor(B)
        say(f"gemv one-hot fmt={fmt} M={M} K={K} k={k}")
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        y = gpu_gemv(q, fmt, dB, dev_tensor(x), M, K).astype(np.float64)
        if fmt == 2:
            # S*q - O may round once in fp32
            assert np.allclose(y, Wd[:, k], rtol=2 ** -23, atol=0)
        else:
            assert np.array_equal(y, Wd[:, k])
        x[k] = -3.0
        y = gpu_gemv(q, fmt, dB, dev_tensor(x), M, K).astype(np.float64)
        assert np.allclose(y, -3.0 * Wd[:, k], rtol=2 ** -22, atol=0)


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemv_activation_range(q, fmt):
    """Per-32 power-of-two prescaling keeps any finite x in fp16 range."""
    rng = np.random.default_rng(400)
    # K = 4096 and K = 11008 take the two GEMV kernels (rows of fewer or more
    # than 256 slices), K = 1024 the strip kernel's pair mode
    cases = [(M, K, name, scale) for M, K in ((24, 4096), (70, 4096), (37, 11008), (40, 1024))
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
    y = gpu_gemv(q, 0, torch.empty(0, dtype=torch.uint8, device="cuda"),
                 torch.empty(0, dtype=torch.float32, device="cuda"), 37, 0)
    assert np.array_equal(y, np.zeros(37, np.float32))
    say("gemv tall M=70000 K=64")
    rng = np.random.default_rng(5)
    W = rng.normal(0, 0.02, (70000, 64)).astype(np.float32)
    x = rng.normal(0, 1, 64).astype(np.float32)
    for fmt in (0, 1):
        y, ref, _ = gemv_case(q, fmt, W, x)
        assert rel_l2(y, ref) <= GEMV_TOL


@pytest.mark.parametrize("fmt", [0, 2])
def test_gemv_tall_two_rows_per_wave(q, fmt):
    """Tall 4-bit matrices take the row kernel with two rows per wave: rows
    past M in the last workgroup, an odd row stride (Q4_0, K = 32 * 131),
    and a row count just past the switch; within the bound, with one-hot x
    giving a column exactly."""
    rng = np.random.default_rng(40 + fmt)
    shapes = [(12289, 4096), (14336 + 17, 256 * 17)]
    if fmt == 0:
        shapes.append((12300, 32 * 131))
    for M, K in shapes:
        say(f"gemv tall two rows fmt={fmt} M={M} K={K}")
        W = rng.normal(0, 0.02, (M, K)).astype(np.float32)
        x = rng.normal(0, 1, K).astype(np.float32)
        y, ref, _ = gemv_case(q, fmt, W, x)
        check_close(y, ref, GEMV_TOL, f"gemv tall fmt={fmt} M={M} K={K}")
    M, K = 12345, 4096
    W = rng.normal(0, 0.02, (M, K)).astype(np.float32)
    x = np.zeros(K, np.float32)
    x[1234] = 1.0
    y, _, B = gemv_case(q, fmt, W, x)
    col = oracle.dequant(fmt, B, M, K)[:, 1234]
    if fmt == 2:  # S*q - O may round once in fp32
        assert np.allclose(y.astype(np.float64), col, rtol=2 ** -23, atol=0)
    else:
        assert np.array_equal(y.astype(np.float64), col), "one-hot"


def test_gemv_workloads_full(q):
    """Every matrix of the decode workloads, every output row."""
    W, x = inputs.gemv_1024()
    y, ref, _ = gemv_case(q, 0, W, x)
    check_close(y, ref, GEMV_TOL, "gemv gemv_1024 q4_0")
    for orient in (0, 1):
        W, x = inputs.llama7b_layer(orient)
        for fmt in (0, 1, 2, 3):
            y, ref, _ = gemv_case(q, fmt, W, x)
            check_close(y, ref, GEMV_TOL, f"gemv llama7b_layer orient={orient} fmt={fmt}")
    for shape in (0, 1):
        W, x = inputs.q4k_rows(shape)
        for fmt in (2, 3):
            y, ref, _ = gemv_case(q, fmt, W, x)
            check_close(y, ref, GEMV_TOL, f"gemv q4k_rows {W.shape} fmt={fmt}")


def test_gemv_lm_head_full(q):
    """The Qwen3-like output head, 151936 x 1024 (a q6_K tensor in the pages'
    model file; Q4_0 as well): every row against the oracle, and the GPU
    quantizer's bytes against the oracle's."""
    W, x = inputs.qwen3_lm_head()
    for fmt in (3, 0):
        say(f"gemv lm_head fmt={fmt}")
        y, ref, B = gemv_case(q, fmt, W, x)
        check_close(y, ref, GEMV_TOL, f"gemv lm_head fmt={fmt}")
        assert_bytes(gpu_quantize(q, fmt, W), B, f"quantize lm_head fmt={fmt}")


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


def test_gemv_batch_qwen3_set(q):
    """The 196-matrix Qwen3-0.6B-like set as one batch (a few launches of up
    to 64 jobs): within the GEMV bound of the oracle (every 7th matrix),
    within 1e-5 of the one-matrix calls (which may add the partial sums in
    another order), and the same bits on a second batch call."""
    import torch
    for fmt in (0, 1):
        say(f"gemv batch qwen3 set fmt={fmt}")
        jobs, refs, guards, dev = [], [], [], []
        for i in range(len(inputs.qwen3_shapes())):
            _, W, x = inputs.qwen3_matrix(i)
            M, K = W.shape
            B = oracle.quantize(fmt, W)
            dB, dx = dev_tensor(B), dev_tensor(x)
            g = Guarded((M,))
            jobs.append((dB, dx, g.out, M, K))
            guards.append(g)
            dev.append((dB, dx))
            if i % 7 == 0:
                refs.append((i, oracle.gemv(fmt, B, x, M, K)))
        q.gemv_batch(fmt, jobs)
        torch.cuda.synchronize()
        first = [g.get() for g in guards]
        for i, ref in refs:
            assert rel_l2(first[i], ref) <= GEMV_TOL, (fmt, i)
        for i, (dB, dx) in enumerate(dev):
            M, K = jobs[i][3], jobs[i][4]
            one = gpu_gemv(q, fmt, dB, dx, M, K)
            assert rel_l2(first[i], one) <= 1e-5, (fmt, i, rel_l2(first[i], one))
        say(f"gemv batch qwen3 set fmt={fmt}: second call")
        for g in guards:
            g.out.fill_(float("nan"))
        q.gemv_batch(fmt, jobs)
        torch.cuda.synchronize()
        for i, g in enumerate(guards):
            assert np.array_equal(g.get().view(np.uint32), first[i].view(np.uint32)), (fmt, i)


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemv_batch_mixed(q, fmt):
    """Jobs of every kind in one call: rows for the row-per-wave kernel, odd
    row strides, a single row, M = 0 and K = 0 jobs, and more than 64 jobs
    (several launches); each output within the GEMV bound of the oracle and
    close to the one-matrix call (which may add the partial sums in another
    order: a single row's sum can differ by a few units in its last place),
    the same bits on a second call."""
    import torch
    rng = np.random.default_rng(1300 + fmt)
    # rows of 256-512 slices (the batched row kernel: several jobs per
    # launch, two strip counts, a single row, ragged workgroups)
    long_rows = [(70, 11008), (20, 8192), (33, 16384), (1, 8192), (17, 256 * 33)]
    if fmt < 2:
        shapes = long_rows + [(33, 32 * 37), (1, 32 * 37), (0, 1024), (19, 0), (129, 4096),
                              (200, 32 * 345), (9, 32 * 257)] + \
                 [(int(rng.integers(1, 90)), 32 * int(rng.integers(1, 200))) for _ in range(70)]
    else:
        shapes = long_rows + [(9, 256 * 9), (1, 256 * 9), (0, 1024), (19, 0), (129, 4096)] + \
                 [(int(rng.integers(1, 90)), 256 * int(rng.integers(1, 40))) for _ in range(70)]
    say(f"gemv batch mixed fmt={fmt}: {len(shapes)} jobs")
    jobs, guards, dev, refs = [], [], [], []
    for M, K in shapes:
        W = rng.normal(0, 0.02, (M, K)).astype(np.float32)
        x = rng.normal(0, 1, K).astype(np.float32)
        Bq = oracle.quantize(fmt, W) if M * K else None
        refs.append(oracle.gemv(fmt, Bq, x, M, K) if M * K else np.zeros(M))
        dB = dev_tensor(Bq) if M * K else torch.empty(
            M * oracle.row_bytes(fmt, K), dtype=torch.uint8, device="cuda")
        dx = dev_tensor(x) if K else torch.empty(0, dtype=torch.float32, device="cuda")
        g = Guarded((M,))
        jobs.append((dB, dx, g.out, M, K))
        guards.append(g)
        dev.append((dB, dx))
    q.gemv_batch(fmt, jobs)
    torch.cuda.synchronize()
    first = [g.get() for g in guards]
    for i, (M, K) in enumerate(shapes):
        if M == 0:
            continue
        one = gpu_gemv(q, fmt, dev[i][0], dev[i][1], M, K)
        if K == 0:
            assert np.array_equal(first[i], one) and not first[i].any(), (fmt, i)
        else:
            assert rel_l2(first[i], refs[i]) <= GEMV_TOL, (fmt, i, M, K)
            assert rel_l2(first[i], one) <= 1e-4, (fmt, i, M, K, rel_l2(first[i], one))
    for g in guards:
        g.out.fill_(float("nan"))
    q.gemv_batch(fmt, jobs)
    torch.cuda.synchronize()
    for i, (M, K) in enumerate(shapes):
        if M:
            assert np.array_equal(guards[i].get().view(np.uint32), first[i].view(np.uint32)), i


@pytest.mark.parametrize("orient", [0, 1])
def test_gemv_deterministic(q, orient):
    """Two calls into two separately NaN-filled buffers give the same bits
    (both orientations: the row-per-wave and the strip kernel)."""
    W, x = inputs.llama7b_layer(orient)
    M, K = W.shape
    for fmt in (0, 1, 2, 3):
        say(f"gemv deterministic orient={orient} fmt={fmt}")
        B = dev_tensor(oracle.quantize(fmt, W))
        dx = dev_tensor(x)
        a = gpu_gemv(q, fmt, B, dx, M, K)
        b = gpu_gemv(q, fmt, B, dx, M, K)
        assert np.all(np.isfinite(a))
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


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
                g = Guarded((M,))
                q.gemv(0, dB, dx, M, K, out=g.out)
                outs.append(g)
    torch.cuda.synchronize()
    for i, g in enumerate(outs):
        ref = cases[i % 2][4]
        y = g.get()
        assert rel_l2(y, ref) <= GEMV_TOL, i
        assert np.array_equal(y, outs[i % 2].get())


# ------------------------------------------------------------------ GEMM --

def gpu_gemm(q, fmt, dB, dXq, M, K, N):
    g = Guarded((N, M))
    q.gemm(fmt, dB, dXq, M, K, N, out=g.out)
    return g.get()


def gemm_case(q, fmt, W, X):
    M, K = W.shape
    N = X.shape[0]
    B = oracle.quantize(fmt, W)
    Xq = oracle.quantize(1, X)
    Y = gpu_gemm(q, fmt, dev_tensor(B), dev_tensor(Xq), M, K, N)
    ref = oracle.gemm(fmt, B, Xq, M, K, N)
    return Y, ref


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemm_small_and_ragged(q, fmt):
    rng = np.random.default_rng(500 + fmt)
    shapes = [(96, 1024, 40), (130, 2048, 3), (257, 768, 17), (128, 4096, 64), (1, 256, 1),
              (200, 256 * 9, 130),
              # 8 and 16 tiles of 128 x 64: the XCD-aware tile order
              (256, 1024, 256), (1024, 512, 128),
              # a few hundred tokens: part of the GPU idle, ragged last tiles
              (1000, 768, 300),
              # long rows: 128 stages per tile; and a decode-batch chunk
              # with 256 stages per row
              (200, 32768, 80), (130, 65536, 20)]
    if fmt < 2:
        shapes += [(1, 32, 1), (33, 32 * 37, 5), (65, 32 * 5, 66)]
        # last stages of 3, 4 and 7 blocks: the two compute waves of a tile
        # split a stage's 8 blocks 4 + 4, so these leave the second share
        # short or empty and the first one full or short
        shapes += [(130, 32 * 11, 64), (129, 32 * 12, 65), (128, 32 * 23, 70)]
    for M, K, N in shapes:
        W = mixed_matrix(rng, M, K) if M > 2 else rng.normal(0, 0.02, (M, K)).astype(np.float32)
        X = rng.normal(0, 1, (N, K)).astype(np.float32)
        Y, ref = gemm_case(q, fmt, W, X)
        assert Y.shape == (N, M)
        check_close(Y, ref, GEMM_TOL, f"gemm fmt={fmt} M={M} K={K} N={N}")


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemm_decode_small_n(q, fmt):
    """Few-token products (the decode batch path, in chunks of 16 tokens):
    every token count around the chunk sizes, odd row strides, ragged row
    counts, and token counts around the switch to the prefill tiles."""
    rng = np.random.default_rng(700 + fmt)
    K1 = 256 * 9 if fmt >= 2 else 32 * 345  # odd block count per row
    cases = [(97, K1, n) for n in (1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 33, 48, 49)]
    cases += [(1, 256, 3), (2, 512, 16), (1000, 1024, 4), (33, 2048, 12)]
    if fmt < 2:
        cases += [(5, 32, 2), (64, 32 * 37, 6)]
        # K a multiple of 256 takes the matrix-core kernel: every chunk size,
        # ragged rows, fewer stages than waves (K = 768), and stage rings that
        # wrap many times (K = 16384)
        cases += [(97, 256 * 9, n) for n in (1, 2, 3, 4, 5, 8, 9, 15, 16, 17, 33, 48)]
        cases += [(16, 2048, 16), (40, 768, 9), (17, 16384, 16), (300, 256 * 43, 7)]
    else:
        # 9 to 16 tokens take the matrix-core kernel (K a multiple of 256):
        # fewer stages than waves, rings that wrap many times, ragged rows,
        # and for Q6_K-style superblocks at every offset in their 16-byte
        # windows (odd superblock counts put rows at every even offset)
        cases += [(16, 2048, 16), (40, 768, 9), (17, 16384, 16), (300, 256 * 43, 12),
                  (33, 256 * 43, 16), (21, 256 * 7, 10)]
    for M, K, N in cases:
        say(f"gemm decode fmt={fmt} M={M} K={K} N={N}")
        W = mixed_matrix(rng, M, K) if M > 2 else rng.normal(0, 0.02, (M, K)).astype(np.float32)
        X = rng.normal(0, 1, (N, K)).astype(np.float32)
        Y, ref = gemm_case(q, fmt, W, X)
        assert Y.shape == (N, M)
        assert rel_l2(Y, ref) <= GEMM_TOL, (M, K, N, rel_l2(Y, ref))


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemm_decode_tall(q, fmt):
    """The matrix-core decode kernel's shape for matrices of more than 4096
    rows (more 16-row workgroups than CUs: 4 waves, 2-stage rings): just
    past the switch, ragged rows, 9 and 16 tokens, the 11008x4096 layer, and
    for Q4_0 an 8-token chunk on rows too long for the row-per-wave kernel;
    every output against the oracle."""
    rng = np.random.default_rng(760 + fmt)
    cases = [(4097, 1024, 16), (4200, 2304, 9), (5003, 256 * 7, 12), (11008, 4096, 16)]
    if fmt == 0:
        cases += [(5000, 8192, 8), (4352, 8192, 5)]
    if fmt == 1:
        # 5-8 tokens on rows too long for the row-per-wave kernel's LDS
        cases += [(4500, 20480, 8), (300, 20480, 6)]
    if fmt == 2:
        # Q4_K-style takes this shape from 5 tokens on tall matrices
        cases += [(4200, 2304, 5), (5003, 4096, 8)]
    for M, K, N in cases:
        say(f"gemm decode tall fmt={fmt} M={M} K={K} N={N}")
        W = rng.normal(0, 0.02, (M, K)).astype(np.float32)
        X = rng.normal(0, 1, (N, K)).astype(np.float32)
        Y, ref = gemm_case(q, fmt, W, X)
        check_close(Y, ref, GEMM_TOL, f"gemm decode tall fmt={fmt} M={M} K={K} N={N}")


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemm_decode_rows_limits(q, fmt):
    """The few-token row-per-wave kernel at the edges of what it takes: one
    slice per row, rows of 8 strips at 4 tokens (80 KB of LDS), 7 strips at
    8 tokens (140 KB), 8 strips at 8 tokens (too large: another kernel), odd
    row strides, a single row, and a row count that leaves the last
    workgroup's second row empty."""
    rng = np.random.default_rng(950 + fmt)
    if fmt < 2:
        cases = [(40, 32, 3), (1, 32, 8), (33, 32 * 17, 6), (17, 16384, 4), (9, 14336, 8),
                 (9, 16384, 8), (31, 16384 - 32, 2)]
    else:
        cases = [(40, 256, 3), (1, 256, 8), (17, 16384, 4), (9, 14336, 8), (9, 16384, 8),
                 (33, 256 * 7, 6)]
    for M, K, N in cases:
        say(f"gemm decode rows fmt={fmt} M={M} K={K} N={N}")
        W = mixed_matrix(rng, M, K) if M > 2 else rng.normal(0, 0.02, (M, K)).astype(np.float32)
        X = rng.normal(0, 1, (N, K)).astype(np.float32)
        Y, ref = gemm_case(q, fmt, W, X)
        assert Y.shape == (N, M)
        check_close(Y, ref, GEMM_TOL, f"gemm decode rows fmt={fmt} M={M} K={K} N={N}")


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemm_decode_full_size(q, fmt):
    """The 4096 x 11008 layer with 4, 8, 16 and 48 tokens (the decode batch
    path: the row-per-wave kernel, the matrix cores or the strip kernel by
    format), weights quantized on the GPU: every output against the oracle,
    and two calls into separately NaN-filled buffers give the same bits."""
    import torch
    W, _ = inputs.llama7b_layer(0)
    M, K = W.shape
    rng = np.random.default_rng(11)
    Xs = rng.normal(0, 1, (48, K)).astype(np.float32)
    dW = dev_tensor(gpu_quantize(q, fmt, W))
    Bh = host(dW)
    for N in (4, 8, 16, 48):
        dXq = dev_tensor(gpu_quantize(q, 1, Xs[:N]))
        Xq = host(dXq)
        Y = gpu_gemm(q, fmt, dW, dXq, M, K, N)
        ref = oracle.gemm(fmt, Bh, Xq, M, K, N)
        check_close(Y, ref, GEMM_TOL, f"gemm decode full fmt={fmt} N={N}")
        Y2 = gpu_gemm(q, fmt, dW, dXq, M, K, N)
        assert np.array_equal(Y.view(np.uint32), Y2.view(np.uint32)), "not deterministic"
    del dW
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemm_k_zero(q, fmt):
    """Empty sums: both the decode-batch path (7 tokens) and the MFMA tiles
    (70 tokens, ragged in M and N) write zeros over a NaN-filled Y."""
    import torch
    e = torch.empty(0, dtype=torch.uint8, device="cuda")
    for N in (7, 70):
        say(f"gemm K=0 fmt={fmt} N={N}")
        Y = gpu_gemm(q, fmt, e, e, 133, 0, N)
        assert np.array_equal(Y, np.zeros((N, 133), np.float32))


def gpu_gemm_ws(q, fmt, dB, dXq, M, K, N):
    """qmat_gemm_ws into a guarded Y, with a NaN-filled, guarded workspace of
    exactly the size it asks for: a partial product read before it is
    written shows as NaN, a write past the workspace trips the guard.
    Returns (Y, workspace bytes)."""
    import torch
    need = q.gemm_workspace_bytes(fmt, M, K, N)
    gw = Guarded((need // 4,)) if need else None
    g = Guarded((N, M))
    q.gemm_ws(fmt, dB, dXq, M, K, N, out=g.out,
              workspace=gw.out.view(torch.uint8) if gw is not None else None)
    Y = g.get()
    if gw is not None:
        gw.check()
    return Y, need


SPLIT_SHAPES = [
    (300, 256 * 43, 64),   # 3 tiles, 11-15 K ranges of 2-4 stages
    (257, 4096, 17),       # the fewest tokens that split: 8 ranges of 2 stages
    (130, 256 * 9, 100),   # 9 stages in 5 ranges (Q6_K-style: pairs, the last one single)
    (1000, 2048, 200),     # 32 tiles x 4 ranges: the XCD-aware order, ragged last tiles
    (200, 256 * 5, 48),    # 48 tokens: split here, the decode batch in qmat_gemm
]


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemm_ws_split(q, fmt):
    """qmat_gemm_ws on products it splits along K: every output against the
    oracle, against qmat_gemm's unsplit result (same block products, other
    summation order), and bit-identical over two calls; with no workspace
    needed it is qmat_gemm, bit for bit."""
    rng = np.random.default_rng(900 + fmt)
    shapes = list(SPLIT_SHAPES)
    if fmt < 2:
        shapes += [(64, 32 * 345, 33)]  # a last stage of one block
    for M, K, N in shapes:
        say(f"gemm_ws split fmt={fmt} M={M} K={K} N={N}")
        W = mixed_matrix(rng, M, K)
        X = rng.normal(0, 1, (N, K)).astype(np.float32)
        B, Xq = oracle.quantize(fmt, W), oracle.quantize(1, X)
        dB, dXq = dev_tensor(B), dev_tensor(Xq)
        Y, need = gpu_gemm_ws(q, fmt, dB, dXq, M, K, N)
        assert need > 0, "this shape is meant to split"
        ref = oracle.gemm(fmt, B, Xq, M, K, N)
        check_close(Y, ref, GEMM_TOL, f"gemm_ws fmt={fmt} M={M} K={K} N={N}")
        Yu = gpu_gemm(q, fmt, dB, dXq, M, K, N)
        assert rel_l2(Y, Yu) <= 1e-5, rel_l2(Y, Yu)
        Y2, _ = gpu_gemm_ws(q, fmt, dB, dXq, M, K, N)
        assert np.array_equal(Y.view(np.uint32), Y2.view(np.uint32)), "not deterministic"
    for M, K, N in ((97, 2048, 16), (129, 32 * 23 if fmt < 2 else 768, 70)):
        say(f"gemm_ws unsplit fmt={fmt} M={M} K={K} N={N}")
        W = mixed_matrix(rng, M, K)
        X = rng.normal(0, 1, (N, K)).astype(np.float32)
        dB, dXq = dev_tensor(oracle.quantize(fmt, W)), dev_tensor(oracle.quantize(1, X))
        Y, need = gpu_gemm_ws(q, fmt, dB, dXq, M, K, N)
        assert need == 0
        assert np.array_equal(Y.view(np.uint32), gpu_gemm(q, fmt, dB, dXq, M, K, N).view(np.uint32))


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemm_random_shapes(q, fmt):
    """Seeded random shapes across every path a product can take (decode
    batch kernels, unsplit and K-split tiles): qmat_gemm and qmat_gemm_ws
    against the oracle, each output buffer NaN-filled and guarded."""
    rng = np.random.default_rng(1000 + fmt)
    be = 256 if fmt >= 2 else 32
    for i in range(14):
        M = int(rng.integers(1, 700))
        K = be * int(rng.integers(1, 6144 // be + 1))
        N = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 80)),
                            int(rng.integers(80, 300))]))
        say(f"gemm random fmt={fmt} case {i}: M={M} K={K} N={N}")
        W = rng.normal(0, 0.05, (M, K)).astype(np.float32)
        X = rng.normal(0, 1, (N, K)).astype(np.float32)
        B, Xq = oracle.quantize(fmt, W), oracle.quantize(1, X)
        dB, dXq = dev_tensor(B), dev_tensor(Xq)
        ref = oracle.gemm(fmt, B, Xq, M, K, N)
        Y = gpu_gemm(q, fmt, dB, dXq, M, K, N)
        check_close(Y, ref, GEMM_TOL, f"gemm random fmt={fmt} M={M} K={K} N={N}")
        Yw, _ = gpu_gemm_ws(q, fmt, dB, dXq, M, K, N)
        check_close(Yw, ref, GEMM_TOL, f"gemm_ws random fmt={fmt} M={M} K={K} N={N}")


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemm_ws_full_size(q, fmt):
    """The 4096 x 11008 layer at 17, 64 and 192 tokens through qmat_gemm_ws
    (8, 8 and 2 K ranges), weights quantized on the GPU: every output
    against the oracle, and two calls give the same bits."""
    import torch
    W, _ = inputs.llama7b_layer(0)
    M, K = W.shape
    rng = np.random.default_rng(12)
    Xs = rng.normal(0, 1, (192, K)).astype(np.float32)
    dW = dev_tensor(gpu_quantize(q, fmt, W))
    Bh = host(dW)
    for N in (17, 64, 192):
        dXq = dev_tensor(gpu_quantize(q, 1, Xs[:N]))
        Xq = host(dXq)
        Y, need = gpu_gemm_ws(q, fmt, dW, dXq, M, K, N)
        assert need > 0
        ref = oracle.gemm(fmt, Bh, Xq, M, K, N)
        check_close(Y, ref, GEMM_TOL, f"gemm_ws full fmt={fmt} N={N}")
        Y2, _ = gpu_gemm_ws(q, fmt, dW, dXq, M, K, N)
        assert np.array_equal(Y.view(np.uint32), Y2.view(np.uint32)), "not deterministic"
    del dW
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_prefill_one_call(q, fmt):
    """qmat_prefill: its workspace holds the oracle's Q8_0 activation bytes,
    and its product is qmat_gemm's on them (same bits) and within the GEMM
    bound of the oracle; a decode batch, an MFMA-sized batch and a ragged one."""
    rng = np.random.default_rng(800 + fmt)
    for M, K, N in ((97, 256 * 9, 4), (130, 2048, 70), (64, 256 * 3, 1)):
        say(f"prefill one call fmt={fmt} M={M} K={K} N={N}")
        W = mixed_matrix(rng, M, K)
        X = rng.normal(0, 1, (N, K)).astype(np.float32)
        dB = dev_tensor(oracle.quantize(fmt, W))
        gY = Guarded((N, M))
        gx = Guarded((N, oracle.row_bytes(1, K)), "u8")
        q.prefill(fmt, dB, dev_tensor(X), M, out=gY.out, xq=gx.out)
        Y, xq = gY.get(), gx.get()
        Xq = oracle.quantize(1, X)
        assert np.array_equal(xq, Xq)
        assert np.array_equal(Y, gpu_gemm(q, fmt, dB, gx.out, M, K, N))
        ref = oracle.gemm(fmt, oracle.quantize(fmt, W), Xq, M, K, N)
        check_close(Y, ref, GEMM_TOL, f"prefill fmt={fmt} M={M} K={K} N={N}")
    # K = 0: nothing to quantize, and every output is an empty sum
    import torch
    say(f"prefill one call fmt={fmt} K=0")
    gY = Guarded((5, 7))
    q.prefill(fmt, torch.empty((7, 0), dtype=torch.uint8, device="cuda"),
              torch.empty((5, 0), dtype=torch.float32, device="cuda"), 7, out=gY.out)
    assert np.array_equal(gY.get(), np.zeros((5, 7), np.float32))


@pytest.fixture(scope="module")
def prefill_full(q):
    """The prefill workload at full size: W and X quantized on the GPU (bytes
    checked against the oracle), kept on the device for the GEMM tests."""
    M, K, N = inputs.PREFILL_SHAPE
    W, X = inputs.prefill()
    say("prefill full: quantize X on the GPU")
    xq = gpu_quantize(q, 1, X)
    assert_bytes(xq, oracle.quantize(1, X), "prefill activations")
    return W, dev_tensor(xq), xq


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_prefill_full_size(q, prefill_full, fmt):
    """4096 x 11008 x 512 in every format: all 2,097,152 outputs against the
    oracle (every tile, in the XCD-aware tile order), and two calls into
    separately NaN-filled buffers give the same bits."""
    import torch
    M, K, N = inputs.PREFILL_SHAPE
    W, dXq, Xq = prefill_full
    say(f"prefill full: quantize W fmt={fmt} on the GPU")
    Bh = gpu_quantize(q, fmt, W)
    assert_bytes(Bh, oracle.quantize(fmt, W), f"prefill W fmt {fmt}")
    dW = dev_tensor(Bh)
    Y = gpu_gemm(q, fmt, dW, dXq, M, K, N)
    ref = oracle.gemm(fmt, Bh, Xq, M, K, N)
    check_close(Y, ref, GEMM_TOL, f"prefill full gemm fmt={fmt}")
    Y2 = gpu_gemm(q, fmt, dW, dXq, M, K, N)
    assert np.array_equal(Y.view(np.uint32), Y2.view(np.uint32)), "GEMM not deterministic"
    del dW
    torch.cuda.empty_cache()
