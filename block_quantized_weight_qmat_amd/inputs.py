"""Seeded synthetic inputs for the block-quantized matmul workloads.

This module draws random numbers and shapes them; it holds none of the
quantization or matmul arithmetic. The tests, the benchmark and the smoke
check use it to feed the same arrays to the HIP library and to the CPU
oracle.

Recipe (numpy PCG64 generators). Every tensor of a workload has its own
generator ``numpy.random.default_rng([seed, index])`` so that any tensor can
be drawn on its own; values are float64 draws cast to float32.

Workloads (shapes of the models the pages measured with; the model files
themselves are not available, so these stand in for them):
  * ``gemv_1024``: W 1024x1024 ~ N(0, 0.02^2), x ~ N(0, 1).
  * ``qwen3_0p6b``: the decode weight set of a Qwen3-0.6B-like model
    (hidden 1024, 16 query heads and 8 key/value heads of 128, FFN 3072,
    28 layers): per layer attn_q 2048x1024, attn_k 1024x1024,
    attn_v 1024x1024, attn_output 1024x2048, ffn_gate 3072x1024,
    ffn_up 3072x1024, ffn_down 1024x3072 (rows x K). Weights ~ N(0, 0.02^2)
    with 1% of the 32-element blocks of each matrix holding one outlier of
    +-10 standard deviations (+-0.2) at a uniformly drawn position; one
    x ~ N(0, 1) per matrix.
  * ``qwen3_lm_head``: that model's output head, the tied token embedding
    (vocabulary 151936 x hidden 1024, a q6_K tensor in the pages' model
    file), W ~ N(0, 0.02^2) with the same 1% outlier blocks, x ~ N(0, 1).
  * ``llama7b_layer``: W 4096x11008 and 11008x4096 ~ N(0, 0.02^2),
    x ~ N(0, 1).
  * ``q4k_rows``: W 4096x4096 and 4096x11008, N(0, 0.02^2) times a per-row
    factor r with ln r ~ U[ln 0.5, ln 2]; x ~ N(0, 1).
  * ``prefill``: W 4096x11008 ~ N(0, 0.02^2), activations of 512 tokens
    X 512x11008 ~ N(0, 1).
"""
from __future__ import annotations

import numpy as np

WEIGHT_STD = 0.02


def _rng(seed: int, index: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(index)])


def normal(shape, std: float, seed: int, index: int) -> np.ndarray:
    """float32 array of N(0, std^2) draws."""
    return _rng(seed, index).normal(0.0, std, size=shape).astype(np.float32)


def with_outlier_blocks(W: np.ndarray, seed: int, index: int, frac: float = 0.01,
                        magnitude: float = 10 * WEIGHT_STD, block: int = 32) -> np.ndarray:
    """Copy of W where round(frac * #blocks) distinct 32-element blocks each get
    one element replaced by +-magnitude (random sign, random position)."""
    rows, K = W.shape
    nblk = rows * (K // block)
    count = int(round(frac * nblk))
    rng = _rng(seed, index)
    chosen = rng.choice(nblk, size=count, replace=False)
    pos = rng.integers(0, block, size=count)
    sign = np.where(rng.integers(0, 2, size=count) == 0, -1.0, 1.0)
    out = W.copy()
    flat = out.reshape(-1)
    flat[chosen * block + pos] = (sign * magnitude).astype(np.float32)
    return out


def with_row_spread(W: np.ndarray, seed: int, index: int, lo: float = 0.5,
                    hi: float = 2.0) -> np.ndarray:
    """W with each row multiplied by r, ln r ~ U[ln lo, ln hi]."""
    r = np.exp(_rng(seed, index).uniform(np.log(lo), np.log(hi), size=W.shape[0]))
    return (W.astype(np.float64) * r[:, None]).astype(np.float32)


# ---------------------------------------------------------------- workloads

def gemv_1024(seed: int = 0):
    W = normal((1024, 1024), WEIGHT_STD, seed, 0)
    x = normal((1024,), 1.0, seed, 1)
    return W, x


QWEN3_LAYER = (
    ("attn_q", 2048, 1024),
    ("attn_k", 1024, 1024),
    ("attn_v", 1024, 1024),
    ("attn_output", 1024, 2048),
    ("ffn_gate", 3072, 1024),
    ("ffn_up", 3072, 1024),
    ("ffn_down", 1024, 3072),
)
QWEN3_LAYERS = 28


def qwen3_shapes():
    """[(name, rows, K)] for the 196 decode matrices, layer by layer."""
    return [(f"blk.{l}.{n}", r, k) for l in range(QWEN3_LAYERS) for (n, r, k) in QWEN3_LAYER]


def qwen3_matrix(i: int, seed: int = 0):
    """(name, W, x) of matrix i (0..195) of the Qwen3-0.6B-like set."""
    name, rows, K = qwen3_shapes()[i]
    W = normal((rows, K), WEIGHT_STD, seed, 3 * i)
    W = with_outlier_blocks(W, seed, 3 * i + 1)
    x = normal((K,), 1.0, seed, 3 * i + 2)
    return name, W, x


QWEN3_VOCAB = 151936


def qwen3_lm_head(seed: int = 0):
    """(W, x) of the Qwen3-0.6B-like output head: vocabulary x hidden."""
    W = normal((QWEN3_VOCAB, 1024), WEIGHT_STD, seed, 600)
    W = with_outlier_blocks(W, seed, 601)
    x = normal((1024,), 1.0, seed, 602)
    return W, x


LLAMA7B_SHAPES = ((4096, 11008), (11008, 4096))


def llama7b_layer(orientation: int = 0, seed: int = 0):
    rows, K = LLAMA7B_SHAPES[orientation]
    W = normal((rows, K), WEIGHT_STD, seed, 2 * orientation)
    x = normal((K,), 1.0, seed, 2 * orientation + 1)
    return W, x


Q4K_SHAPES = ((4096, 4096), (4096, 11008))


def q4k_rows(shape: int = 0, seed: int = 0):
    rows, K = Q4K_SHAPES[shape]
    W = normal((rows, K), WEIGHT_STD, seed, 3 * shape)
    W = with_row_spread(W, seed, 3 * shape + 1)
    x = normal((K,), 1.0, seed, 3 * shape + 2)
    return W, x


PREFILL_SHAPE = (4096, 11008, 512)  # M, K, N


def prefill(seed: int = 0, M: int = 4096, K: int = 11008, N: int = 512):
    W = normal((M, K), WEIGHT_STD, seed, 0)
    X = normal((N, K), 1.0, seed, 1)
    return W, X
