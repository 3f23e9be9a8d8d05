"""The seeded workload generator: deterministic, right shapes and statistics."""
import numpy as np

from block_quantized_weight_qmat_amd import inputs


def test_deterministic_and_independent():
    a = inputs.normal((64, 64), 0.02, 0, 0)
    b = inputs.normal((64, 64), 0.02, 0, 0)
    c = inputs.normal((64, 64), 0.02, 0, 1)
    assert a.dtype == np.float32 and np.array_equal(a, b) and not np.array_equal(a, c)


def test_outlier_blocks():
    W = inputs.normal((64, 1024), 0.02, 0, 0)
    Wo = inputs.with_outlier_blocks(W, 0, 1)
    changed = np.argwhere(W != Wo)
    nblk = 64 * 1024 // 32
    assert len(changed) == round(0.01 * nblk)
    blocks = {(r, c // 32) for r, c in changed}
    assert len(blocks) == len(changed)           # one per block, distinct blocks
    assert np.allclose(np.abs(Wo[W != Wo]), 0.2)


def test_row_spread_range():
    W = np.ones((2000, 32), np.float32)
    r = inputs.with_row_spread(W, 0, 0)[:, 0]
    assert r.min() >= 0.5 and r.max() <= 2.0
    assert abs(np.log(r).mean()) < 0.05


def test_workload_shapes():
    assert len(inputs.qwen3_shapes()) == 196
    assert sum(r * k for _, r, k in inputs.qwen3_shapes()) == 440_401_920
    W, x = inputs.gemv_1024()
    assert W.shape == (1024, 1024) and x.shape == (1024,)
    assert abs(W.std() - 0.02) < 5e-4 and abs(x.std() - 1) < 0.1
