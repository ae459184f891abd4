"""Host logic of the sparse/dense switch: the expected union of a batch and the
time comparison (no GPU)."""
import numpy as np
import pytest

from activation_sparse_ffn_amd.switch import SparseDenseSwitch, expected_union


def test_expected_union_closed_forms():
    p = np.full(100, 0.1)
    assert expected_union(p, 1) == pytest.approx(10.0)
    assert expected_union(p, 2) == pytest.approx(100 * (1 - 0.81))
    assert expected_union(np.array([0.0, 1.0, 0.5]), 3) == pytest.approx(1.0 + 0.875)


def test_expected_union_matches_sampling():
    rng = np.random.default_rng(4)
    p = rng.random(300) ** 3
    B, n = 6, 4000
    masks = rng.random((n, B, 300)) < p
    emp = masks.any(axis=1).sum(axis=1).mean()
    assert expected_union(p, B) == pytest.approx(emp, rel=0.01)


def test_expected_union_grows_with_batch():
    p = np.linspace(0.0, 0.9, 50)
    u = [expected_union(p, B) for B in range(1, 40)]
    assert all(b >= a for a, b in zip(u, u[1:])) and u[-1] <= 50


def test_switch_time_model_and_crossover():
    sw = SparseDenseSwitch(pred_bytes=168e6, row_bytes=32772.0, f=32768, sparse_gbps=3000.0, dense_gbps=4500.0)
    kx = sw.crossover_k()
    assert sw.use_dense(kx + 1.0) and not sw.use_dense(kx - 1.0)
    assert sw.dense_us() == pytest.approx(32768 * 32772.0 / 4.5e6)
    # a fast-enough sparse path never switches
    never = SparseDenseSwitch(pred_bytes=1e3, row_bytes=100.0, f=1000, sparse_gbps=1e4, dense_gbps=1e3)
    assert never.crossover_k() > 1000 and never.choose(np.ones(1000), 64) == "sparse"
    p = np.full(32768, 0.5)
    assert sw.choose(p, 64) == "dense" and sw.choose(np.full(32768, 0.01), 1) == "sparse"
