"""The seeded input generator: determinism and the configured distributions."""
import numpy as np

from integer_only_quantized_int8_amd import workloads as W


def test_deterministic_and_seed_dependent():
    a = W.make_workload(2, 3, 17, 64, seed=5)
    b = W.make_workload(2, 3, 17, 64, seed=5)
    c = W.make_workload(2, 3, 17, 64, seed=6)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    assert a.params == b.params
    assert not np.array_equal(a.q, c.q)
    assert not np.array_equal(a.q, a.k)  # independent streams


def test_gaussian_int8_distribution():
    w = W.make_workload(4, 4, 197, 64, seed=1)
    x = w.q.astype(np.float64)
    assert abs(x.std() - 24.0) < 0.3
    assert abs(x.mean()) < 0.2
    assert w.q.min() >= -127 and w.q.max() <= 127


def test_dyadic_draws_in_range():
    for s in range(50):
        p = W.default_params(s)
        assert (1 << 14) <= p["qk_b"] < (1 << 15) and (1 << 14) <= p["pv_b"] < (1 << 15)
        assert p["qk_c"] == 22 and p["pv_c"] == 20
    assert W.default_params(3, W.LIS)["pv_c"] == 28


def test_headline_shape_sigma_and_outliers():
    spec = dict(W.CONFIGS[2])
    spec.update(batch=4)
    w = W.make_workload(seed=1002, **spec)
    v = w.v.astype(np.float64)
    stds = v.std(axis=(0, 2, 3))
    assert stds.min() > 7 and stds.max() < 41
    q = w.q.astype(np.float64)
    assert np.allclose(stds, q.std(axis=(0, 2, 3)), rtol=0.08)
    # about 5 % of K rows are tripled: their std is about 3x the head's
    kstd = w.k.astype(np.float64).std(axis=3)
    ratio = kstd / stds[None, :, None]
    frac = (ratio > 2.0).mean()
    assert 0.03 < frac < 0.07


def test_window_bias_table():
    w = W.make_workload(2, 3, 49, 32, seed=4, window=7)
    t = w.params["rel_bias"]
    assert t.shape == (3, 169) and t.dtype == np.int32
    assert t.min() >= -512 and t.max() <= 512
