"""The seeded input generator: determinism, shapes and the outlier recipe (CPU only)."""
import numpy as np

import workloads as W


def test_decode_generator_is_deterministic_and_shaped():
    a = W.decode_config(2, batch=3, T=40)
    b = W.decode_config(2, batch=3, T=40)
    for x, y in [(a.prefix_k, b.prefix_k), (a.q, b.q), (a.k, b.k), (a.v, b.v)]:
        np.testing.assert_array_equal(x, y)
    assert a.prefix_k.shape == (3 * 272, 16, 128) and a.prefix_k.dtype == np.uint16
    assert a.q.shape == (40, 3, 16, 128)
    assert a.active(40).tolist() == [1, 1, 1] and a.active(41).tolist() == [0, 0, 0]


def test_outliers_are_one_percent_times_eight():
    base = W.make_decode("x", 2, "f32", [64], [8], [300], seed=0, outlier_p=0.0)
    out = W.make_decode("x", 2, "f32", [64], [8], [300], seed=0, outlier_p=0.01)
    for x, y in [(base.prefix_k, out.prefix_k), (base.k, out.k), (base.q, out.q)]:
        diff = x != y
        frac = diff.mean()
        assert 0.008 < frac < 0.012
        np.testing.assert_array_equal(y[diff], x[diff] * np.float32(8))


def test_varlen_metadata_ranges():
    w = W.varlen_config(0, T_max=300)
    pages = np.array(w.meta["pages"])
    assert w.batch == 32
    assert pages.min() >= 1 and pages.max() <= 50
    np.testing.assert_array_equal(w.prefix_len, pages * 256 + 16)
    assert set(np.unique(w.window).tolist()) <= {64, 128, 256, 512}
    assert 256 <= w.steps.min() and w.steps.max() <= 300


def test_prefill_generator_layout():
    p = W.prefill_config(S=300, prefix_len=100, window=16)
    assert p.q.shape == (300, 16, 128) and p.cu_seqlens.tolist() == [0, 300]
    assert p.prefix_len.tolist() == [100] and p.window.tolist() == [16]
