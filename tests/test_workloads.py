"""The seeded input recipe: shapes, distinct top-K, weight normalisation and
the skew statistics of the Zipf(1.2) routing."""
import numpy as np
import pytest

import workloads as W


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_shapes_and_distinct_topk(name):
    wl = W.WORKLOADS[name]
    T = min(wl.T, 1024)
    d = W.make_inputs(name, T=T)
    assert d["idx"].shape == (T, wl.K) and d["idx"].dtype == np.int32
    assert d["w"].shape == (T, wl.K) and d["w"].dtype == np.float32
    assert d["x"].shape == (T, wl.H)
    assert d["x"].dtype == (np.float32 if wl.x_dtype == "f32" else np.uint16)
    s = np.sort(d["idx"], axis=1)
    assert np.all(np.diff(s, axis=1) > 0) and s.min() >= 0 and s.max() < wl.E
    assert np.all(np.abs(d["w"].astype(np.float64).sum(axis=1) - 1) < 1e-6)
    # same seed, same draw
    d2 = W.make_inputs(name, T=T)
    assert np.array_equal(d["idx"], d2["idx"]) and np.array_equal(d["x"], d2["x"])


def test_zipf_skew():
    d = W.make_inputs("skewed_fp8", T=2048)
    cnt = np.bincount(d["idx"].ravel(), minlength=256)
    top = np.sort(cnt)[::-1]
    # the top expert is picked by ~93% of tokens; the expert ids are permuted
    assert 0.85 * 2048 < top[0] <= 2048
    assert top[4] > 0.25 * 2048


def test_dedup_unique_ranks():
    d = W.make_inputs("dedup", T=4096)
    U = np.array([len(set((row // 8).tolist())) for row in d["idx"]])
    # E[U] = 8 * (1 - C(56,6)/C(64,6)) = 4.5355
    assert abs(U.mean() - 4.5355) < 0.05
