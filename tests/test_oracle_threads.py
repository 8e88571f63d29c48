"""The oracle's OpenMP loops give the same bits on one thread as on many.

Each output element is computed by one thread in the fixed order of its
definition, so the thread count may change the speed only; this runs every
parallel loop (row copy, fp8 / fp4 pack, plain / quantized / dedup combine, the
dedup dispatch) both ways and compares bitwise."""
import numpy as np
import pytest

import oracle
import workloads as W


@pytest.fixture
def threads():
    n0 = oracle.get_threads()
    yield max(4, n0)
    oracle.set_threads(n0)


def _both(fn, n):
    oracle.set_threads(1)
    assert oracle.get_threads() == 1
    a = fn()
    oracle.set_threads(n)
    assert oracle.get_threads() == n
    b = fn()
    return a, b


def _same(a, b):
    if isinstance(a, dict):
        assert a.keys() == b.keys()
        for k in a:
            _same(a[k], b[k])
    elif isinstance(a, (tuple, list)):
        for u, v in zip(a, b):
            _same(u, v)
    elif a is None:
        assert b is None
    else:
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


@pytest.mark.parametrize("packed_dt", [None, "fp8", "fp4"])
def test_dispatch_and_combine_thread_count(threads, packed_dt):
    rng = np.random.default_rng(41)
    T, H, K, E = 1500, 256, 6, 40
    idx = rng.integers(-1, E, size=(T, K)).astype(np.int32)
    x = W.normal_x(rng, T, H, "bf16")
    x[::97] = oracle.bf16_encode(rng.standard_normal((len(x[::97]), H)).astype(np.float32) * 900)
    w = rng.random((T, K)).astype(np.float32)
    d1, d2 = _both(lambda: oracle.dispatch(x, "bf16", idx, E, packed_dt=packed_dt), threads)
    _same(d1, d2)
    tm = d1["tok_map"]
    if packed_dt is None:
        c1, c2 = _both(lambda: oracle.combine(d1["packed"], "bf16", tm, w, "bf16"), threads)
    elif packed_dt == "fp8":
        c1, c2 = _both(lambda: oracle.combine_fp8(d1["packed"], d1["scales"], tm, w, "f32"), threads)
    else:
        c1, c2 = _both(lambda: oracle.combine_fp4(d1["packed"], d1["scales"], tm, w, "bf16"), threads)
    _same(c1, c2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_dedup_thread_count(threads, dtype):
    rng = np.random.default_rng(42)
    T, H, K, E, R = 1200, 128, 6, 32, 8
    idx = rng.integers(-1, E, size=(T, K)).astype(np.int32)
    x = W.normal_x(rng, T, H, dtype)
    w = rng.random((T, K)).astype(np.float32)
    d1, d2 = _both(lambda: oracle.dedup_dispatch(x, dtype, idx, E, R), threads)
    _same(d1, d2)
    rr = int(d1["recv_cnt"].sum())
    c1, c2 = _both(lambda: oracle.dedup_combine(d1["packed"], dtype, d1["tok_map"], w, idx, E, R,
                                                d1["rank_slot"], rr, "f32", want_partial=True),
                   threads)
    _same(c1, c2)
