"""Pins for the oracle's combine (weighted f32 gather-reduce) and out_weights.

The identity-expert closed form out = (sum_k w_k) * x (stated on the pages),
exact dyadic cases, two hand-derived cases that fail if the k order or the
unfused multiply-then-add rule is broken, and a numpy float32 loop."""
import os

import numpy as np
import pytest

import oracle
import workloads as W


def _golden(key):
    path = os.path.join(os.path.dirname(__file__), "golden", "page_facts.txt")
    for line in open(path):
        if line.startswith(key + " "):
            return line.split()[1]
    raise KeyError(key)


def _bf16(v):
    return W.bf16_bits_from_f32(np.asarray(v, np.float32))


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill"])
def test_identity_experts_closed_form(name):
    assert _golden("identity_telescoping") == "1"
    d = W.make_inputs(name, T=min(256, W.WORKLOADS[name].T))
    E = d["E"]
    r = oracle.dispatch(d["x"], "bf16", d["idx"], E)
    out, ow = oracle.combine(r["packed"], "bf16", r["tok_map"], d["w"], "bf16")
    xf = W.f32_from_bf16_bits(d["x"]).astype(np.float64)
    sw = d["w"].astype(np.float64).sum(axis=1)
    ref = sw[:, None] * xf
    of = W.f32_from_bf16_bits(out).astype(np.float64)
    # within one bf16 ulp (relative 2^-7) of the exact value
    assert np.all(np.abs(of - ref) <= 2.0**-7 * np.abs(ref) + 1e-30)
    # out_weights is the f32 sum of the weights, close to 1 for softmax weights
    assert np.all(np.abs(ow.astype(np.float64) - sw) <= d["K"] * 2.0**-23)
    assert np.all(np.abs(ow - 1.0) <= d["K"] * 2.0**-23)


def test_dyadic_exact():
    """Integer x and power-of-two weights: every product and sum is exact."""
    rng = np.random.default_rng(0)
    T, K, E, H = 50, 4, 6, 64
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    x = rng.integers(-64, 65, size=(T, H)).astype(np.float32)
    w = (2.0 ** -rng.integers(1, 6, size=(T, K))).astype(np.float32)
    r = oracle.dispatch(_bf16(x), "bf16", idx, E)
    out, ow = oracle.combine(r["packed"], "bf16", r["tok_map"], w, "f32")
    exact = w.astype(np.float64).sum(axis=1)[:, None] * x
    np.testing.assert_array_equal(out.astype(np.float64), exact)
    np.testing.assert_array_equal(ow.astype(np.float64), w.astype(np.float64).sum(axis=1))
    out_b, _ = oracle.combine(r["packed"], "bf16", r["tok_map"], w, "bf16")
    np.testing.assert_array_equal(out_b, _bf16(exact))


def test_order_is_ascending_k():
    """rows 2^24, 1, -2^24 with unit weights: ascending k gives 0, any order
    that adds the 1 after cancelling gives 1."""
    y = np.float32([[2.0**24], [1.0], [-(2.0**24)]])
    tm = np.array([[0, 1, 2]], np.int64)
    w = np.ones((1, 3), np.float32)
    out, _ = oracle.combine(y, "f32", tm, w, "f32")
    assert out[0, 0] == 0.0
    out, _ = oracle.combine(y, "f32", tm[:, ::-1].copy(), w, "f32")
    assert out[0, 0] == 1.0


def test_multiply_then_add_is_unfused():
    """w0*y0 = -(1+2^-7+2^-23+2^-30) rounds to -(1+2^-7+2^-23); adding the
    rounded +w1*y1 gives exactly 0, a fused multiply-add would give 2^-30."""
    a = np.float32(1.0 + 2.0**-23)
    yv = np.float32(1.0 + 2.0**-7)
    y = _bf16([[yv], [yv]])
    assert W.f32_from_bf16_bits(y)[0, 0] == yv
    w = np.float32([[-a, a]])
    tm = np.array([[0, 1]], np.int64)
    out, ow = oracle.combine(y, "bf16", tm, w, "f32")
    assert out[0, 0] == 0.0 and ow[0] == 0.0
    assert np.float64(-a) * np.float64(yv) + np.float64(a) * np.float64(yv) == 0.0
    fused = np.float32(np.float64(np.float32(-a * yv)) + np.float64(a) * np.float64(yv))
    assert fused == np.float32(2.0**-30)


def test_skips_sentinel_and_out_of_range_rows():
    y = np.float32([[1.0], [2.0], [4.0]])
    tm = np.array([[-1, 2, 7], [-1, -1, -1], [0, 3, 1]], np.int64)
    w = np.float32([[9.0, 0.5, 9.0], [1.0, 1.0, 1.0], [0.25, 9.0, 2.0]])
    out, ow = oracle.combine(y, "f32", tm, w, "f32")
    assert out[:, 0].tolist() == [2.0, 0.0, 0.25 + 4.0]
    assert ow.tolist() == [0.5, 0.0, 2.25]


@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
def test_matches_numpy_float32_loop(out_dt):
    rng = np.random.default_rng(11)
    T, K, H, rows = 40, 8, 96, 300
    y = W.normal_x(rng, rows, H, "bf16")
    tm = rng.integers(-1, rows, size=(T, K)).astype(np.int64)
    w = rng.random((T, K)).astype(np.float32)
    out, ow = oracle.combine(y, "bf16", tm, w, out_dt)
    yf = W.f32_from_bf16_bits(y)
    acc = np.zeros((T, H), np.float32)
    ws = np.zeros(T, np.float32)
    for k in range(K):
        ok = tm[:, k] >= 0
        p = (w[:, k:k + 1] * yf[np.maximum(tm[:, k], 0)]).astype(np.float32)
        acc = np.where(ok[:, None], (acc + p).astype(np.float32), acc)
        ws = np.where(ok, (ws + w[:, k]).astype(np.float32), ws)
    exp = acc if out_dt == "f32" else W.bf16_bits_from_f32(acc)
    np.testing.assert_array_equal(out, exp)
    np.testing.assert_array_equal(ow, ws)


def test_decode_expert_scale_bound():
    """Decode workload: out = sum_k w_k c_{e_k} x within two bf16 ulps."""
    d = W.make_inputs("decode")
    r = oracle.dispatch(d["x"], "bf16", d["idx"], d["E"])
    y = oracle.expert_scale(r["packed"], r["packed_cnt"], r["packed_off"], d["c"])
    out, _ = oracle.combine(y, "bf16", r["tok_map"], d["w"], "bf16")
    xf = W.f32_from_bf16_bits(d["x"]).astype(np.float64)
    coef = (d["w"].astype(np.float64) * d["c"][d["idx"]].astype(np.float64)).sum(axis=1)
    ref = coef[:, None] * xf
    # bound per term: the expert's bf16 rounding (2^-8 relative) then the sum
    bound = 2.0**-7 * np.abs(ref) + (d["w"].astype(np.float64) * d["c"][d["idx"]]).sum(axis=1)[:, None] * np.abs(xf) * 2.0**-8
    of = W.f32_from_bf16_bits(out).astype(np.float64)
    assert np.all(np.abs(of - ref) <= bound + 1e-30)
