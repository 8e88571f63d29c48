"""Pins of the oracle's replay dispatch and pre-quantized dispatch against numpy
fancy indexing, the separately pinned fp8 row pack, and the routing of the
plain dispatch (which does not depend on the payload)."""
import numpy as np
import pytest

import oracle
import workloads as W


def _routing(rng, T, K, E):
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    idx[rng.random((T, K)) < 0.1] = -1
    return idx


def _distinct_map(rng, T, K, rows, extra=10):
    """A tok_map as a dispatch leaves it: distinct rows, some -1, and (for the
    replay's bound check) some rows at or past packed_rows."""
    tm = rng.permutation(rows + extra)[:T * K].astype(np.int64).reshape(T, K)
    tm[rng.random((T, K)) < 0.1] = -1
    return tm


def _expect_rows(x, tok_map, rows):
    """numpy: packed[tok_map[t,k]] = x[t] for 0 <= tok_map < rows; None elsewhere."""
    exp = [None] * rows
    T, K = tok_map.shape
    for t in range(T):
        for k in range(K):
            r = tok_map[t, k]
            if 0 <= r < rows:
                exp[r] = x[t]
    return exp


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_replay_bit_copy(dt):
    rng = np.random.default_rng(11)
    T, H, K, rows = 50, 64, 3, 160
    x = W.normal_x(rng, T, H, dt)
    tm = _distinct_map(rng, T, K, rows)
    r = oracle.dispatch_replay(x, dt, tm, rows)
    exp = _expect_rows(x, tm, rows)
    poison = np.full(H * (2 if dt == "bf16" else 4), oracle.POISON_BYTE, np.uint8)
    for row in range(rows):
        got = r["packed"][row]
        if exp[row] is None:
            assert np.array_equal(got.view(np.uint8), poison), row
        else:
            assert np.array_equal(got.view(np.uint8), exp[row].view(np.uint8)), row


def test_replay_fp8_pack_matches_row_pack_and_dispatch():
    rng = np.random.default_rng(12)
    T, H, K, E = 40, 256, 4, 9
    x = W.inject_outliers(W.normal_x(rng, T, H, "bf16"), np.arange(0, T, 7), 1000.0)
    idx = _routing(rng, T, K, E)
    d = oracle.dispatch(x, "bf16", idx, E, packed_dt="fp8")
    rows = d["packed"].shape[0]
    r = oracle.dispatch_replay(x, "bf16", d["tok_map"], rows, packed_dt="fp8")
    q, s = oracle.fp8_pack_rows(x)
    for t in range(T):
        for k in range(K):
            row = d["tok_map"][t, k]
            if row >= 0:
                assert np.array_equal(r["packed"][row], q[t])
                assert np.array_equal(r["scales"][row].view(np.uint32), s[t].view(np.uint32))
    assert np.array_equal(r["packed"], d["packed"])
    assert np.array_equal(r["scales"].view(np.uint32), d["scales"].view(np.uint32))


def test_prequant_dispatch_forwards_codes_and_scales():
    rng = np.random.default_rng(13)
    T, H, K, E = 60, 384, 5, 11
    q = rng.integers(0, 256, size=(T, H), dtype=np.uint8)
    s = (rng.random((T, H // 128)) + 0.5).astype(np.float32)
    idx = _routing(rng, T, K, E)
    idx[3, 0] = E + 4                       # invalid id: counted, skipped
    for cap, rows in [(0, None), (3, None), (0, 100)]:
        d = oracle.dispatch(q, "fp8", idx, E, cap=cap, packed_rows=rows, x_scales=s)
        ref = oracle.dispatch(W.normal_x(rng, T, 16, "bf16"), "bf16", idx, E, cap=cap,
                              packed_rows=rows)
        for key in ("tok_map", "packed_cnt", "packed_off", "packed_src", "stats"):
            assert np.array_equal(d[key], ref[key]), key
        for row, t in enumerate(d["packed_src"]):
            if t == oracle.POISON_I32:
                assert np.all(d["packed"][row] == oracle.POISON_BYTE)
                continue
            assert np.array_equal(d["packed"][row], q[t])
            assert np.array_equal(d["scales"][row].view(np.uint32), s[t].view(np.uint32))


def test_prequant_replay_numpy():
    rng = np.random.default_rng(14)
    T, H, K, rows = 33, 128, 6, 200
    q = rng.integers(0, 256, size=(T, H), dtype=np.uint8)
    s = rng.random((T, 1)).astype(np.float32)
    tm = _distinct_map(rng, T, K, rows, extra=5)
    r = oracle.dispatch_replay(q, "fp8", tm, rows, x_scales=s)
    exp = _expect_rows(q, tm, rows)
    exps = _expect_rows(s, tm, rows)
    for row in range(rows):
        if exp[row] is None:
            assert np.all(r["packed"][row] == oracle.POISON_BYTE)
        else:
            assert np.array_equal(r["packed"][row], exp[row])
            assert np.array_equal(r["scales"][row], exps[row])
