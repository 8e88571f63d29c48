"""Pins for the oracle's virtual-rank dedup dispatch and its combine.

Rank masks against python sets, recv rows against numpy's stable sort of the
(rank, token) pairs, the packed outputs against the plain dispatch of the same
ids, the -1 sentinel trap, and the combine against the closed form and against
the plain combine where the two must agree bit for bit."""
import itertools
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


def _case(T=400, seed=0, neg=0.05):
    d = W.make_inputs("dedup", T=T, seed=seed)
    idx = d["idx"].copy()
    rng = np.random.default_rng(seed + 100)
    idx[rng.random(idx.shape) < neg] = -1
    return d, idx


def test_rank_masks_and_recv_rows():
    d, idx = _case()
    T, K, E, R = d["T"], d["K"], d["E"], d["R"]
    er = E // R
    r = oracle.dedup_dispatch(d["x"], "f32", idx, E, R)
    sets = [sorted({int(e) // er for e in row if 0 <= e < E}) for row in idx]
    U = np.array([len(s) for s in sets])
    assert r["recv_off"][R] == U.sum()
    np.testing.assert_array_equal(r["recv_cnt"], [sum(rk in s for s in sets) for rk in range(R)])
    # rows: pairs (r, t) sorted by rank, then token (numpy stable sort of the pair list)
    pairs = np.array([(rk, t) for t, s in enumerate(sets) for rk in s], np.int64)
    order = pairs[np.argsort(pairs[:, 0], kind="stable")]
    np.testing.assert_array_equal(r["recv_src"][:len(order)], order[:, 1])
    rs = np.full((T, R), -1, np.int32)
    rs[order[:, 1], order[:, 0]] = np.arange(len(order))
    np.testing.assert_array_equal(r["rank_slot"], rs)
    np.testing.assert_array_equal(r["recv_x"][:len(order)], d["x"][order[:, 1]])
    assert np.all(r["recv_x"][len(order):].view(np.uint8) == oracle.POISON_BYTE)


def test_sentinel_does_not_fake_rank_zero():
    assert _golden("sentinel") == "-1"
    er = int(_golden("sentinel_trap_experts_per_rank"))
    E, R = er * 2, 2
    idx = np.array([[-1, er + 1], [er, -1], [-1, -1]], np.int32)
    x = np.arange(3 * 4, dtype=np.float32).reshape(3, 4)
    r = oracle.dedup_dispatch(x, "f32", idx, E, R)
    assert r["rank_slot"].tolist() == [[-1, 0], [-1, 1], [-1, -1]]
    assert r["recv_cnt"].tolist() == [0, 2]


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("layout", ["compact", "padded"])
def test_packed_outputs_equal_plain_dispatch(seed, layout):
    d, idx = _case(seed=seed)
    E, R = d["E"], d["R"]
    cnt, _, _ = oracle.route_count(idx, E)
    cap = int(cnt.max()) - 2 if layout == "padded" else 0
    a = oracle.dedup_dispatch(d["x"], "f32", idx, E, R, cap=cap)
    b = oracle.dispatch(d["x"], "f32", idx, E, cap=cap)
    for key in ["packed", "packed_cnt", "packed_off", "packed_src", "tok_map"]:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    assert a["stats"].tolist() == b["stats"].tolist()


def test_recv_drops_equal_plain_dispatch_of_surviving_ids():
    d, idx = _case(T=300, seed=2)
    E, R, T = d["E"], d["R"], d["T"]
    er = E // R
    full = oracle.dedup_dispatch(d["x"], "f32", idx, E, R)
    n_recv = int(full["recv_off"][R])
    recv_rows = n_recv - 123
    a = oracle.dedup_dispatch(d["x"], "f32", idx, E, R, recv_rows=recv_rows)
    # rows past recv_rows belong to the latest tokens of the highest ranks
    survive = full["rank_slot"] < recv_rows
    assert np.array_equal(a["rank_slot"] >= 0, survive & (full["rank_slot"] >= 0))
    idx2 = idx.copy()
    for t in range(T):
        for k in range(d["K"]):
            e = idx[t, k]
            if 0 <= e < E and not survive[t, e // er]:
                idx2[t, k] = -1
    b = oracle.dispatch(d["x"], "f32", idx2, E)
    for key in ["packed", "packed_cnt", "packed_off", "packed_src", "tok_map"]:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    assert a["stats"][2] == 123
    assert a["stats"][1] == np.sum((idx2 == -1) & (idx != -1))


def test_dedup_brute_force_tiny():
    """Every routing of 2 tokens x 2 picks over ids {-1..3} with E=4, R=2."""
    E, R, K, T = 4, 2, 2, 2
    x = np.arange(T * 4, dtype=np.float32).reshape(T, 4)
    for ids in itertools.product(range(-1, E), repeat=T * K):
        idx = np.array(ids, np.int32).reshape(T, K)
        a = oracle.dedup_dispatch(x, "f32", idx, E, R)
        b = oracle.dispatch(x, "f32", idx, E)
        assert a["tok_map"].tolist() == b["tok_map"].tolist()
        sets = [{e // 2 for e in row if e >= 0} for row in idx]
        assert a["recv_off"][R] == sum(len(s) for s in sets)


def test_dedup_combine_closed_form_and_grouping():
    d, idx = _case(T=256, seed=3)
    E, R, K = d["E"], d["R"], d["K"]
    a = oracle.dedup_dispatch(d["x"], "f32", idx, E, R)
    rr = a["recv_x"].shape[0]
    out, ow, part = oracle.dedup_combine(a["packed"], "f32", a["tok_map"], d["w"], idx, E, R,
                                         a["rank_slot"], rr, "f32", want_partial=True)
    valid = (idx >= 0) & (idx < E)
    sw = np.where(valid, d["w"], 0).astype(np.float64).sum(axis=1)
    ref = sw[:, None] * d["x"].astype(np.float64)
    assert np.all(np.abs(out - ref) <= K * 2.0**-23 * np.abs(d["x"]) * (1 + sw[:, None]) + 1e-30)
    # partial rows: numpy float32 per-rank sums in ascending k; out = 0 + partials by rank
    er = E // R
    acc = np.zeros_like(d["x"])
    for t in range(d["T"]):
        for r in range(R):
            rs = a["rank_slot"][t, r]
            if rs < 0:
                continue
            p = np.zeros(d["x"].shape[1], np.float32)
            for k in range(K):
                e = idx[t, k]
                if 0 <= e < E and e // er == r:
                    p = (p + (d["w"][t, k] * a["packed"][a["tok_map"][t, k]]).astype(np.float32)).astype(np.float32)
            np.testing.assert_array_equal(part[rs], p)
            acc[t] = (acc[t] + p).astype(np.float32)
    np.testing.assert_array_equal(out, acc)
    n_recv = a["recv_off"][R]
    assert np.all(part[n_recv:].view(np.uint8) == oracle.POISON_BYTE)


def test_dedup_combine_equals_plain_when_one_entry_per_rank():
    """Ascending expert ids with at most one entry per rank: both orders add the
    same rounded products in the same sequence, so the results agree bitwise."""
    rng = np.random.default_rng(9)
    T, K, E, R, H = 64, 4, 32, 8, 48
    er = E // R
    idx = np.zeros((T, K), np.int32)
    for t in range(T):
        ranks = np.sort(rng.permutation(R)[:K])
        idx[t] = ranks * er + rng.integers(0, er, K)
    x = W.normal_x(rng, T, H, "bf16")
    w = W.softmax_weights(rng, T, K)
    a = oracle.dedup_dispatch(x, "bf16", idx, E, R)
    o1, w1, _ = oracle.dedup_combine(a["packed"], "bf16", a["tok_map"], w, idx, E, R,
                                     a["rank_slot"], a["recv_x"].shape[0], "bf16")
    o2, w2 = oracle.combine(a["packed"], "bf16", a["tok_map"], w, "bf16")
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(w1, w2)
