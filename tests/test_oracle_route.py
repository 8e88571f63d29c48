"""Pins for the oracle's route count, slot assignment and row copy.

Checked against library routines (numpy bincount / cumsum / stable argsort and
fancy indexing), a sort-based brute force over every tiny routing, and the
structural invariants of a stable counting sort."""
import itertools

import numpy as np
import pytest

import oracle
import workloads as W


def _golden(key):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "page_facts.txt")
    for line in open(path):
        if line.startswith(key + " "):
            return line.split()[1]
    raise KeyError(key)


def _expected_rows_by_argsort(idx, E, cap, packed_rows):
    """Library pin: rows from numpy's stable argsort of the valid ids."""
    flat = idx.ravel().astype(np.int64)
    valid = (flat >= 0) & (flat < E)
    f_valid = np.nonzero(valid)[0]
    order = f_valid[np.argsort(flat[f_valid], kind="stable")]   # sorted by (e, f)
    e_sorted = flat[order]
    cnt = np.bincount(flat[valid], minlength=E)
    off = np.concatenate([[0], np.cumsum(cnt)])
    slot = np.arange(len(order)) - off[e_sorted]                 # position inside its expert
    base = e_sorted * cap if cap > 0 else off[e_sorted]
    row = base + slot
    ok = (row < packed_rows) & ((slot < cap) if cap > 0 else True)
    tok = np.full(flat.shape, -1, np.int64)
    tok[order[ok]] = row[ok]
    return tok.reshape(idx.shape), cnt, off


def _mixed_idx(rng, T, K, E, p_neg=0.05, p_bad=0.02):
    idx = rng.integers(0, E, size=(T, K)).astype(np.int32)
    u = rng.random((T, K))
    idx[u < p_neg] = -1
    bad = u > 1 - p_bad
    idx[bad] = rng.choice(np.array([E, E + 5, -2, -1000, 2**31 - 1], np.int64),
                          size=int(bad.sum())).astype(np.int32)
    return idx


def test_golden_scan_convention():
    cnt, off, _ = oracle.route_count(np.array([[0, 1]], np.int32), 3)
    assert off[0] == int(_golden("exclusive_scan_initial"))


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_route_count_matches_bincount(name):
    d = W.make_inputs(name, T=min(W.WORKLOADS[name].T, 2048))
    rng = np.random.default_rng(7)
    idx = d["idx"].copy()
    idx[rng.random(idx.shape) < 0.03] = -1
    idx[rng.random(idx.shape) < 0.01] = d["E"] + 3
    cnt, off, stats = oracle.route_count(idx, d["E"])
    flat = idx.ravel()
    valid = (flat >= 0) & (flat < d["E"])
    np.testing.assert_array_equal(cnt, np.bincount(flat[valid], minlength=d["E"]))
    np.testing.assert_array_equal(off, np.concatenate([[0], np.cumsum(cnt)]))
    assert stats[0] == np.sum(~valid & (flat != -1))


@pytest.mark.parametrize("layout", ["compact", "padded", "compact_short", "padded_tight"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_dispatch_slots_match_stable_argsort(layout, seed):
    rng = np.random.default_rng(seed)
    T, K, E, H = 300, 4, 13, 16
    idx = _mixed_idx(rng, T, K, E)
    cnt_true = np.bincount(idx.ravel()[(idx.ravel() >= 0) & (idx.ravel() < E)], minlength=E)
    cap = {"compact": 0, "padded": int(cnt_true.max()), "compact_short": 0,
           "padded_tight": max(1, int(cnt_true.max()) - 7)}[layout]
    rows = {"compact": T * K, "padded": E * cap, "compact_short": int(cnt_true.sum()) - 50,
            "padded_tight": E * cap - cap // 2}[layout]
    x = rng.standard_normal((T, H)).astype(np.float32)
    r = oracle.dispatch(x, "f32", idx, E, cap=cap, packed_rows=rows)
    tok, cnt, off = _expected_rows_by_argsort(idx, E, cap, rows)
    np.testing.assert_array_equal(r["tok_map"], tok)
    flat = idx.ravel()
    valid = (flat >= 0) & (flat < E)
    written = tok.ravel() >= 0
    # counts of rows written per expert and the segment starts
    np.testing.assert_array_equal(r["packed_cnt"], np.bincount(flat[written], minlength=E))
    base = np.arange(E + 1) * cap if cap > 0 else off
    np.testing.assert_array_equal(r["packed_off"], np.minimum(base, rows))
    assert r["stats"][0] == np.sum(~valid & (flat != -1))
    assert r["stats"][1] == np.sum(valid & ~written)
    # packed_src names the source token of every written row; other rows stay poisoned
    t_of_f = np.repeat(np.arange(T), K)
    expect_src = np.full(rows, oracle.POISON_I32, np.int32)
    expect_src[tok.ravel()[written]] = t_of_f[written]
    np.testing.assert_array_equal(r["packed_src"], expect_src)
    # rows: bitwise copies of x[packed_src], untouched rows keep the poison pattern
    pk = r["packed"].view(np.uint8)
    wr = expect_src >= 0
    np.testing.assert_array_equal(r["packed"][wr].view(np.uint32), x[expect_src[wr]].view(np.uint32))
    assert np.all(pk[~wr] == oracle.POISON_BYTE)


def _brute_rows(flat, E, cap, packed_rows, K):
    """Sort-based brute force on a tiny routing: rank of each entry inside its expert."""
    N = len(flat)
    valid = [f for f in range(N) if 0 <= flat[f] < E]
    groups = {}
    for f in sorted(valid, key=lambda f: (flat[f], f)):
        groups.setdefault(flat[f], []).append(f)
    start, acc = {}, 0
    for e in range(E):
        start[e] = acc
        acc += len(groups.get(e, []))
    tok = [-1] * N
    for e, fs in groups.items():
        for s, f in enumerate(fs):
            base = e * cap if cap > 0 else start[e]
            if (cap > 0 and s >= cap) or base + s >= packed_rows:
                continue
            tok[f] = base + s
    return tok


def test_dispatch_brute_force_tiny():
    """Every routing with T*K = 6 entries over ids {-1, 0, 1, 2} (E = 3)."""
    E = 3
    x = np.arange(3 * 8, dtype=np.float32).reshape(3, 8)
    n = 0
    for T, K in [(3, 2), (2, 3), (6, 1), (1, 6)]:
        xx = np.resize(x, (T, 8))
        for ids in itertools.product(range(-1, E), repeat=T * K):
            idx = np.array(ids, np.int32).reshape(T, K)
            for cap, rows in [(0, T * K), (0, 3), (1, E), (2, 2 * E), (2, 5)]:
                r = oracle.dispatch(xx, "f32", idx, E, cap=cap, packed_rows=rows)
                exp = _brute_rows(list(ids), E, cap, rows, K)
                assert r["tok_map"].ravel().tolist() == exp, (ids, cap, rows)
                # invariants of the written rows
                tm = r["tok_map"].ravel()
                w = tm[tm >= 0]
                assert len(set(w.tolist())) == len(w)
                for f in np.nonzero(tm >= 0)[0]:
                    assert r["packed_src"][tm[f]] == f // K
                n += 1
    assert n == 4 * 4096 * 5


def test_dispatch_bf16_rows_bitwise_and_expert_lists_increasing():
    d = W.make_inputs("prefill", T=512)
    E = d["E"]
    r = oracle.dispatch(d["x"], "bf16", d["idx"], E, cap=0)
    tm = r["tok_map"]
    assert np.all(tm >= 0)
    np.testing.assert_array_equal(r["packed"], d["x"][r["packed_src"]])
    # each expert's segment lists its entries in increasing flat order
    flat = d["idx"].ravel()
    for e in range(0, E, 17):
        fs = np.nonzero(flat == e)[0]
        rows = tm.ravel()[fs]
        assert np.all(np.diff(rows) == 1)
        assert rows[0] == r["packed_off"][e]


def test_route_count_edge_cases():
    cnt, off, st = oracle.route_count(np.zeros((0, 4), np.int32), 5)
    assert cnt.tolist() == [0] * 5 and off.tolist() == [0] * 6 and st[0] == 0
    cnt, off, st = oracle.route_count(np.full((7, 3), -1, np.int32), 5)
    assert cnt.sum() == 0 and st[0] == 0
    cnt, off, st = oracle.route_count(np.full((7, 3), 2, np.int32), 5)
    assert cnt.tolist() == [0, 0, 21, 0, 0] and off.tolist() == [0, 0, 0, 21, 21, 21]
