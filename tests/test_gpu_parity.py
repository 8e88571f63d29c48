"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on the
same seeded inputs.

Bar: counts, offsets, slot maps, packed rows, fp8 bytes and scales, recv rows
bit-exact; combine within one bf16 ulp per element (relative error <= 2^-7;
the arithmetic is the same sequence of correctly rounded f32 operations, so the
results are expected to be bit-identical and the tests also report that).
Outputs are poisoned before each call so a skipped write cannot pass."""
import numpy as np
import pytest
import torch

import combine_moe_route_count_amd as moe
import oracle
import workloads as W
from _gpu_util import (DEV, assert_dispatch_equal, bf16_ulp_diff, dev, dev_bf16, dev_x,
                       gpu_dispatch, host, note, poison_)

pytestmark = pytest.mark.gpu


def _mixed_idx(rng, T, K, E, p_neg=0.05, p_bad=0.02):
    idx = np.stack([rng.permutation(E)[:K] if K <= E else rng.integers(0, E, K)
                    for _ in range(T)]).astype(np.int32)
    u = rng.random((T, K))
    idx[u < p_neg] = -1
    bad = u > 1 - p_bad
    idx[bad] = rng.choice(np.array([E, E + 9, -2, -77], np.int64), size=int(bad.sum())).astype(np.int32)
    return idx


def _check_combine(got, exp, dtype):
    """<= 1 bf16 ulp for bf16 output, relative 2^-7 for f32; returns bit-exact flag."""
    if dtype == "bf16":
        d = bf16_ulp_diff(got, exp)
        assert d.max() <= 1, f"max {d.max()} bf16 ulps at {np.unravel_index(d.argmax(), d.shape)}"
        return bool((d == 0).all())
    g = got.astype(np.float64)
    e = exp.astype(np.float64)
    assert np.all(np.abs(g - e) <= 2.0**-7 * np.abs(e)), "f32 combine off by more than 2^-7"
    return bool(np.array_equal(got.view(np.uint32), exp.view(np.uint32)))


# ---------------------------------------------------------------------------
# route count
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_route_count_workloads(name):
    d = W.make_inputs(name)
    idx = d["idx"].copy()
    rng = np.random.default_rng(1)
    idx[rng.random(idx.shape) < 0.02] = -1
    idx[rng.random(idx.shape) < 0.01] = 5000
    note(f"route_count {name} T={d['T']} K={d['K']} E={d['E']}")
    cnt, off, st = moe.route_count(dev(idx), d["E"])
    torch.cuda.synchronize()
    rc, ro, rs = oracle.route_count(idx, d["E"])
    np.testing.assert_array_equal(host(cnt), rc)
    np.testing.assert_array_equal(host(off), ro)
    np.testing.assert_array_equal(host(st), rs)


@pytest.mark.parametrize("T,K,E", [(0, 4, 16), (1, 1, 1), (1, 16, 1024), (257, 3, 5),
                                   (1000, 8, 1024), (5000, 6, 64), (3, 16, 2)])
def test_route_count_shapes(T, K, E):
    rng = np.random.default_rng(T + K + E)
    idx = rng.integers(-1, E, size=(T, K)).astype(np.int32)
    note(f"route_count shape T={T} K={K} E={E}")
    cnt, off, st = moe.route_count(dev(idx) if T else torch.empty((0, K), dtype=torch.int32, device=DEV), E)
    torch.cuda.synchronize()
    rc, ro, rs = oracle.route_count(idx, E)
    np.testing.assert_array_equal(host(cnt), rc)
    np.testing.assert_array_equal(host(off), ro)
    np.testing.assert_array_equal(host(st), rs)


# ---------------------------------------------------------------------------
# dispatch
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", ["compact", "padded", "padded_tight", "compact_short"])
@pytest.mark.parametrize("T,K,E,H", [(300, 4, 13, 64), (2100, 8, 256, 136), (64, 2, 8, 256)])
def test_dispatch_small(dtype, layout, T, K, E, H):
    rng = np.random.default_rng(T * 7 + K)
    idx = _mixed_idx(rng, T, K, E)
    x = W.normal_x(rng, T, H, dtype)
    flat = idx.ravel()
    cnt = np.bincount(flat[(flat >= 0) & (flat < E)], minlength=E)
    cap = {"compact": 0, "padded": int(cnt.max()), "padded_tight": max(1, int(cnt.max()) // 2),
           "compact_short": 0}[layout]
    rows = {"compact": T * K, "padded": E * cap, "padded_tight": E * cap - 3,
            "compact_short": max(0, int(cnt.sum()) - 37)}[layout]
    note(f"dispatch {dtype} {layout} T={T} K={K} E={E} H={H} cap={cap} rows={rows}")
    o = gpu_dispatch(dev_x(x, dtype), idx, E, cap=cap, packed_rows=rows)
    ref = oracle.dispatch(x, dtype, idx, E, cap=cap, packed_rows=rows)
    assert_dispatch_equal(o, ref)


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill"])
def test_dispatch_workload_full(name):
    d = W.make_inputs(name)
    E = d["E"]
    cap = int(np.bincount(d["idx"].ravel(), minlength=E).max()) if d["layout"] == "padded" else 0
    note(f"dispatch workload {name} cap={cap}")
    o = gpu_dispatch(dev_x(d["x"], d["x_dtype"]), d["idx"], E, cap=cap)
    ref = oracle.dispatch(d["x"], d["x_dtype"], d["idx"], E, cap=cap)
    assert_dispatch_equal(o, ref)


def test_dispatch_fp8_skewed_full():
    d = W.make_inputs("skewed_fp8")
    x = W.inject_outliers(d["x"], np.arange(0, d["T"], 97), 1000.0)
    note("dispatch fp8 skewed full T=8192")
    o = gpu_dispatch(dev_bf16(x), d["idx"], d["E"], fp8=True)
    ref = oracle.dispatch(x, "bf16", d["idx"], d["E"], packed_dt="fp8")
    assert_dispatch_equal(o, ref, fp8=True)


def test_fp8_encoder_exhaustive_via_dispatch():
    """Every bf16 value with |v| <= 448 goes through the unscaled branch once;
    rows with a 1000x outlier put the rest through the scaled branch."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = W.f32_from_bf16_bits(bits)
    keep = bits[np.isfinite(v) & (np.abs(v) <= 448)]
    H = 1024
    n = (len(keep) + H - 1) // H * H
    xs = np.resize(keep, n).reshape(-1, H)
    rng = np.random.default_rng(3)
    sc = rng.permutation(xs.reshape(-1)).reshape(-1, H)
    scf = W.f32_from_bf16_bits(sc)
    scf[:, ::131] = np.float32(3000.0)          # every block scaled, amax at several lanes
    x = np.concatenate([xs, W.bf16_bits_from_f32(scf)])
    T = x.shape[0]
    idx = np.zeros((T, 1), np.int32)
    note(f"fp8 exhaustive T={T} H={H}")
    o = gpu_dispatch(dev_bf16(x), idx, 1, fp8=True)
    ref = oracle.dispatch(x, "bf16", idx, 1, packed_dt="fp8")
    assert_dispatch_equal(o, ref, fp8=True)


@pytest.mark.parametrize("case", ["T0", "T1", "all_neg", "one_expert", "bad_ids", "H8", "K16_E1024",
                                  "E1", "dup_expert", "rows0"])
def test_dispatch_edges(case):
    rng = np.random.default_rng(5)
    T, K, E, H, cap, rows = 40, 4, 16, 64, 0, None
    idx = None
    if case == "T0":
        T = 0
    elif case == "T1":
        T = 1
    elif case == "all_neg":
        idx = np.full((T, K), -1, np.int32)
    elif case == "one_expert":
        idx = np.full((T, K), 3, np.int32)
    elif case == "bad_ids":
        idx = rng.integers(-5, E + 5, size=(T, K)).astype(np.int32)
    elif case == "H8":
        H = 8
    elif case == "K16_E1024":
        K, E, T = 16, 1024, 700
    elif case == "E1":
        E = 1
        idx = rng.integers(-1, 1, size=(T, K)).astype(np.int32)
    elif case == "dup_expert":
        idx = rng.integers(0, 3, size=(T, K)).astype(np.int32)
    elif case == "rows0":
        rows = 0
    if idx is None:
        idx = rng.integers(-1, E, size=(T, K)).astype(np.int32)
    x = W.normal_x(rng, T, H, "bf16")
    note(f"dispatch edge {case}")
    xd = dev_bf16(x) if T else torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    o = gpu_dispatch(xd, idx, E, cap=cap, packed_rows=rows)
    ref = oracle.dispatch(x, "bf16", idx, E, cap=cap, packed_rows=rows)
    assert_dispatch_equal(o, ref)


# ---------------------------------------------------------------------------
# combine
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("y_dt", ["bf16", "f32"])
@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
@pytest.mark.parametrize("K", [1, 2, 3, 8, 16])
def test_combine_random(y_dt, out_dt, K):
    rng = np.random.default_rng(K * 11)
    T, H, rows = 333, 200, 900
    y = W.normal_x(rng, rows, H, y_dt)
    tm = rng.integers(-1, rows + 3, size=(T, K)).astype(np.int64)   # -1 and out-of-range rows
    w = rng.random((T, K)).astype(np.float32)
    note(f"combine y={y_dt} out={out_dt} K={K}")
    out_t = torch.empty((T, H), dtype=torch.bfloat16 if out_dt == "bf16" else torch.float32, device=DEV)
    ow_t = torch.empty(T, dtype=torch.float32, device=DEV)
    poison_(out_t)
    poison_(ow_t)
    moe.combine(dev_x(y, y_dt), dev(tm), dev(w), out_dtype=out_t.dtype, out=out_t, out_weights=ow_t)
    torch.cuda.synchronize()
    eo, ew = oracle.combine(y, y_dt, tm, w, out_dt)
    _check_combine(host(out_t), eo, out_dt)
    np.testing.assert_array_equal(host(ow_t), ew)


def test_combine_order_and_fusion_cases():
    """Hand-derived cases that only pass with ascending k and unfused mul/add."""
    y = np.float32([[2.0**24] * 8, [1.0] * 8, [-(2.0**24)] * 8])
    tm = np.array([[0, 1, 2]], np.int64)
    w = np.ones((1, 3), np.float32)
    out, _ = moe.combine(dev(y), dev(tm), dev(w), out_dtype=torch.float32)
    assert np.all(host(out) == 0.0)
    a = np.float32(1.0 + 2.0**-23)
    yv = W.bf16_bits_from_f32(np.full((2, 8), 1.0 + 2.0**-7, np.float32))
    out, ow = moe.combine(dev_bf16(yv), dev(np.array([[0, 1]], np.int64)), dev(np.float32([[-a, a]])),
                          out_dtype=torch.float32)
    assert np.all(host(out) == 0.0) and host(ow)[0] == 0.0


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skewed_fp8"])
def test_end_to_end_workload(name):
    """dispatch -> expert stand-in -> combine, GPU against oracle at full size."""
    d = W.make_inputs(name)
    E, T, K, H = d["E"], d["T"], d["K"], d["H"]
    cap = int(np.bincount(d["idx"].ravel(), minlength=E).max()) if d["layout"] == "padded" else 0
    fp8 = d["packed_dtype"] == "fp8"
    note(f"e2e {name}")
    o = gpu_dispatch(dev_bf16(d["x"]), d["idx"], E, cap=cap, fp8=fp8)
    ref = oracle.dispatch(d["x"], "bf16", d["idx"], E, cap=cap, packed_dt="fp8" if fp8 else None)
    assert_dispatch_equal(o, ref, fp8=fp8)
    # expert stand-ins (harness, untimed): identity, x*c_e, or fp8 dequantize
    if d["expert"] == "dequant":
        y_ref = oracle.fp8_dequant(ref["packed"], ref["scales"])
        y_dev = moe.fp8_dequant(o.packed, o.scales)
        torch.cuda.synchronize()
        wr = ref["packed_src"] >= 0
        np.testing.assert_array_equal(host(y_dev)[wr], y_ref[wr])
    elif d["expert"] == "scale":
        y_ref = oracle.expert_scale(ref["packed"], ref["packed_cnt"], ref["packed_off"], d["c"])
        y_dev = dev_bf16(y_ref)
    else:
        y_ref = ref["packed"]
        y_dev = o.packed
    out, ow = moe.combine(y_dev, o.tok_map, dev(d["w"]), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    eo, ew = oracle.combine(y_ref, "bf16", ref["tok_map"], d["w"], "bf16")
    exact = _check_combine(host(out), eo, "bf16")
    np.testing.assert_array_equal(host(ow), ew)
    print(f"{name}: combine bit-exact={exact}")


# ---------------------------------------------------------------------------
# fp8 dequant helper
# ---------------------------------------------------------------------------

def test_fp8_dequant_random():
    rng = np.random.default_rng(2)
    q = rng.integers(0, 256, size=(77, 384), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x42
    s = (rng.random((77, 3)) * 8 + 2.0**-6).astype(np.float32)
    note("fp8 dequant random")
    y = moe.fp8_dequant(dev(q), dev(s))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(y), oracle.fp8_dequant(q, s))


# ---------------------------------------------------------------------------
# dedup
# ---------------------------------------------------------------------------

def _gpu_dedup(x_dev, idx_np, E, R, recv_rows=None, cap=0):
    T, H = x_dev.shape
    K = idx_np.shape[1]
    recv_rows = T * min(K, R) if recv_rows is None else recv_rows
    packed_rows = E * cap if cap > 0 else T * K
    o = moe._lib.alloc_dedup(T, H, K, E, R, recv_rows, packed_rows, x_dev.dtype, DEV)
    for f in ("recv_x", "recv_cnt", "recv_off", "recv_src", "rank_slot", "packed", "packed_cnt",
              "packed_off", "packed_src", "tok_map", "stats"):
        poison_(getattr(o, f))
    moe.dedup_dispatch(x_dev, dev(idx_np), E, R, recv_rows=recv_rows, cap=cap, out=o)
    torch.cuda.synchronize()
    return o


def _assert_dedup_equal(o, ref):
    for f in ("recv_cnt", "recv_off", "recv_src", "rank_slot", "packed_cnt", "packed_off",
              "packed_src", "tok_map", "stats"):
        np.testing.assert_array_equal(host(getattr(o, f)), ref[f], err_msg=f)
    for f in ("recv_x", "packed"):
        g = host(getattr(o, f)).view(np.uint8)
        e = ref[f].view(np.uint8)
        assert np.array_equal(g, e), f"{f} rows differ: {np.nonzero(np.any(g != e, axis=1))[0][:8]}"


@pytest.mark.parametrize("case", ["plain", "recv_drop", "padded", "bf16"])
def test_dedup_small(case):
    d = W.make_inputs("dedup", T=1500, seed=11)
    idx = d["idx"].copy()
    rng = np.random.default_rng(4)
    idx[rng.random(idx.shape) < 0.04] = -1
    idx[rng.random(idx.shape) < 0.01] = 999
    E, R, K, T = d["E"], d["R"], d["K"], d["T"]
    x = d["x"] if case != "bf16" else W.bf16_bits_from_f32(d["x"])
    dt = "bf16" if case == "bf16" else "f32"
    full = oracle.dedup_dispatch(x, dt, idx, E, R)
    recv_rows = int(full["recv_off"][R]) - 200 if case == "recv_drop" else T * min(K, R)
    cap = int(full["packed_cnt"].max()) - 3 if case == "padded" else 0
    note(f"dedup {case} recv_rows={recv_rows} cap={cap}")
    o = _gpu_dedup(dev_x(x, dt), idx, E, R, recv_rows=recv_rows, cap=cap)
    ref = oracle.dedup_dispatch(x, dt, idx, E, R, recv_rows=recv_rows, cap=cap)
    _assert_dedup_equal(o, ref)
    # combine: two-stage (partials materialized) and one-kernel forms
    y = ref["packed"]
    for with_partial in (True, False):
        part = torch.empty((recv_rows, d["H"]), dtype=torch.float32, device=DEV) if with_partial else None
        poison_(part)
        plan = dict(R=R, idx=dev(idx), rank_slot=o.rank_slot, recv_rows=recv_rows, partial=part)
        out, ow = moe.combine(o.packed, o.tok_map, dev(d["w"]), E=E, out_dtype=torch.float32, dedup=plan)
        torch.cuda.synchronize()
        eo, ew, ep = oracle.dedup_combine(y, dt, ref["tok_map"], d["w"], idx, E, R, ref["rank_slot"],
                                          recv_rows, "f32", want_partial=True)
        _check_combine(host(out), eo, "f32")
        np.testing.assert_array_equal(host(ow), ew)
        if with_partial:
            n = min(int(ref["recv_off"][R]), recv_rows)
            np.testing.assert_array_equal(host(part)[:n].view(np.uint32), ep[:n].view(np.uint32))


@pytest.mark.parametrize("K,E,R,H", [(2, 16, 4, 256), (4, 64, 32, 128), (5, 40, 8, 512),
                                     (8, 64, 8, 384), (12, 96, 16, 256), (16, 64, 32, 128)])
def test_dedup_shapes(K, E, R, H):
    """Every entry-count instantiation and rank counts up to 32 (several rank
    batches per token in the expansion and the partial sums)."""
    rng = np.random.default_rng(K * 31 + R)
    T = 700
    idx = _mixed_idx(rng, T, K, E)
    x = W.normal_x(rng, T, H, "f32")
    w = rng.random((T, K)).astype(np.float32)
    note(f"dedup shapes K={K} E={E} R={R} H={H}")
    o = _gpu_dedup(dev(x), idx, E, R)
    ref = oracle.dedup_dispatch(x, "f32", idx, E, R)
    _assert_dedup_equal(o, ref)
    rr = T * min(K, R)
    for with_partial in (True, False):
        part = torch.empty((rr, H), dtype=torch.float32, device=DEV) if with_partial else None
        poison_(part)
        plan = dict(R=R, idx=dev(idx), rank_slot=o.rank_slot, recv_rows=rr, partial=part)
        out, ow = moe.combine(o.packed, o.tok_map, dev(w), E=E, out_dtype=torch.float32, dedup=plan)
        torch.cuda.synchronize()
        eo, ew, _ = oracle.dedup_combine(ref["packed"], "f32", ref["tok_map"], w, idx, E, R,
                                         ref["rank_slot"], rr, "f32")
        _check_combine(host(out), eo, "f32")
        np.testing.assert_array_equal(host(ow), ew)


@pytest.mark.parametrize("mode", ["local", "one_rank"])
def test_dedup_local_routing(mode):
    """Routings the dedup exists for: every token's experts inside one virtual
    rank ("local": rank t mod R; "one_rank": rank 0 for all), so each token has
    one recv row that expands to all its experts (and, for one_rank, every
    other rank's segments stay empty)."""
    T, K, E, R, H = 1200, 4, 64, 8, 256
    er = E // R
    rng = np.random.default_rng(77 if mode == "local" else 78)
    rank = np.arange(T) % R if mode == "local" else np.zeros(T, np.int64)
    idx = (rank[:, None] * er + np.argsort(rng.random((T, er)), axis=1)[:, :K]).astype(np.int32)
    idx[rng.random((T, K)) < 0.05] = -1
    x = W.normal_x(rng, T, H, "f32")
    w = rng.random((T, K)).astype(np.float32)
    note(f"dedup {mode} routing")
    o = _gpu_dedup(dev(x), idx, E, R)
    ref = oracle.dedup_dispatch(x, "f32", idx, E, R)
    _assert_dedup_equal(o, ref)
    assert int(ref["recv_off"][R]) == int((idx >= 0).any(axis=1).sum())   # one recv row per token
    rr = T * min(K, R)
    eo, ew, ep = oracle.dedup_combine(ref["packed"], "f32", ref["tok_map"], w, idx, E, R,
                                      ref["rank_slot"], rr, "f32", want_partial=True)
    for with_partial in (True, False):
        part = torch.empty((rr, H), dtype=torch.float32, device=DEV) if with_partial else None
        poison_(part)
        plan = dict(R=R, idx=dev(idx), rank_slot=o.rank_slot, recv_rows=rr, partial=part)
        out, ow = moe.combine(o.packed, o.tok_map, dev(w), E=E, out_dtype=torch.float32, dedup=plan)
        torch.cuda.synchronize()
        _check_combine(host(out), eo, "f32")
        np.testing.assert_array_equal(host(ow), ew)
        if with_partial:
            n = int(ref["recv_off"][R])
            np.testing.assert_array_equal(host(part)[:n].view(np.uint32), ep[:n].view(np.uint32))


@pytest.mark.parametrize("T", [1, 37, 128])
def test_dedup_one_tile(T):
    """Both routing levels of a small dedup dispatch fit one tile (T*R and T*K
    at most 1024): the one-tile routing keeps its counts in LDS."""
    K, E, R, H = 6, 64, 8, 256
    rng = np.random.default_rng(T + 91)
    idx = _mixed_idx(rng, T, K, E)
    x = W.normal_x(rng, T, H, "f32")
    w = rng.random((T, K)).astype(np.float32)
    note(f"dedup one tile T={T}")
    o = _gpu_dedup(dev(x), idx, E, R)
    ref = oracle.dedup_dispatch(x, "f32", idx, E, R)
    _assert_dedup_equal(o, ref)
    rr = T * min(K, R)
    plan = dict(R=R, idx=dev(idx), rank_slot=o.rank_slot, recv_rows=rr)
    out, ow = moe.combine(o.packed, o.tok_map, dev(w), E=E, out_dtype=torch.float32, dedup=plan)
    torch.cuda.synchronize()
    eo, ew, _ = oracle.dedup_combine(ref["packed"], "f32", ref["tok_map"], w, idx, E, R,
                                     ref["rank_slot"], rr, "f32")
    _check_combine(host(out), eo, "f32")
    np.testing.assert_array_equal(host(ow), ew)


def test_dedup_workload_full():
    d = W.make_inputs("dedup")
    E, R, K, T, H = d["E"], d["R"], d["K"], d["T"], d["H"]
    note("dedup full T=16384")
    o = _gpu_dedup(dev(d["x"]), d["idx"], E, R)
    ref = oracle.dedup_dispatch(d["x"], "f32", d["idx"], E, R)
    _assert_dedup_equal(o, ref)
    plain = oracle.dispatch(d["x"], "f32", d["idx"], E)
    np.testing.assert_array_equal(host(o.tok_map), plain["tok_map"])
    rr = T * min(K, R)
    eo, ew, ep = oracle.dedup_combine(ref["packed"], "f32", ref["tok_map"], d["w"], d["idx"], E, R,
                                      ref["rank_slot"], rr, "f32", want_partial=True)
    # fused (partials in registers) and two-stage (partial rows through memory)
    for with_partial in (False, True):
        part = torch.empty((rr, H), dtype=torch.float32, device=DEV) if with_partial else None
        poison_(part)
        plan = dict(R=R, idx=dev(d["idx"]), rank_slot=o.rank_slot, recv_rows=rr, partial=part)
        out, ow = moe.combine(o.packed, o.tok_map, dev(d["w"]), E=E, out_dtype=torch.float32,
                              dedup=plan)
        torch.cuda.synchronize()
        _check_combine(host(out), eo, "f32")
        np.testing.assert_array_equal(host(ow), ew)
        if with_partial:
            n = int(ref["recv_off"][R])
            np.testing.assert_array_equal(host(part)[:n].view(np.uint32), ep[:n].view(np.uint32))
        del part


# ---------------------------------------------------------------------------
# determinism
# ---------------------------------------------------------------------------

def test_repeat_launches_bitwise_identical():
    d = W.make_inputs("skewed_fp8", T=2048)
    x = dev_bf16(d["x"])
    idx = dev(d["idx"])
    w = dev(d["w"])
    note("determinism x100")
    o = moe.dispatch(x, idx, d["E"], fp8=True)
    y = moe.fp8_dequant(o.packed, o.scales)
    out0, _ = moe.combine(y, o.tok_map, w)
    tm0, pk0, sc0 = o.tok_map.clone(), o.packed.clone(), o.scales.clone()
    for _ in range(100):
        o2 = moe.dispatch(x, idx, d["E"], fp8=True, out=o)
        out, _ = moe.combine(y, o2.tok_map, w)
        assert torch.equal(o2.tok_map, tm0) and torch.equal(o2.packed, pk0)
        assert torch.equal(o2.scales.view(torch.int32), sc0.view(torch.int32))
        assert torch.equal(out.view(torch.int16), out0.view(torch.int16))


@pytest.mark.parametrize("payload,H", [("bf16", 65536), ("f32", 32768), ("fp8", 65536),
                                       ("fp4", 65536), ("prequant", 65536)])
def test_wide_rows(payload, H):
    """Rows far wider than one pass of a workgroup (128 KB bf16 / f32 rows, 512
    scale blocks): every row mover loops over passes, the e4m3 halves hold 256
    blocks each, and the combines run 32-64 chunks per token."""
    T, K, E = 40, 4, 16
    rng = np.random.default_rng(H + len(payload))
    idx = _mixed_idx(rng, T, K, E)
    w = rng.standard_normal((T, K)).astype(np.float32)
    note(f"wide rows {payload} H={H}")
    if payload == "prequant":
        x = rng.integers(0, 256, size=(T, H), dtype=np.uint8)
        x[(x & 0x7F) == 0x7F] = 0x11                    # no NaN codes: plain comparison below
        xs = (rng.random((T, H // 128)) * 4 + 2.0**-8).astype(np.float32)
        o = moe._lib.alloc_dispatch(T, H, K, E, T * K, torch.uint8, True, DEV)
        for t in (o.packed, o.scales, o.packed_src, o.tok_map, o.packed_cnt, o.packed_off, o.stats):
            poison_(t)
        moe.dispatch_prequant(dev(x), dev(xs), dev(idx), E, out=o)
        torch.cuda.synchronize()
        ref = oracle.dispatch(x, "fp8", idx, E, x_scales=xs)
    else:
        dt = "f32" if payload == "f32" else "bf16"
        x = W.normal_x(rng, T, H, dt)
        if payload in ("fp8", "fp4"):
            x = W.inject_outliers(x, np.arange(0, T, 3), 1000.0)
        o = gpu_dispatch(dev_x(x, dt), idx, E, fp8=payload == "fp8", fp4=payload == "fp4")
        ref = oracle.dispatch(x, dt, idx, E, packed_dt=payload if payload in ("fp8", "fp4") else None)
    quant = payload in ("fp8", "fp4", "prequant")
    assert_dispatch_equal(o, ref, fp8=quant)
    if payload in ("bf16", "f32"):
        out, ow = moe.combine(o.packed, o.tok_map, dev(w), out_dtype=torch.bfloat16)
        eo, ew = oracle.combine(ref["packed"], payload, ref["tok_map"], w, "bf16")
    elif payload == "fp4":
        out, ow = moe.combine_fp4(o.packed, o.scales, o.tok_map, dev(w))
        eo, ew = oracle.combine_fp4(ref["packed"], ref["scales"], ref["tok_map"], w, "bf16")
    else:
        out, ow = moe.combine_fp8(o.packed, o.scales, o.tok_map, dev(w))
        eo, ew = oracle.combine_fp8(ref["packed"], ref["scales"], ref["tok_map"], w, "bf16")
    torch.cuda.synchronize()
    _check_combine(host(out), eo, "bf16")
    np.testing.assert_array_equal(host(ow), ew)


def test_grid_stride_wrap_past_max_grid():
    """More tokens than the launch cap of 2^22 workgroups, so the token loops
    wrap; small rows keep it cheap.  Covers dispatch, fp8 pack and combine."""
    T, K, E, H = (1 << 22) + 37, 1, 4, 128
    rng = np.random.default_rng(21)
    idx = rng.integers(-1, E, size=(T, K)).astype(np.int32)
    x = rng.integers(0, 1 << 16, size=(T, H), dtype=np.uint16)
    x[(x & 0x7F80) == 0x7F80] = 0x3F80            # no inf/nan patterns
    note(f"grid wrap T={T}")
    for fp8 in (False, True):
        o = gpu_dispatch(dev_bf16(x), idx, E, fp8=fp8)
        ref = oracle.dispatch(x, "bf16", idx, E, packed_dt="fp8" if fp8 else None)
        assert_dispatch_equal(o, ref, fp8=fp8)
    w = rng.random((T, K)).astype(np.float32)
    plain = oracle.dispatch(x, "bf16", idx, E)
    out, ow = moe.combine(dev_bf16(plain["packed"]), dev(plain["tok_map"]), dev(w),
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    eo, ew = oracle.combine(plain["packed"], "bf16", plain["tok_map"], w, "f32")
    _check_combine(host(out), eo, "f32")
    np.testing.assert_array_equal(host(ow), ew)


@pytest.mark.parametrize("payload,H", [("bf16", 7168), ("fp8", 16384)])
def test_byte_offsets_past_4gib(payload, H):
    """Packed buffers larger than 4 GiB (320000 rows of 14 KB bf16 or 16 KB e4m3):
    the rows at the end lie past 2^32 bytes, so any 32-bit row offset would land
    elsewhere.  Routing outputs in full (numpy's stable sort states the slot
    rule independently); rows, scales and the combine on sampled rows and
    tokens, the last ones included, against the oracle."""
    T, K, E = 40000, 8, 256
    rng = np.random.default_rng(44)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    x = rng.integers(0, 1 << 16, size=(T, H), dtype=np.uint16)
    x[(x & 0x7F80) == 0x7F80] = 0x3F80            # finite values only
    fp8 = payload == "fp8"
    note(f"byte offsets past 4 GiB: {payload} T={T} K={K} E={E} H={H}")
    o = gpu_dispatch(dev_bf16(x), idx, E, fp8=fp8)
    row_bytes = H if fp8 else 2 * H
    assert T * K * row_bytes > (1 << 32)
    flat = idx.ravel()
    order = np.argsort(flat, kind="stable")
    tm = np.empty(T * K, np.int64)
    tm[order] = np.arange(T * K)
    np.testing.assert_array_equal(host(o.tok_map).ravel(), tm)
    np.testing.assert_array_equal(host(o.packed_src), (order // K).astype(np.int32))
    rc, ro, _ = oracle.route_count(idx, E)
    np.testing.assert_array_equal(host(o.packed_cnt), rc)
    np.testing.assert_array_equal(host(o.packed_off), ro)
    # sampled rows: the last 2000 (all past 2^32 bytes) and 2000 spread out
    rows = np.unique(np.concatenate([np.arange(T * K - 2000, T * K),
                                     rng.integers(0, T * K, 2000)]))
    assert rows[-1] * row_bytes > (1 << 32)
    src = order[rows] // K
    got = host(o.packed[torch.from_numpy(rows).to(DEV)])
    if fp8:
        q, sc = oracle.fp8_pack_rows(x[src])
        np.testing.assert_array_equal(got, q)
        np.testing.assert_array_equal(host(o.scales[torch.from_numpy(rows).to(DEV)]).view(np.uint32),
                                      sc.view(np.uint32))
    else:
        np.testing.assert_array_equal(got.view(np.uint16), x[src])
    # combine of sampled tokens (the last ones read the rows past 2^32 bytes):
    # the oracle combines the same tokens over the rows they name
    w = rng.random((T, K)).astype(np.float32)
    if fp8:
        out, ow = moe.combine_fp8(o.packed, o.scales, o.tok_map, dev(w))
    else:
        out, ow = moe.combine(o.packed, o.tok_map, dev(w))
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([order[-2000:] // K, rng.integers(0, T, 1000)]))
    sub_rows = np.unique(tm.reshape(T, K)[toks].ravel())
    remap = {int(r): i for i, r in enumerate(sub_rows)}
    sub_tm = np.vectorize(lambda r: remap[int(r)])(tm.reshape(T, K)[toks]).astype(np.int64)
    y_sub = host(o.packed[torch.from_numpy(sub_rows).to(DEV)])
    if fp8:
        s_sub = host(o.scales[torch.from_numpy(sub_rows).to(DEV)])
        eo, ew = oracle.combine_fp8(y_sub, s_sub, sub_tm, w[toks], "bf16")
    else:
        eo, ew = oracle.combine(y_sub.view(np.uint16), "bf16", sub_tm, w[toks], "bf16")
    assert _check_combine(host(out[torch.from_numpy(toks).to(DEV)]), eo, "bf16")
    np.testing.assert_array_equal(host(ow)[toks], ew)


def test_dedup_byte_offsets_past_4gib():
    """Dedup dispatch and combine with recv and packed buffers larger than 4 GiB
    (about 272000 recv rows and 360000 packed rows of 16 KB f32): recv and
    packed rows at the end lie past 2^32 bytes.  Routing outputs in full
    against numpy statements of the rank-mask and slot rules, rows and the
    fused and two-stage combines on samples against the oracle."""
    T, K, E, R, H = 60000, 6, 64, 8, 4096
    er = E // R
    rng = np.random.default_rng(45)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    x = rng.standard_normal((T, H), dtype=np.float32)
    note(f"dedup byte offsets past 4 GiB: T={T} K={K} E={E} R={R} H={H}")
    o = _gpu_dedup(dev(x), idx, E, R)
    # rank masks and recv rows: for each rank, its tokens in token order
    mask = np.zeros(T, np.int64)
    for k in range(K):
        mask |= 1 << (idx[:, k] // er)
    rs = np.full((T, R), -1, np.int64)
    recv_src = []
    base = 0
    for r in range(R):
        toks = np.nonzero(mask & (1 << r))[0]
        rs[toks, r] = base + np.arange(len(toks))
        recv_src.append(toks)
        base += len(toks)
    recv_src = np.concatenate(recv_src)
    n_recv = base
    assert n_recv * H * 4 > (1 << 32)
    np.testing.assert_array_equal(host(o.rank_slot), rs.astype(np.int32))
    np.testing.assert_array_equal(host(o.recv_src)[:n_recv], recv_src.astype(np.int32))
    order = np.argsort(idx.ravel(), kind="stable")
    tm = np.empty(T * K, np.int64)
    tm[order] = np.arange(T * K)
    np.testing.assert_array_equal(host(o.tok_map).ravel(), tm)
    np.testing.assert_array_equal(host(o.stats), np.zeros(3, np.int32))
    for buf, src, n in ((o.recv_x, recv_src, n_recv), (o.packed, order // K, T * K)):
        rows = np.unique(np.concatenate([np.arange(n - 1500, n), rng.integers(0, n, 1500)]))
        got = host(buf[torch.from_numpy(rows).to(DEV)])
        np.testing.assert_array_equal(got.view(np.uint32), x[src[rows]].view(np.uint32))
    # combines of sampled tokens, the last ones included
    w = rng.random((T, K)).astype(np.float32)
    toks = np.unique(np.concatenate([np.arange(T - 1000, T), rng.integers(0, T, 1000)]))
    sub_rows = np.unique(tm.reshape(T, K)[toks].ravel())
    lookup = np.full(T * K, -1, np.int64)
    lookup[sub_rows] = np.arange(len(sub_rows))
    sub_tm = lookup[tm.reshape(T, K)[toks]]
    y_sub = x[(order // K)[sub_rows]]           # the identity expert: packed rows are x rows
    eo, ew, _ = oracle.dedup_combine(y_sub, "f32", sub_tm, w[toks], idx[toks], E, R,
                                     rs[toks].astype(np.int32), (1 << 31) - 1, "f32")
    rr = T * min(K, R)
    for with_partial in (False, True):
        part = torch.empty((rr, H), dtype=torch.float32, device=DEV) if with_partial else None
        plan = dict(R=R, idx=dev(idx), rank_slot=o.rank_slot, recv_rows=rr, partial=part)
        out, ow = moe.combine(o.packed, o.tok_map, dev(w), E=E, out_dtype=torch.float32,
                              dedup=plan)
        torch.cuda.synchronize()
        _check_combine(host(out[torch.from_numpy(toks).to(DEV)]), eo, "f32")
        np.testing.assert_array_equal(host(ow)[toks], ew)
        del part, out


# ---------------------------------------------------------------------------
# one-launch routing: the arrival ticket lives in the caller's workspace
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fill", [0x00, 0xFF, 0xA5, "random"])
def test_routing_any_workspace_contents(fill):
    """The workspace needs no initialisation: whatever it holds (including a
    ticket left by an earlier call), every call counts its own tiles."""
    T, K, E = 5000, 8, 256
    rng = np.random.default_rng(31)
    idx = _mixed_idx(rng, T, K, E)
    ws = moe.workspace(T, K, E)
    if fill == "random":
        ws.copy_(torch.from_numpy(rng.integers(0, 256, ws.numel(), dtype=np.uint8)).to(DEV))
    else:
        ws.fill_(fill)
    rc, ro, rs = oracle.route_count(idx, E)
    idx_d = dev(idx)
    note(f"routing workspace fill={fill}")
    for _ in range(3):
        cnt, off, st = moe.route_count(idx_d, E, ws=ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(cnt), rc)
        np.testing.assert_array_equal(host(off), ro)
        np.testing.assert_array_equal(host(st), rs)


@pytest.mark.parametrize("T", [3000, 100])
def test_dispatch_graph_replays(T):
    """A captured dispatch replays with the same launch arguments each time;
    every replay, with eager launches on the same workspace in between, must
    give the eager result.  T=100 (800 entries) is the one-launch dispatch."""
    K, E, H = 8, 64, 256
    rng = np.random.default_rng(37)
    idx = _mixed_idx(rng, T, K, E)
    x = W.normal_x(rng, T, H, "bf16")
    ref = oracle.dispatch(x, "bf16", idx, E, packed_dt="fp8")
    x_d, idx_d = dev_bf16(x), dev(idx)
    ws = moe.workspace(T, K, E)
    o = moe._lib.alloc_dispatch(T, H, K, E, T * K, x_d.dtype, True, DEV)
    other = moe._lib.alloc_dispatch(T, H, K, E, T * K, x_d.dtype, True, DEV)
    note("dispatch graph capture")
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        moe.dispatch(x_d, idx_d, E, fp8=True, out=o, ws=ws)   # warm up on the capture stream
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cs):
            moe.dispatch(x_d, idx_d, E, fp8=True, out=o, ws=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (o.packed, o.scales, o.packed_src, o.tok_map, o.packed_cnt, o.packed_off, o.stats):
            poison_(t)
        note(f"dispatch graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert_dispatch_equal(o, ref, fp8=True)
        for t in (other.packed, other.scales, other.packed_src, other.tok_map, other.packed_cnt,
                  other.packed_off, other.stats):
            poison_(t)   # rows past the counts keep the poison, as in the oracle
        moe.dispatch(x_d, idx_d, E, fp8=True, out=other, ws=ws)  # eager call in between
        torch.cuda.synchronize()
        assert_dispatch_equal(other, ref, fp8=True)


def _concurrent_setups():
    """Two independent callers' inputs, buffers, workspaces and streams: a
    one-launch dispatch (bf16) and a multi-tile one with the fp8 pack."""
    cases = [(100, 8, 64, 256, False), (3000, 8, 256, 512, True)]
    setups = []
    for n, (T, K, E, H, fp8) in enumerate(cases):
        rng = np.random.default_rng(500 + n)
        idx = _mixed_idx(rng, T, K, E)
        x = W.normal_x(rng, T, H, "bf16")
        w = rng.random((T, K)).astype(np.float32)
        if fp8:
            x = W.inject_outliers(x, np.arange(0, T, 31), 1000.0)   # some scaled blocks
        ref = oracle.dispatch(x, "bf16", idx, E, packed_dt="fp8" if fp8 else None)
        if fp8:
            eo, ew = oracle.combine_fp8(ref["packed"], ref["scales"], ref["tok_map"], w, "bf16")
        else:
            eo, ew = oracle.combine(ref["packed"], "bf16", ref["tok_map"], w, "bf16")
        st = torch.cuda.Stream()
        o = moe._lib.alloc_dispatch(T, H, K, E, T * K, torch.bfloat16, fp8, DEV)
        for t in (o.packed, o.scales, o.packed_src, o.tok_map, o.packed_cnt, o.packed_off, o.stats):
            poison_(t)   # rows past the counts are never written: they keep the poison
        setups.append(dict(E=E, fp8=fp8, st=st, ws=moe.workspace(T, K, E), o=o, x=dev_bf16(x),
                           idx=dev(idx), w=dev(w), ref=ref, eo=eo, ew=ew,
                           out=torch.empty((T, H), dtype=torch.bfloat16, device=DEV),
                           ow=torch.empty(T, dtype=torch.float32, device=DEV)))
    torch.cuda.synchronize()
    return setups


def _round(s_):
    with torch.cuda.stream(s_["st"]):
        moe.dispatch(s_["x"], s_["idx"], s_["E"], fp8=s_["fp8"], out=s_["o"], ws=s_["ws"])
        if s_["fp8"]:
            moe.combine_fp8(s_["o"].packed, s_["o"].scales, s_["o"].tok_map, s_["w"],
                            out=s_["out"], out_weights=s_["ow"])
        else:
            moe.combine(s_["o"].packed, s_["o"].tok_map, s_["w"], out=s_["out"],
                        out_weights=s_["ow"])


def _check_setups(setups):
    for s_ in setups:
        assert_dispatch_equal(s_["o"], s_["ref"], fp8=s_["fp8"])
        _check_combine(host(s_["out"]), s_["eo"], "bf16")
        np.testing.assert_array_equal(host(s_["ow"]), s_["ew"])


def test_two_streams_two_workspaces():
    """The library keeps no state between calls: two streams, each with its own
    workspace and buffers, dispatch and combine concurrently, many times over;
    both end with the oracle's results."""
    setups = _concurrent_setups()
    note("two streams, two workspaces")
    for it in range(50):
        for s_ in setups:
            _round(s_)
    torch.cuda.synchronize()
    _check_setups(setups)


def test_two_host_threads():
    """The same two callers, each driven from a host thread of its own (ctypes
    releases the GIL, so the library's host code runs concurrently): argument
    checks, workspace carving and launches share nothing but the HIP runtime."""
    import threading
    setups = _concurrent_setups()
    note("two host threads, two streams, two workspaces")
    errors = []

    def run(s_):
        try:
            torch.cuda.set_device(0)
            for it in range(50):
                _round(s_)
            s_["st"].synchronize()
        except Exception as e:   # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=run, args=(s_,)) for s_ in setups]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a host thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    _check_setups(setups)


@pytest.mark.parametrize("nbytes", [0, 16, 4096 + 16, (1 << 20) + 48])
def test_copy16_bytes(nbytes):
    """The copy-ceiling helper moves the bytes exactly (grid tail included)."""
    rng = np.random.default_rng(nbytes)
    src = torch.from_numpy(rng.integers(0, 256, nbytes + 16, dtype=np.uint8)).to(DEV)
    dst = torch.full((nbytes + 16,), 0xA5, dtype=torch.uint8, device=DEV)
    note(f"copy16 bytes={nbytes}")
    moe.copy16(src[:nbytes], dst[:nbytes])
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes])
    assert bool((dst[nbytes:] == 0xA5).all()), "copy wrote past its end"


# ---------------------------------------------------------------------------
# combine of fp8 expert outputs
# ---------------------------------------------------------------------------

def _fp8_codes(rng, shape):
    q = rng.integers(0, 256, size=shape, dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38          # no NaN codes
    return q


@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
@pytest.mark.parametrize("K,H,T,scaled", [(1, 128, 37, True), (3, 384, 300, True), (8, 7168, 129, True),
                                          (8, 7168, 65, False), (16, 256, 513, True), (6, 4096, 1000, False)])
def test_combine_fp8_random(out_dt, K, H, T, scaled):
    rng = np.random.default_rng(K * 1000 + H + T)
    rows = max(T * K // 2, K)
    q = _fp8_codes(rng, (rows, H))
    sc = (rng.random((rows, H // 128)) * 8 + 2.0 ** -6).astype(np.float32) if scaled else None
    tm = rng.integers(-1, rows, size=(T, K)).astype(np.int64)
    tm[rng.random((T, K)) < 0.02] = rows + 3          # out of range: skipped
    w = rng.standard_normal((T, K)).astype(np.float32)
    note(f"combine_fp8 K={K} H={H} T={T} scaled={scaled} out={out_dt}")
    odt = torch.float32 if out_dt == "f32" else torch.bfloat16
    out = torch.empty((T, H), dtype=odt, device=DEV)
    ow = torch.empty(T, dtype=torch.float32, device=DEV)
    poison_(out)
    poison_(ow)
    moe.combine_fp8(dev(q), dev(sc) if scaled else None, dev(tm), dev(w), out=out, out_weights=ow)
    torch.cuda.synchronize()
    exp, ew = oracle.combine_fp8(q, sc, tm, w, out_dt)
    exact = _check_combine(host(out), exp, out_dt)
    np.testing.assert_array_equal(host(ow), ew)
    print(f"bit-exact={exact}")


def test_combine_fp8_direct_cast_equals_bf16_combine():
    """No scales: the fp8 combine equals the bf16 combine of the decoded rows
    (both on the GPU, bitwise)."""
    rng = np.random.default_rng(7)
    rows, H, T, K = 3000, 1024, 700, 8
    q = _fp8_codes(rng, (rows, H))
    tm = rng.integers(-1, rows, size=(T, K)).astype(np.int64)
    w = rng.random((T, K)).astype(np.float32)
    qd = dev(q)
    yb = qd.view(torch.float8_e4m3fn).to(torch.bfloat16)
    note("combine_fp8 direct cast vs bf16 combine")
    a, aw = moe.combine_fp8(qd, None, dev(tm), dev(w))
    b, bw = moe.combine(yb, dev(tm), dev(w))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(aw, bw)


def test_combine_fp8_skewed_full():
    """The metric workload with the fp8 packed rows themselves as the expert
    output (identity expert, no dequantize pass)."""
    d = W.make_inputs("skewed_fp8")
    x = W.inject_outliers(d["x"], np.arange(0, d["T"], 97), 1000.0)
    note("combine_fp8 skewed_fp8 full T=8192")
    o = gpu_dispatch(dev_bf16(x), d["idx"], d["E"], fp8=True)
    out, ow = moe.combine_fp8(o.packed, o.scales, o.tok_map, dev(d["w"]))
    torch.cuda.synchronize()
    ref = oracle.dispatch(x, "bf16", d["idx"], d["E"], packed_dt="fp8")
    exp, ew = oracle.combine_fp8(ref["packed"], ref["scales"], ref["tok_map"], d["w"], "bf16")
    assert _check_combine(host(out), exp, "bf16")
    np.testing.assert_array_equal(host(ow), ew)


# ---------------------------------------------------------------------------
# pre-quantized dispatch and replay dispatch
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["compact", "padded", "padded_tight", "compact_short"])
@pytest.mark.parametrize("T,K,E,H", [(300, 4, 13, 128), (2100, 8, 256, 384), (64, 2, 8, 7168)])
def test_dispatch_prequant_small(layout, T, K, E, H):
    rng = np.random.default_rng(T * 5 + K + H)
    idx = _mixed_idx(rng, T, K, E)
    q = rng.integers(0, 256, size=(T, H), dtype=np.uint8)
    sc = (rng.random((T, H // 128)) + 0.5).astype(np.float32)
    flat = idx.ravel()
    cnt = np.bincount(flat[(flat >= 0) & (flat < E)], minlength=E)
    cap = {"compact": 0, "padded": int(cnt.max()), "padded_tight": max(1, int(cnt.max()) // 2),
           "compact_short": 0}[layout]
    rows = {"compact": T * K, "padded": E * cap, "padded_tight": E * cap - 3,
            "compact_short": max(0, int(cnt.sum()) - 37)}[layout]
    note(f"dispatch_prequant {layout} T={T} K={K} E={E} H={H} cap={cap} rows={rows}")
    o = moe._lib.alloc_dispatch(T, H, K, E, rows, torch.uint8, True, DEV)
    for t in (o.packed, o.scales, o.packed_src, o.tok_map, o.packed_cnt, o.packed_off, o.stats):
        poison_(t)
    moe.dispatch_prequant(dev(q), dev(sc), dev(idx), E, cap=cap, packed_rows=rows, out=o)
    torch.cuda.synchronize()
    ref = oracle.dispatch(q, "fp8", idx, E, cap=cap, packed_rows=rows, x_scales=sc)
    assert_dispatch_equal(o, ref, fp8=True)


def test_dispatch_prequant_full():
    d = W.make_inputs("skewed_fp8")
    rng = np.random.default_rng(41)
    q, sc = oracle.fp8_pack_rows(W.inject_outliers(d["x"], np.arange(0, d["T"], 97), 1000.0))
    note("dispatch_prequant full T=8192")
    o = moe._lib.alloc_dispatch(d["T"], d["H"], d["K"], d["E"], d["T"] * d["K"], torch.uint8, True, DEV)
    for t in (o.packed, o.scales, o.packed_src, o.tok_map, o.packed_cnt, o.packed_off, o.stats):
        poison_(t)
    moe.dispatch_prequant(dev(q), dev(sc), dev(d["idx"]), d["E"], out=o)
    torch.cuda.synchronize()
    ref = oracle.dispatch(q, "fp8", d["idx"], d["E"], x_scales=sc)
    assert_dispatch_equal(o, ref, fp8=True)


def _replay_map(rng, T, K, rows, extra=8):
    tm = rng.permutation(rows + extra)[:T * K].astype(np.int64).reshape(T, K)
    tm[rng.random((T, K)) < 0.1] = -1
    return tm


@pytest.mark.parametrize("mode", ["bf16", "f32", "fp8_pack", "prequant"])
@pytest.mark.parametrize("T,K,H", [(1, 1, 128), (300, 4, 256), (1500, 8, 7168)])
def test_dispatch_replay_random_map(mode, T, K, H):
    """A cached map with -1 entries and rows past packed_rows (skipped); rows
    nobody names keep their poison."""
    rng = np.random.default_rng(T + K + H)
    rows = T * K + 5
    tm = _replay_map(rng, T, K, rows)
    xs = None
    if mode == "prequant":
        x = rng.integers(0, 256, size=(T, H), dtype=np.uint8)
        xs = (rng.random((T, H // 128)) + 0.5).astype(np.float32)
        x_dev, xdt, pdt = dev(x), "fp8", "fp8"
    else:
        xdt = "f32" if mode == "f32" else "bf16"
        x = W.inject_outliers(W.normal_x(rng, T, H, xdt), np.arange(0, T, 11), 1000.0) if xdt == "bf16" else W.normal_x(rng, T, H, xdt)
        x_dev = dev_x(x, xdt)
        pdt = "fp8" if mode == "fp8_pack" else xdt
    fp8 = pdt == "fp8"
    pt = torch.uint8 if fp8 else x_dev.dtype
    packed = torch.empty((rows, H), dtype=pt, device=DEV)
    scales = torch.empty((rows, H // 128), dtype=torch.float32, device=DEV) if fp8 else None
    poison_(packed)
    poison_(scales)
    note(f"dispatch_replay {mode} T={T} K={K} H={H}")
    moe.dispatch_replay(x_dev, dev(tm), packed, scales=scales, x_scales=dev(xs) if xs is not None else None)
    torch.cuda.synchronize()
    ref = oracle.dispatch_replay(x, xdt, tm, rows, packed_dt=pdt, x_scales=xs)
    np.testing.assert_array_equal(host(packed).view(np.uint8), ref["packed"].view(np.uint8))
    if fp8:
        np.testing.assert_array_equal(host(scales).view(np.uint32), ref["scales"].view(np.uint32))


def test_dispatch_replay_equals_routed_dispatch():
    """Replaying the metric workload's own tok_map reproduces the routed
    dispatch's packed rows and scales bitwise, with new token rows each time."""
    d = W.make_inputs("skewed_fp8")
    E = d["E"]
    note("dispatch_replay after routed dispatch, T=8192 fp8")
    o = gpu_dispatch(dev_bf16(d["x"]), d["idx"], E, fp8=True)
    x2 = W.inject_outliers(W.normal_x(np.random.default_rng(5), d["T"], d["H"], "bf16"),
                           np.arange(0, d["T"], 13), 1000.0)
    packed = torch.empty_like(o.packed)
    scales = torch.empty_like(o.scales)
    poison_(packed)
    poison_(scales)
    moe.dispatch_replay(dev_bf16(x2), o.tok_map, packed, scales=scales)
    o2 = gpu_dispatch(dev_bf16(x2), d["idx"], E, fp8=True)
    torch.cuda.synchronize()
    assert torch.equal(packed, o2.packed)
    assert torch.equal(scales.view(torch.int32), o2.scales.view(torch.int32))


# ---------------------------------------------------------------------------
# fp4 (e2m1) payload
# ---------------------------------------------------------------------------

def test_fp4_encoder_exhaustive_via_dispatch():
    """Every bf16 value with |v| <= 6 goes through the unscaled branch once; the
    finite values up to 448 fill scaled rows (arbitrary f32 quotients)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = W.f32_from_bf16_bits(bits)
    small = bits[np.isfinite(v) & (np.abs(v) <= 6)]
    big = bits[np.isfinite(v) & (np.abs(v) <= 448)]
    H = 1024
    n = (len(small) + H - 1) // H * H
    xs = np.resize(small, n).reshape(-1, H)
    rng = np.random.default_rng(4)
    nb = (len(big) + H - 1) // H * H
    sc = rng.permutation(np.resize(big, nb)).reshape(-1, H)
    scf = W.f32_from_bf16_bits(sc)
    scf[:, ::131] = np.float32(3000.0)
    x = np.concatenate([xs, W.bf16_bits_from_f32(scf)])
    T = x.shape[0]
    idx = np.zeros((T, 1), np.int32)
    note(f"fp4 exhaustive T={T} H={H}")
    o = gpu_dispatch(dev_bf16(x), idx, 1, fp4=True)
    ref = oracle.dispatch(x, "bf16", idx, 1, packed_dt="fp4")
    assert_dispatch_equal(o, ref, fp8=True)


@pytest.mark.parametrize("layout", ["compact", "padded_tight", "compact_short"])
@pytest.mark.parametrize("T,K,E,H", [(300, 4, 13, 128), (2100, 8, 256, 384)])
def test_dispatch_fp4_small(layout, T, K, E, H):
    rng = np.random.default_rng(T + K * 3 + H)
    idx = _mixed_idx(rng, T, K, E)
    x = W.inject_outliers(W.normal_x(rng, T, H, "bf16"), np.arange(0, T, 17), 100.0)
    flat = idx.ravel()
    cnt = np.bincount(flat[(flat >= 0) & (flat < E)], minlength=E)
    cap = {"compact": 0, "padded_tight": max(1, int(cnt.max()) // 2), "compact_short": 0}[layout]
    rows = {"compact": T * K, "padded_tight": E * cap - 3,
            "compact_short": max(0, int(cnt.sum()) - 37)}[layout]
    note(f"dispatch fp4 {layout} T={T} K={K} E={E} H={H}")
    o = gpu_dispatch(dev_bf16(x), idx, E, cap=cap, packed_rows=rows, fp4=True)
    ref = oracle.dispatch(x, "bf16", idx, E, cap=cap, packed_rows=rows, packed_dt="fp4")
    assert_dispatch_equal(o, ref, fp8=True)


# The e4m3 scatter splits each token row over two workgroups of whole scale
# blocks: one block (no split), an odd block count (uneven halves), and halves
# wider than one pass of the workgroup (H=16512: 65 blocks per half).
@pytest.mark.parametrize("layout", ["compact", "padded_tight", "compact_short"])
@pytest.mark.parametrize("T,K,E,H", [(300, 4, 13, 128), (2100, 8, 256, 384), (257, 8, 64, 7296),
                                     (97, 3, 7, 16512)])
def test_dispatch_fp8_small(layout, T, K, E, H):
    rng = np.random.default_rng(T + K * 5 + H)
    idx = _mixed_idx(rng, T, K, E)
    x = W.inject_outliers(W.normal_x(rng, T, H, "bf16"), np.arange(0, T, 13), 1000.0)
    flat = idx.ravel()
    cnt = np.bincount(flat[(flat >= 0) & (flat < E)], minlength=E)
    cap = {"compact": 0, "padded_tight": max(1, int(cnt.max()) // 2), "compact_short": 0}[layout]
    rows = {"compact": T * K, "padded_tight": E * cap - 3,
            "compact_short": max(0, int(cnt.sum()) - 37)}[layout]
    note(f"dispatch fp8 {layout} T={T} K={K} E={E} H={H}")
    o = gpu_dispatch(dev_bf16(x), idx, E, cap=cap, packed_rows=rows, fp8=True)
    ref = oracle.dispatch(x, "bf16", idx, E, cap=cap, packed_rows=rows, packed_dt="fp8")
    assert_dispatch_equal(o, ref, fp8=True)


@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
@pytest.mark.parametrize("K,H,T,scaled", [(1, 128, 37, True), (3, 384, 300, False), (8, 7168, 129, True),
                                          (16, 256, 513, True)])
def test_combine_fp4_random(out_dt, K, H, T, scaled):
    rng = np.random.default_rng(K * 100 + H + T + 1)
    rows = max(T * K // 2, K)
    q = rng.integers(0, 256, size=(rows, H // 2), dtype=np.uint8)
    sc = (rng.random((rows, H // 128)) * 8 + 2.0 ** -6).astype(np.float32) if scaled else None
    tm = rng.integers(-1, rows, size=(T, K)).astype(np.int64)
    tm[rng.random((T, K)) < 0.02] = rows + 3
    w = rng.standard_normal((T, K)).astype(np.float32)
    note(f"combine_fp4 K={K} H={H} T={T} scaled={scaled} out={out_dt}")
    odt = torch.float32 if out_dt == "f32" else torch.bfloat16
    out = torch.empty((T, H), dtype=odt, device=DEV)
    ow = torch.empty(T, dtype=torch.float32, device=DEV)
    poison_(out)
    poison_(ow)
    moe.combine_fp4(dev(q), dev(sc) if scaled else None, dev(tm), dev(w), out=out, out_weights=ow)
    torch.cuda.synchronize()
    exp, ew = oracle.combine_fp4(q, sc, tm, w, out_dt)
    _check_combine(host(out), exp, out_dt)
    np.testing.assert_array_equal(host(ow), ew)


def test_fp4_end_to_end_skewed_full():
    """The metric shape with an fp4 payload: dispatch packs, the packed rows are
    the expert outputs (identity expert), combine_fp4 reduces; and a replay of
    the same map reproduces the packed rows."""
    d = W.make_inputs("skewed_fp8")
    x = W.inject_outliers(d["x"], np.arange(0, d["T"], 97), 1000.0)
    note("fp4 end to end skewed T=8192")
    o = gpu_dispatch(dev_bf16(x), d["idx"], d["E"], fp4=True)
    out, ow = moe.combine_fp4(o.packed, o.scales, o.tok_map, dev(d["w"]))
    packed = torch.empty_like(o.packed)
    scales = torch.empty_like(o.scales)
    moe.dispatch_replay(dev_bf16(x), o.tok_map, packed, scales=scales, fp4=True)
    torch.cuda.synchronize()
    ref = oracle.dispatch(x, "bf16", d["idx"], d["E"], packed_dt="fp4")
    assert_dispatch_equal(o, ref, fp8=True)
    exp, ew = oracle.combine_fp4(ref["packed"], ref["scales"], ref["tok_map"], d["w"], "bf16")
    assert _check_combine(host(out), exp, "bf16")
    np.testing.assert_array_equal(host(ow), ew)
    assert torch.equal(packed, o.packed) and torch.equal(scales.view(torch.int32), o.scales.view(torch.int32))


# ---------------------------------------------------------------------------
# one-launch dispatch of a single routing tile (T*K <= 1024, E <= 512) and its
# boundary: the same ids just inside and just outside it give the oracle's
# outputs either way
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,K,E", [(128, 8, 512), (128, 8, 513), (129, 8, 64), (1024, 1, 7)])
@pytest.mark.parametrize("layout", ["compact", "padded_tight"])
@pytest.mark.parametrize("payload", ["bf16", "f32", "fp8", "fp4", "prequant"])
def test_dispatch_one_tile_boundary(T, K, E, layout, payload):
    rng = np.random.default_rng(T + K + E)
    idx = _mixed_idx(rng, T, K, E)
    H = 256
    flat = idx.ravel()
    cnt = np.bincount(flat[(flat >= 0) & (flat < E)], minlength=E)
    cap = 0 if layout == "compact" else max(1, int(cnt.max()) // 2)
    rows = T * K if layout == "compact" else E * cap - 3
    note(f"dispatch one-tile boundary {payload} {layout} T={T} K={K} E={E}")
    if payload == "prequant":
        q = rng.integers(0, 256, size=(T, H), dtype=np.uint8)
        sc = (rng.random((T, H // 128)) + 0.5).astype(np.float32)
        o = moe._lib.alloc_dispatch(T, H, K, E, rows, torch.uint8, True, DEV)
        for t in (o.packed, o.scales, o.packed_src, o.tok_map, o.packed_cnt, o.packed_off, o.stats):
            poison_(t)
        moe.dispatch_prequant(dev(q), dev(sc), dev(idx), E, cap=cap, packed_rows=rows, out=o)
        torch.cuda.synchronize()
        ref = oracle.dispatch(q, "fp8", idx, E, cap=cap, packed_rows=rows, x_scales=sc)
        assert_dispatch_equal(o, ref, fp8=True)
        return
    dt = "f32" if payload == "f32" else "bf16"
    x = W.normal_x(rng, T, H, dt)
    if payload in ("fp8", "fp4"):
        x = W.inject_outliers(x, np.arange(0, T, 11), 1000.0)
    o = gpu_dispatch(dev_x(x, dt), idx, E, cap=cap, packed_rows=rows, fp8=payload == "fp8",
                     fp4=payload == "fp4")
    ref = oracle.dispatch(x, dt, idx, E, cap=cap, packed_rows=rows,
                          packed_dt=payload if payload in ("fp8", "fp4") else None)
    assert_dispatch_equal(o, ref, fp8=payload in ("fp8", "fp4"))


# ---------------------------------------------------------------------------
# edge cases of the quantized and replay entry points
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", ["T0", "rows0", "K16_E1024", "all_neg", "H128"])
@pytest.mark.parametrize("payload", ["fp8", "fp4", "prequant"])
def test_quantized_dispatch_edges(case, payload):
    rng = np.random.default_rng(6)
    T, K, E, H, rows = 40, 4, 16, 256, None
    if case == "T0":
        T = 0
    elif case == "K16_E1024":
        K, E, T = 16, 1024, 300
    elif case == "H128":
        H = 128
    idx = rng.integers(-1, E, size=(T, K)).astype(np.int32)
    if case == "all_neg":
        idx[:] = -1
    if case == "rows0":
        rows = 0
    note(f"quantized dispatch edge {case} {payload}")
    if rows is None:
        rows = T * K
    if payload == "prequant":
        q = rng.integers(0, 256, size=(T, H), dtype=np.uint8)
        sc = (rng.random((T, H // 128)) + 0.5).astype(np.float32)
        o = moe._lib.alloc_dispatch(T, H, K, E, rows, torch.uint8, True, DEV)
        for t in (o.packed, o.scales, o.packed_src, o.tok_map, o.packed_cnt, o.packed_off, o.stats):
            poison_(t)
        qd = dev(q) if T else torch.empty((0, H), dtype=torch.uint8, device=DEV)
        sd = dev(sc) if T else torch.empty((0, H // 128), dtype=torch.float32, device=DEV)
        moe.dispatch_prequant(qd, sd, dev(idx) if T else torch.empty((0, K), dtype=torch.int32, device=DEV),
                              E, packed_rows=rows, out=o)
        torch.cuda.synchronize()
        ref = oracle.dispatch(q, "fp8", idx, E, packed_rows=rows, x_scales=sc)
    else:
        x = W.normal_x(rng, T, H, "bf16")
        xd = dev_bf16(x) if T else torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
        o = gpu_dispatch(xd, idx, E, packed_rows=rows, fp8=payload == "fp8", fp4=payload == "fp4")
        ref = oracle.dispatch(x, "bf16", idx, E, packed_rows=rows, packed_dt=payload)
    assert_dispatch_equal(o, ref, fp8=True)


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_quantized_combine_and_replay_empty(fmt):
    """T = 0 and zero rows are no-ops that return OK."""
    H, K = 128, 4
    width = H // 2 if fmt == "fp4" else H
    q = torch.empty((0, width), dtype=torch.uint8, device=DEV)
    tm = torch.empty((0, K), dtype=torch.int64, device=DEV)
    w = torch.empty((0, K), dtype=torch.float32, device=DEV)
    fn = moe.combine_fp4 if fmt == "fp4" else moe.combine_fp8
    out, ow = fn(q, None, tm, w)
    x = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    moe.dispatch_replay(x, tm, torch.empty((0, width), dtype=torch.uint8, device=DEV),
                        scales=torch.empty((0, 1), dtype=torch.float32, device=DEV), fp4=fmt == "fp4")
    torch.cuda.synchronize()
    assert out.shape == (0, H) and ow.shape == (0,)



# ---------------------------------------------------------------------------
# guard rows: buffers longer than the row counts passed in; nothing past them
# is written (the row stores go through per-row buffer descriptors, so this
# checks the row indices they are given)
# ---------------------------------------------------------------------------

_GUARD = 5


def _guard_intact(t, rows, name):
    tail = host(t[rows:]).view(np.uint8)
    poison = oracle.POISON_BYTE if t.dtype != torch.int32 else None
    if poison is None:
        assert (host(t[rows:]) == oracle.POISON_I32).all(), f"{name}: guard rows written"
    else:
        assert (tail == poison).all(), f"{name}: guard rows written"


@pytest.mark.parametrize("payload", ["bf16", "f32", "fp8", "fp4", "prequant"])
@pytest.mark.parametrize("layout", ["compact_short", "padded_tight"])
def test_dispatch_guard_rows(payload, layout):
    T, H, K, E = 700, 256, 6, 16
    rng = np.random.default_rng(91)
    idx = _mixed_idx(rng, T, K, E)
    flat = idx.ravel()
    cnt = np.bincount(flat[(flat >= 0) & (flat < E)], minlength=E)
    cap = 0 if layout == "compact_short" else max(1, int(cnt.max()) // 2)
    rows = int(cnt.sum()) - 41 if cap == 0 else E * cap - 3
    quant = payload in ("fp8", "fp4", "prequant")
    x_dt = {"f32": torch.float32}.get(payload, torch.bfloat16)
    note(f"dispatch guard rows {payload} {layout} rows={rows}")
    o = moe._lib.alloc_dispatch(T, H, K, E, rows + _GUARD, torch.uint8 if quant else x_dt, quant,
                                DEV, fp4=payload == "fp4")
    for t in (o.packed, o.scales, o.packed_src, o.tok_map, o.packed_cnt, o.packed_off, o.stats):
        poison_(t)
    if payload == "prequant":
        q = rng.integers(0, 256, size=(T, H), dtype=np.uint8)
        sc = (rng.random((T, H // 128)) + 0.5).astype(np.float32)
        moe.dispatch_prequant(dev(q), dev(sc), dev(idx), E, cap=cap, packed_rows=rows, out=o)
        ref = oracle.dispatch(q, "fp8", idx, E, cap=cap, packed_rows=rows, x_scales=sc)
    else:
        dt = "f32" if payload == "f32" else "bf16"
        x = W.normal_x(rng, T, H, dt)
        moe.dispatch(dev_x(x, dt), dev(idx), E, cap=cap, packed_rows=rows, fp8=payload == "fp8",
                     fp4=payload == "fp4", out=o)
        ref = oracle.dispatch(x, dt, idx, E, cap=cap, packed_rows=rows,
                              packed_dt=payload if quant else None)
    torch.cuda.synchronize()
    view = moe._lib.DispatchOut(packed=o.packed[:rows],
                                scales=o.scales[:rows] if quant else None,
                                packed_cnt=o.packed_cnt, packed_off=o.packed_off,
                                packed_src=o.packed_src[:rows], tok_map=o.tok_map, stats=o.stats)
    assert_dispatch_equal(view, ref, fp8=quant)
    _guard_intact(o.packed, rows, "packed")
    _guard_intact(o.packed_src, rows, "packed_src")
    if quant:
        _guard_intact(o.scales, rows, "scales")


@pytest.mark.parametrize("payload", ["bf16", "fp8", "fp4", "prequant"])
def test_replay_guard_rows(payload):
    """Replay into the first `rows` rows of a longer buffer, with cached rows at
    and past the limit: those entries are skipped and the guard stays."""
    T, H, K = 400, 256, 4
    rows = T * K - 50
    rng = np.random.default_rng(92)
    tm = rng.permutation(T * K + 2 * _GUARD)[:T * K].astype(np.int64).reshape(T, K)
    tm[rng.random((T, K)) < 0.05] = -1
    tm[0, 0], tm[1, 1] = rows, rows + _GUARD + 7          # just past the limit, past the guard
    quant = payload != "bf16"
    width = H // 2 if payload == "fp4" else H
    packed = torch.empty((rows + _GUARD, width), dtype=torch.uint8 if quant else torch.bfloat16,
                         device=DEV)
    scales = torch.empty((rows + _GUARD, H // 128), dtype=torch.float32, device=DEV) if quant else None
    poison_(packed)
    if quant:
        poison_(scales)
    note(f"replay guard rows {payload} rows={rows}")
    if payload == "prequant":
        q = rng.integers(0, 256, size=(T, H), dtype=np.uint8)
        sc = (rng.random((T, H // 128)) + 0.5).astype(np.float32)
        moe.dispatch_replay(dev(q), dev(tm), packed[:rows], scales=scales[:rows], x_scales=dev(sc))
        ref = oracle.dispatch_replay(q, "fp8", tm, rows, x_scales=sc)
    else:
        x = W.normal_x(rng, T, H, "bf16")
        moe.dispatch_replay(dev_bf16(x), dev(tm), packed[:rows],
                            scales=scales[:rows] if quant else None, fp4=payload == "fp4")
        ref = oracle.dispatch_replay(x, "bf16", tm, rows, packed_dt=payload if quant else None)
    torch.cuda.synchronize()
    got = host(packed[:rows]).view(np.uint8)
    np.testing.assert_array_equal(got, ref["packed"].view(np.uint8).reshape(got.shape))
    if quant:
        np.testing.assert_array_equal(host(scales[:rows]).view(np.uint32),
                                      ref["scales"].view(np.uint32))
    _guard_intact(packed, rows, "packed")
    if quant:
        _guard_intact(scales, rows, "scales")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_dedup_guard_rows(dtype):
    T, H, K, E, R = 600, 128, 6, 32, 8
    rng = np.random.default_rng(93)
    idx = _mixed_idx(rng, T, K, E)
    x = W.normal_x(rng, T, H, dtype)
    full = oracle.dedup_dispatch(x, dtype, idx, E, R)
    recv_rows = int(full["recv_cnt"].sum()) - 23
    packed_rows = int(full["packed_cnt"].sum()) - 31
    note(f"dedup guard rows {dtype} recv_rows={recv_rows} packed_rows={packed_rows}")
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    o = moe._lib.alloc_dedup(T, H, K, E, R, recv_rows + _GUARD, packed_rows + _GUARD, tdt, DEV)
    for f in ("recv_x", "recv_cnt", "recv_off", "recv_src", "rank_slot", "packed", "packed_cnt",
              "packed_off", "packed_src", "tok_map", "stats"):
        poison_(getattr(o, f))
    moe.dedup_dispatch(dev_x(x, dtype), dev(idx), E, R, recv_rows=recv_rows,
                       packed_rows=packed_rows, out=o)
    torch.cuda.synchronize()
    ref = oracle.dedup_dispatch(x, dtype, idx, E, R, recv_rows=recv_rows, packed_rows=packed_rows)
    for f in ("recv_cnt", "recv_off", "rank_slot", "packed_cnt", "packed_off", "tok_map", "stats"):
        np.testing.assert_array_equal(host(getattr(o, f)), ref[f], err_msg=f)
    np.testing.assert_array_equal(host(o.recv_src[:recv_rows]), ref["recv_src"])
    np.testing.assert_array_equal(host(o.packed_src[:packed_rows]), ref["packed_src"])
    np.testing.assert_array_equal(host(o.recv_x[:recv_rows]).view(np.uint8),
                                  ref["recv_x"].view(np.uint8))
    np.testing.assert_array_equal(host(o.packed[:packed_rows]).view(np.uint8),
                                  ref["packed"].view(np.uint8))
    for f, n in (("recv_x", recv_rows), ("recv_src", recv_rows), ("packed", packed_rows),
                 ("packed_src", packed_rows)):
        _guard_intact(getattr(o, f), n, f)


# ---------------------------------------------------------------------------
# soak: a random T in [0, Tmax] per call on reused buffers and one workspace
# ---------------------------------------------------------------------------

def test_soak_random_T():
    """10^4 rounds of dispatch + combine, bf16 and fp8 payloads alternating, T
    drawn from [0, Tmax] each time (T = 0 included), buffers and workspace
    allocated once for Tmax.  Every round: counts, offsets and stats against
    numpy; every 10th round: slots, used rows and the combine against the oracle."""
    Tmax, H, K, E = 600, 256, 4, 24
    rng = np.random.default_rng(77)
    ws = moe.workspace(Tmax, K, E, 0, DEV)
    ob = moe._lib.alloc_dispatch(Tmax, H, K, E, Tmax * K, torch.bfloat16, False, DEV)
    oq = moe._lib.alloc_dispatch(Tmax, H, K, E, Tmax * K, torch.uint8, True, DEV)
    out = torch.empty((Tmax, H), dtype=torch.bfloat16, device=DEV)
    ow = torch.empty(Tmax, dtype=torch.float32, device=DEV)
    for r in range(10000):
        T = 0 if r % 500 == 7 else int(rng.integers(1, Tmax + 1))
        fp8 = r % 2 == 1
        idx = rng.integers(-1, E, size=(T, K)).astype(np.int32)
        x = W.normal_x(rng, T, H, "bf16")
        w = rng.random((T, K)).astype(np.float32)
        o = oq if fp8 else ob
        rows = T * K
        xd = dev_bf16(x) if T else torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
        idd = dev(idx) if T else torch.empty((0, K), dtype=torch.int32, device=DEV)
        wd = dev(w) if T else torch.empty((0, K), dtype=torch.float32, device=DEV)
        moe.dispatch(xd, idd, E, packed_rows=rows, fp8=fp8, out=o, ws=ws)
        tm = o.tok_map[:T]
        if fp8:
            moe.combine_fp8(o.packed[:rows], o.scales[:rows], tm, wd, out=out[:T], out_weights=ow[:T])
        else:
            moe.combine(o.packed[:rows], tm, wd, out=out[:T], out_weights=ow[:T])
        torch.cuda.synchronize()
        flat = idx.ravel()
        cnt = np.bincount(flat[(flat >= 0) & (flat < E)], minlength=E)
        np.testing.assert_array_equal(host(o.packed_cnt), cnt, err_msg=f"round {r} T={T}")
        np.testing.assert_array_equal(host(o.packed_off), np.concatenate([[0], np.cumsum(cnt)]))
        np.testing.assert_array_equal(host(o.stats), [int(((flat < -1) | (flat >= E)).sum()), 0, 0])
        if r % 10 or T == 0:
            continue
        ref = oracle.dispatch(x, "bf16", idx, E, packed_rows=rows, packed_dt="fp8" if fp8 else None)
        np.testing.assert_array_equal(host(tm), ref["tok_map"], err_msg=f"round {r} T={T}")
        used = np.unique(ref["tok_map"][ref["tok_map"] >= 0])
        got = host(o.packed[:rows]).view(np.uint8)[used]
        np.testing.assert_array_equal(got, ref["packed"].view(np.uint8)[used], err_msg=f"round {r}")
        if fp8:
            eo, ew = oracle.combine_fp8(ref["packed"], ref["scales"], ref["tok_map"], w, "bf16")
        else:
            eo, ew = oracle.combine(ref["packed"], "bf16", ref["tok_map"], w, "bf16")
        _check_combine(host(out[:T]), eo, "bf16")
        np.testing.assert_array_equal(host(ow[:T]).view(np.uint32), ew.view(np.uint32))


# ---------------------------------------------------------------------------
# the ABI from plain C (no Python, no torch): tests/c_abi_smoke.c, built by build()
# ---------------------------------------------------------------------------

def test_c_abi_program():
    import os
    import subprocess
    exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_smoke")
    assert os.path.exists(exe), "tests/c_abi_smoke is missing: run __graft_entry__.build()"
    note("c abi smoke program")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "c abi smoke: ok" in r.stdout, (r.returncode, r.stdout, r.stderr)
