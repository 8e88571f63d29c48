"""GPU parity over a seeded sweep of the whole argument space: every payload
(bf16, f32, e4m3 pack, e2m1 pack, pre-quantized e4m3), every layout (compact,
padded, padded below the largest count, compact with too few rows), expert
counts on both sides of the one-launch routing limit (512), token counts from
empty through one routing tile to several, K from 1 to 16 and odd row widths.

Each case runs the routed dispatch against the oracle (bit-exact), the replay
of its tok_map against the routed rows (bit-exact), and the combine of the
dispatched rows (identity experts) against the oracle (within one bf16 ulp,
out_weights exact).  A second sweep does the same for the dedup dispatch and
both dedup combine forms.  The cases are drawn once, at import, from a fixed
seed, so a failure names a case that reruns as it failed."""
import os

import numpy as np
import pytest
import torch

import combine_moe_route_count_amd as moe
import oracle
import workloads as W
from _gpu_util import (DEV, assert_dispatch_equal, bf16_ulp_diff, dev, dev_x, host, note,
                       poison_)

pytestmark = pytest.mark.gpu

# MOE_SWEEP_CASES / MOE_SWEEP_SEED widen the sweep for a longer run (the
# defaults are what the suite runs)
N_CASES = int(os.environ.get("MOE_SWEEP_CASES", 160))
N_DEDUP_CASES = max(1, N_CASES * 3 // 10)
SEED = int(os.environ.get("MOE_SWEEP_SEED", 20261203))
MAX_ELEMS = 12_000_000          # T*K*H bound: every case's oracle runs in well under a second
QUANT = ("fp8", "fp4", "prequant")


def _draw_cases():
    rng = np.random.default_rng(SEED)
    cases = []
    for i in range(N_CASES):
        payload = str(rng.choice(["bf16", "f32", "fp8", "fp4", "prequant"]))
        layout = str(rng.choice(["compact", "padded", "padded_tight", "compact_short"]))
        E = int(rng.choice([1, 2, 7, 8, 64, 255, 256, 511, 512, 513, 777, 1024]))
        K = int(rng.integers(1, 17))
        size = str(rng.choice(["tiny", "one_tile", "multi"]))
        if size == "tiny":
            T = int(rng.integers(0, 9))
        elif size == "one_tile":   # T*K within a few entries of one routing tile (1024)
            T = int(rng.integers(max(1, 1024 // K - 3), 1024 // K + 4))
        else:
            T = int(rng.integers(1024 // K + 2, 6000))
        if payload in QUANT:
            H = 128 * int(rng.integers(1, 60))
        else:
            H = 8 * int(rng.integers(1, 1000))
        step = 128 if payload in QUANT else 8
        while T * K * H > MAX_ELEMS and H > step:
            H = max(step, (H // 2) // step * step)
        cases.append(dict(i=i, payload=payload, layout=layout, T=T, K=K, E=E, H=H,
                          direct=bool(rng.random() < 0.3), out_dt=str(rng.choice(["bf16", "f32"]))))
    return cases


def _draw_dedup_cases():
    rng = np.random.default_rng(SEED + 1)
    cases = []
    for i in range(N_DEDUP_CASES):
        R = int(rng.choice([1, 2, 4, 8, 16, 32]))
        E = R * int(rng.choice([1, 2, 3, 8, 16]))
        K = int(rng.integers(1, 17))
        T = int(rng.choice([0, 1, int(rng.integers(2, 200)), int(rng.integers(200, 3000))]))
        H = 8 * int(rng.integers(1, 700))
        while T * K * H > MAX_ELEMS and H > 8:
            H = max(8, (H // 2) // 8 * 8)
        cases.append(dict(i=i, R=R, E=E, K=K, T=T, H=H, dt=str(rng.choice(["bf16", "f32"])),
                          recv_drop=bool(rng.random() < 0.3), padded=bool(rng.random() < 0.3)))
    return cases


CASES = _draw_cases()
DEDUP_CASES = _draw_dedup_cases()


def _case_id(c):
    return "-".join(f"{k}{v}" for k, v in c.items())


def _idx(rng, T, K, E):
    """K distinct experts per token where K <= E (else with repeats); about 5%
    -1 sentinels and 2% ids outside [0, E)."""
    if T == 0:
        return np.zeros((0, K), np.int32)
    if K <= E:
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    else:
        idx = rng.integers(0, E, size=(T, K)).astype(np.int32)
    u = rng.random((T, K))
    idx[u < 0.05] = -1
    bad = u > 0.98
    idx[bad] = rng.choice(np.array([E, E + 5, -2, -1000], np.int64), size=int(bad.sum())).astype(np.int32)
    return idx


def _layout(layout, idx, E, T, K):
    flat = idx.ravel()
    cnt = np.bincount(flat[(flat >= 0) & (flat < E)], minlength=E)
    top = int(cnt.max()) if cnt.size else 0
    if layout == "compact":
        return 0, T * K
    if layout == "padded":
        cap = max(1, top)
        return cap, E * cap
    if layout == "padded_tight":
        cap = max(1, top // 2)
        return cap, max(0, E * cap - 3)
    return 0, max(0, int(cnt.sum()) - 37)


def _check_out(got, exp, out_dt):
    if out_dt == "bf16":
        d = bf16_ulp_diff(got, exp)
        assert d.size == 0 or d.max() <= 1, f"max {d.max()} bf16 ulps"
    else:
        g, e = got.astype(np.float64), exp.astype(np.float64)
        assert np.all(np.abs(g - e) <= 2.0**-7 * np.abs(e)), "f32 combine off by more than 2^-7"


@pytest.mark.parametrize("c", CASES, ids=_case_id)
def test_sweep_dispatch_replay_combine(c):
    T, K, E, H, payload = c["T"], c["K"], c["E"], c["H"], c["payload"]
    rng = np.random.default_rng(SEED + 1000 + c["i"])
    idx = _idx(rng, T, K, E)
    cap, rows = _layout(c["layout"], idx, E, T, K)
    w = rng.standard_normal((T, K)).astype(np.float32)
    quant = payload in QUANT
    x_dt = "f32" if payload == "f32" else "bf16"
    if payload == "prequant":
        x = rng.integers(0, 256, size=(T, H), dtype=np.uint8)
        xs = (rng.random((T, H // 128)) * 4 + 2.0**-8).astype(np.float32)
    else:
        x = W.normal_x(rng, T, H, x_dt)
        if quant and T > 0:
            x = W.inject_outliers(x, np.arange(0, T, 11), 1000.0)
        xs = None
    note(f"sweep {_case_id(c)} cap={cap} rows={rows}")

    # routed dispatch
    fp4 = payload == "fp4"
    o = moe._lib.alloc_dispatch(T, H, K, E, rows, torch.uint8 if payload == "prequant" else
                                (torch.float32 if x_dt == "f32" else torch.bfloat16),
                                quant, DEV, fp4=fp4)
    for t in (o.packed, o.scales, o.packed_src, o.tok_map, o.packed_cnt, o.packed_off, o.stats):
        poison_(t)
    idx_d = dev(idx)
    if payload == "prequant":
        x_d, xs_d = dev(x), dev(xs)
        moe.dispatch_prequant(x_d, xs_d, idx_d, E, cap=cap, packed_rows=rows, out=o)
        ref = oracle.dispatch(x, "fp8", idx, E, cap=cap, packed_rows=rows, x_scales=xs)
    else:
        x_d, xs_d = dev_x(x, x_dt), None
        moe.dispatch(x_d, idx_d, E, cap=cap, packed_rows=rows, fp8=payload == "fp8", fp4=fp4,
                     out=o)
        ref = oracle.dispatch(x, x_dt, idx, E, cap=cap, packed_rows=rows,
                              packed_dt=payload if quant else None)
    torch.cuda.synchronize()
    assert_dispatch_equal(o, ref, fp8=quant)

    # replay of the routed map: the same rows, bit for bit (untouched rows keep the poison)
    rp = torch.empty_like(o.packed)
    rs = torch.empty_like(o.scales) if o.scales is not None else None
    poison_(rp)
    poison_(rs)
    moe.dispatch_replay(x_d, o.tok_map, rp, scales=rs, x_scales=xs_d, fp4=fp4)
    torch.cuda.synchronize()
    assert torch.equal(rp.view(torch.uint8), o.packed.view(torch.uint8)), "replay rows"
    if rs is not None:
        assert torch.equal(rs.view(torch.int32), o.scales.view(torch.int32)), "replay scales"

    # combine of the dispatched rows
    odt = torch.float32 if c["out_dt"] == "f32" else torch.bfloat16
    w_d = dev(w)
    if payload in ("bf16", "f32"):
        out, ow = moe.combine(o.packed, o.tok_map, w_d, out_dtype=odt)
        eo, ew = oracle.combine(ref["packed"], x_dt, ref["tok_map"], w, c["out_dt"])
    else:
        sc = None if c["direct"] else o.scales
        esc = None if c["direct"] else ref["scales"]
        comb, ocomb = (moe.combine_fp4, oracle.combine_fp4) if fp4 else \
            (moe.combine_fp8, oracle.combine_fp8)
        out, ow = comb(o.packed, sc, o.tok_map, w_d, out_dtype=odt)
        eo, ew = ocomb(ref["packed"], esc, ref["tok_map"], w, c["out_dt"])
    torch.cuda.synchronize()
    got = host(out)
    # NaN-free by construction except where e4m3 codes are NaN patterns (pre-quantized input)
    nan = np.isnan(eo.astype(np.float32)) if c["out_dt"] == "f32" else \
        ((eo & 0x7FFF) > 0x7F80)
    if c["out_dt"] == "f32":
        assert np.array_equal(np.isnan(got), nan), "NaN positions"
    else:
        assert np.array_equal((got & 0x7FFF) > 0x7F80, nan), "NaN positions"
    _check_out(np.where(nan, 0, got), np.where(nan, 0, eo), c["out_dt"])
    np.testing.assert_array_equal(host(ow), ew)


@pytest.mark.parametrize("c", DEDUP_CASES, ids=_case_id)
def test_sweep_dedup(c):
    T, K, E, R, H, dt = c["T"], c["K"], c["E"], c["R"], c["H"], c["dt"]
    rng = np.random.default_rng(SEED + 500000 + c["i"])
    idx = _idx(rng, T, K, E)
    x = W.normal_x(rng, T, H, dt)
    w = rng.random((T, K)).astype(np.float32)
    full = oracle.dedup_dispatch(x, dt, idx, E, R)
    n_recv = int(full["recv_off"][R])
    recv_rows = max(0, n_recv - 1 - n_recv // 5) if c["recv_drop"] else T * min(K, R)
    cap = max(1, int(full["packed_cnt"].max()) - 2) if c["padded"] else 0
    rows = E * cap if cap > 0 else T * K
    note(f"sweep dedup {_case_id(c)} recv_rows={recv_rows} cap={cap}")
    o = moe._lib.alloc_dedup(T, H, K, E, R, recv_rows, rows,
                             torch.float32 if dt == "f32" else torch.bfloat16, DEV)
    for f in ("recv_x", "recv_cnt", "recv_off", "recv_src", "rank_slot", "packed", "packed_cnt",
              "packed_off", "packed_src", "tok_map", "stats"):
        poison_(getattr(o, f))
    idx_d = dev(idx)
    moe.dedup_dispatch(dev_x(x, dt), idx_d, E, R, recv_rows=recv_rows, cap=cap, out=o)
    torch.cuda.synchronize()
    ref = oracle.dedup_dispatch(x, dt, idx, E, R, recv_rows=recv_rows, cap=cap)
    for f in ("recv_cnt", "recv_off", "recv_src", "rank_slot", "packed_cnt", "packed_off",
              "packed_src", "tok_map", "stats"):
        np.testing.assert_array_equal(host(getattr(o, f)), ref[f], err_msg=f)
    for f in ("recv_x", "packed"):
        assert np.array_equal(host(getattr(o, f)).view(np.uint8), ref[f].view(np.uint8)), f
    eo, ew, ep = oracle.dedup_combine(ref["packed"], dt, ref["tok_map"], w, idx, E, R,
                                      ref["rank_slot"], recv_rows, "f32", want_partial=True)
    for with_partial in (True, False):
        part = torch.empty((recv_rows, H), dtype=torch.float32, device=DEV) if with_partial else None
        poison_(part)
        plan = dict(R=R, idx=idx_d, rank_slot=o.rank_slot, recv_rows=recv_rows, partial=part)
        out, ow = moe.combine(o.packed, o.tok_map, dev(w), E=E, out_dtype=torch.float32, dedup=plan)
        torch.cuda.synchronize()
        _check_out(host(out), eo, "f32")
        np.testing.assert_array_equal(host(ow), ew)
        if with_partial:
            n = min(n_recv, recv_rows)
            np.testing.assert_array_equal(host(part)[:n].view(np.uint32), ep[:n].view(np.uint32))
