"""GPU parity on non-finite and near-overflow payload values (reading
R-nonfinite): infinities, NaNs of both signs, the bf16 maximum, values near
2^127 whose product with 448 overflows f32, and blocks without any finite
value, through the fp8 and fp4 dispatch (routed in one launch and in two, and
replayed), the fp8 dequantize and every combine.

Codes and scales must equal the oracle's bit for bit (a NaN block scale is the
quiet NaN 0x7FC00000 on both sides).  Results of f32 arithmetic on NaN may
carry any NaN bit pattern, so combine and dequantize outputs are compared as
"NaN at the same elements" plus the usual bar everywhere else."""
import numpy as np
import pytest
import torch

import combine_moe_route_count_amd as moe
import oracle
import workloads as W
from _gpu_util import (DEV, assert_dispatch_equal, bf16_ulp_diff, dev, dev_bf16, gpu_dispatch,
                       host, note, poison_)

pytestmark = pytest.mark.gpu

SPECIAL = np.array([0x7F80, 0xFF80,                  # +-inf
                    0x7FC0, 0xFFC0, 0x7F81, 0xFFFF,  # NaNs of both signs, one signalling
                    0x7F7F, 0xFF7F,                  # +-bf16 maximum
                    0x7F00, 0x7EC0, 0xFE80,          # 2^127, 1.5*2^126, -2^126
                    0x0001, 0x8000], np.uint16)      # smallest subnormal, -0


def _rows(rng, T, H):
    """bf16 rows: N(0,1) with specials sprinkled in, plus whole blocks that are
    all infinite, all NaN, huge-and-tiny, or outlier-scaled."""
    x = W.normal_x(rng, T, H, "bf16")
    flat = x.reshape(-1)
    pos = rng.choice(flat.size, size=max(1, flat.size // 97), replace=False)
    flat[pos] = rng.choice(SPECIAL, size=pos.size)
    nb = H // 128
    for t in range(0, T, 5):
        b = int(rng.integers(0, nb))
        kind = t // 5 % 5
        blk = x[t, b * 128:(b + 1) * 128]
        if kind == 0:
            blk[:] = rng.choice(np.uint16([0x7F80, 0xFF80]), 128)
        elif kind == 1:
            blk[:] = rng.choice(np.uint16([0x7FC0, 0xFFC0]), 128)
        elif kind == 2:
            blk[::7] = 0x7F00                              # 2^127 next to N(0,1) values
        elif kind == 3:   # values past the bf16 range become infinities (meant)
            with np.errstate(over="ignore", invalid="ignore"):
                blk[:] = W.bf16_bits_from_f32(W.f32_from_bf16_bits(blk) * np.float32(2.0**120))
        else:
            blk[::13] = W.bf16_bits_from_f32(np.float32([3000.0]))[0]
    return x


def _nan_bf16(b):
    return (b & 0x7FFF) > 0x7F80


def _check_bf16(got, exp):
    gn, en = _nan_bf16(got), _nan_bf16(exp)
    assert np.array_equal(gn, en), f"NaN at different elements: {np.argwhere(gn != en)[:5]}"
    d = bf16_ulp_diff(np.where(gn, 0, got), np.where(en, 0, exp))
    assert d.max() <= 1, f"max {d.max()} bf16 ulps"
    return bool((d == 0).all())


def _check_f32(got, exp):
    gn, en = np.isnan(got), np.isnan(exp)
    assert np.array_equal(gn, en)
    g, e = got[~gn].astype(np.float64), exp[~en].astype(np.float64)
    same = (g == e)
    fin = np.isfinite(e) & np.isfinite(g)
    with np.errstate(invalid="ignore"):
        close = np.abs(g - e) <= 2.0**-7 * np.abs(e)
    assert np.all(same | (fin & close)), "f32 combine off"


def _idx(rng, T, K, E):
    return np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("payload", ["fp8", "fp4"])
@pytest.mark.parametrize("T,K,E,H", [(40, 4, 16, 256),        # one routing tile: one launch
                                     (1500, 4, 16, 512),      # several tiles: two launches
                                     (300, 8, 64, 7168)])     # half-row e4m3 workgroups
def test_dispatch_nonfinite(payload, T, K, E, H):
    rng = np.random.default_rng(T + K + H)
    x = _rows(rng, T, H)
    idx = _idx(rng, T, K, E)
    note(f"nonfinite dispatch {payload} T={T} K={K} E={E} H={H}")
    o = gpu_dispatch(dev_bf16(x), idx, E, fp8=payload == "fp8", fp4=payload == "fp4")
    ref = oracle.dispatch(x, "bf16", idx, E, packed_dt=payload)
    assert_dispatch_equal(o, ref, fp8=True)
    if payload == "fp4":
        assert np.isnan(ref["scales"]).any()
    # the replay along the routed map writes the same rows
    packed = torch.empty_like(o.packed)
    scales = torch.empty_like(o.scales)
    poison_(packed)
    poison_(scales)
    note(f"nonfinite replay {payload} T={T}")
    moe.dispatch_replay(dev_bf16(x), o.tok_map, packed, scales=scales, fp4=payload == "fp4")
    torch.cuda.synchronize()
    assert np.array_equal(host(packed), ref["packed"])
    assert np.array_equal(host(scales).view(np.uint32), ref["scales"].view(np.uint32))


@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
@pytest.mark.parametrize("payload", ["fp8", "fp4"])
def test_quantized_combine_and_dequant_nonfinite(payload, out_dt):
    rng = np.random.default_rng(11)
    T, K, E, H = 700, 6, 32, 1024
    x = _rows(rng, T, H)
    idx = _idx(rng, T, K, E)
    w = rng.standard_normal((T, K)).astype(np.float32)
    ref = oracle.dispatch(x, "bf16", idx, E, packed_dt=payload)
    q, sc, tm = dev(ref["packed"]), dev(ref["scales"]), dev(ref["tok_map"])
    odt = torch.float32 if out_dt == "f32" else torch.bfloat16
    note(f"nonfinite combine {payload} out={out_dt}")
    comb = moe.combine_fp8 if payload == "fp8" else moe.combine_fp4
    out, ow = comb(q, sc, tm, dev(w), out_dtype=odt)
    torch.cuda.synchronize()
    ocomb = oracle.combine_fp8 if payload == "fp8" else oracle.combine_fp4
    exp, ew = ocomb(ref["packed"], ref["scales"], ref["tok_map"], w, out_dt)
    if out_dt == "bf16":
        _check_bf16(host(out), exp)
    else:
        _check_f32(host(out), exp)
    np.testing.assert_array_equal(host(ow), ew)
    assert np.isnan(exp.astype(np.float32) if out_dt == "f32" else W.f32_from_bf16_bits(exp)).any()
    if payload == "fp8":
        note("nonfinite fp8 dequant")
        y = moe.fp8_dequant(q, sc)
        torch.cuda.synchronize()
        _check_bf16(host(y), oracle.fp8_dequant(ref["packed"], ref["scales"]))


def test_bf16_combine_nonfinite():
    rng = np.random.default_rng(12)
    rows, H, T, K = 900, 512, 300, 8
    y = _rows(rng, rows, H)
    tm = rng.integers(-1, rows, size=(T, K)).astype(np.int64)
    w = rng.standard_normal((T, K)).astype(np.float32)
    note("nonfinite bf16 combine")
    out, ow = moe.combine(dev_bf16(y), dev(tm), dev(w))
    torch.cuda.synchronize()
    exp, ew = oracle.combine(y, "bf16", tm, w, "bf16")
    _check_bf16(host(out), exp)
    np.testing.assert_array_equal(host(ow), ew)
