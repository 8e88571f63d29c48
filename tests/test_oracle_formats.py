"""Pins for the oracle's number formats and the fp8 blockwise pack.

bf16 rounding is checked against torch's float32 -> bfloat16 conversion, the
e4m3 encoder exhaustively against torch.float8_e4m3fn on every bf16 value in
range (and on random float32 values, which the scaled branch produces), the
decoder on all 256 codes, and the pack against the fixed facts of the format
page (max 448, 128-element blocks) plus error bounds any correct blockwise
quantizer meets."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _golden(key):
    path = os.path.join(os.path.dirname(__file__), "golden", "page_facts.txt")
    for line in open(path):
        if line.startswith(key + " "):
            return line.split()[1]
    raise KeyError(key)


def _torch_e4m3(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def _all_bf16_in_range():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = W.f32_from_bf16_bits(bits)
    keep = np.isfinite(v) & (np.abs(v) <= 448.0)
    return bits[keep], v[keep]


def test_bf16_encode_matches_torch():
    rng = np.random.default_rng(0)
    u = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # ties, carries into the exponent, overflow to inf, signed zeros, denormals
    extra = np.array([0x3f808000, 0x3f818000, 0x3f80ffff, 0x7f7fffff, 0xff7fffff, 0x00008000,
                      0x80018000, 0x00000000, 0x80000000, 0x7f800000, 0x3fffffff, 0x00000001],
                     np.uint32)
    u = np.concatenate([u, extra])
    v = u.view(np.float32)
    v = v[np.isfinite(v)]
    ours = oracle.bf16_encode(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_encode_exhaustive_over_bf16():
    bits, v = _all_bf16_in_range()
    assert len(v) > 30000
    np.testing.assert_array_equal(oracle.e4m3_encode(v), _torch_e4m3(v))


def test_e4m3_encode_random_f32_and_ties():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(1_000_000) * rng.choice([1e-3, 1e-1, 1, 30, 200], 1_000_000)) \
        .astype(np.float32)
    v = np.clip(v, -448, 448)
    # exact midpoints between neighbouring e4m3 values (ties go to even)
    codes = np.arange(0, 0x7e, dtype=np.uint8)
    lo = oracle.e4m3_decode(codes)
    hi = oracle.e4m3_decode(codes + 1)
    mid = ((lo.astype(np.float64) + hi) / 2).astype(np.float32)
    v = np.concatenate([v, mid, -mid, np.float32([0.0, -0.0, 448.0, -448.0, 2**-9, 2**-10,
                                                  3 * 2**-11, 2**-6 - 2**-10])])
    np.testing.assert_array_equal(oracle.e4m3_encode(v), _torch_e4m3(v))


def test_e4m3_decode_all_codes():
    b = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(b)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2
    np.testing.assert_array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_golden_e4m3_facts():
    vmax = float(_golden("e4m3_max_value"))
    code = int(_golden("e4m3_max_code"), 16)
    assert oracle.e4m3_encode(np.float32([vmax]))[0] == code
    assert oracle.e4m3_decode(np.uint8([code]))[0] == vmax
    assert np.isnan(oracle.e4m3_decode(np.uint8([code + 1]))[0])
    # the fnuz maximum is an ordinary interior value of the OCP format
    assert oracle.e4m3_decode(oracle.e4m3_encode(np.float32([240.0])))[0] == 240.0
    assert int(_golden("fp8_block_elems")) == 128


def _pack_inputs(rows=64, H=1024, seed=3):
    rng = np.random.default_rng(seed)
    x = W.normal_x(rng, rows, H, "bf16")
    x = W.inject_outliers(x, np.arange(0, rows, 5), 1000.0)
    # a few single-element spikes so amax sits at different lanes
    f = W.f32_from_bf16_bits(x)
    for r in range(1, rows, 7):
        f[r, rng.integers(0, H)] = np.float32(rng.choice([500.0, -3000.0, 449.0, 447.0]))
    return W.bf16_bits_from_f32(f)


def test_fp8_pack_scale_rule_and_values():
    x = _pack_inputs()
    q, s = oracle.fp8_pack_rows(x)
    xf = W.f32_from_bf16_bits(x)
    rows, H = x.shape
    blocks = xf.reshape(rows, H // 128, 128)
    amax = np.abs(blocks).max(axis=2)
    scaled = amax > np.float32(448.0)
    assert scaled.any() and (~scaled).any()
    # scale: amax / 448 rounded to f32 where scaled, exactly 1 elsewhere
    exp_s = np.where(scaled, (amax / np.float32(448.0)).astype(np.float32), np.float32(1.0))
    np.testing.assert_array_equal(s, exp_s)
    # values: e4m3(x) in unscaled blocks; e4m3((x*448)/amax) in scaled ones (numpy f32 math)
    num = (blocks * np.float32(448.0)).astype(np.float32)
    quo = (num / amax[:, :, None]).astype(np.float32)
    pre = np.where(scaled[:, :, None], np.clip(quo, -448, 448), blocks)
    np.testing.assert_array_equal(q.reshape(rows, H // 128, 128), _torch_e4m3(pre))
    # the block maximum lands exactly on +-448 in scaled blocks
    qs = q.reshape(rows, H // 128, 128)
    am = np.abs(blocks).argmax(axis=2)
    top = np.take_along_axis(qs, am[:, :, None], axis=2)[:, :, 0]
    assert np.all((top[scaled] & 0x7F) == 0x7E)


def test_fp8_dequant_roundtrip_error_bound():
    x = _pack_inputs(seed=4)
    q, s = oracle.fp8_pack_rows(x)
    y = oracle.fp8_dequant(q, s)
    xf = W.f32_from_bf16_bits(x).astype(np.float64)
    yf = W.f32_from_bf16_bits(y).astype(np.float64)
    rows, H = x.shape
    sf = np.repeat(s.astype(np.float64), 128, axis=1)
    # e4m3 keeps 3 mantissa bits: relative half-ulp 2^-4 for normals, absolute 2^-10
    # below 2^-6 (times the scale); the bf16 store adds at most a 2^-8 relative rounding
    v = np.abs(xf) / sf
    bound = np.maximum(v * 2.0**-4, 2.0**-10) * sf * (1 + 2**-7) + np.abs(xf) * 2.0**-8
    assert np.all(np.abs(yf - xf) <= bound + 1e-30)


def test_fp8_dequant_matches_torch_arithmetic():
    rng = np.random.default_rng(5)
    q = rng.integers(0, 256, size=(8, 256), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x11        # no NaN codes
    s = (rng.random((8, 2)) * 4 + 0.25).astype(np.float32)
    y = oracle.fp8_dequant(q, s)
    vt = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float32)
    st = torch.from_numpy(np.repeat(s, 128, axis=1))
    ref = (vt * st).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(y, ref)


def test_fp8_dispatch_rows_equal_pack_of_source():
    d = W.make_inputs("skewed_fp8", T=64)
    x = W.inject_outliers(d["x"], np.array([3, 10]), 1000.0)
    r = oracle.dispatch(x, "bf16", d["idx"], d["E"], packed_dt="fp8")
    q, s = oracle.fp8_pack_rows(x)
    src = r["packed_src"]
    np.testing.assert_array_equal(r["packed"], q[src])
    np.testing.assert_array_equal(r["scales"], s[src])
