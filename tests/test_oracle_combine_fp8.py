"""Pins of the oracle's fp8-input combine (oracle_combine_fp8) against things
other than itself: torch's float8_e4m3fn decoding with the separately pinned
bf16 combine, exact dyadic closed forms, a hand-derived case that separates the
no-intermediate-rounding reading from a bf16 dequantize, and numpy float32
arithmetic (each numpy float32 operation is one correctly rounded IEEE op)."""
import numpy as np
import pytest
import torch

import oracle


def _codes(rng, shape):
    """Random e4m3 codes without the two NaN codes (0x7F, 0xFF)."""
    q = rng.integers(0, 256, size=shape, dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38          # 1.0
    return q


def _decode(q):
    """e4m3fn codes -> float32 via torch (independent of the oracle's decoder)."""
    t = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy()


def _routing(rng, T, K, rows, p_neg=0.1):
    tm = np.stack([rng.permutation(rows)[:K] for _ in range(T)]).astype(np.int64)
    tm[rng.random((T, K)) < p_neg] = -1
    return tm


@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
def test_direct_cast_equals_bf16_combine(out_dt):
    """Every e4m3 value is a bf16 value, so with no scales the fp8 combine is the
    bf16 combine of the decoded rows (decoded by torch, not by the oracle)."""
    rng = np.random.default_rng(1)
    rows, H, T, K = 40, 256, 17, 5
    q = _codes(rng, (rows, H))
    ybits = torch.from_numpy(_decode(q)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(torch.from_numpy(ybits.view(np.int16)).view(torch.bfloat16).float().numpy(),
                          _decode(q))
    tm = _routing(rng, T, K, rows)
    w = rng.random((T, K)).astype(np.float32)
    exp, ew = oracle.combine(ybits, "bf16", tm, w, out_dt)
    got, gw = oracle.combine_fp8(q, None, tm, w, out_dt)
    assert np.array_equal(got.view(np.uint8), exp.view(np.uint8))
    assert np.array_equal(gw, ew)
    got1, _ = oracle.combine_fp8(q, np.ones((rows, H // 128), np.float32), tm, w, out_dt)
    assert np.array_equal(got1.view(np.uint8), exp.view(np.uint8))


def test_scaled_dyadic_closed_form():
    """Powers-of-two codes, scales and weights: every product and sum is exact, so
    the result is the exact sum; scales differ per row and per block, so a wrong
    row or block index changes the answer."""
    rng = np.random.default_rng(2)
    rows, H, T, K = 12, 384, 9, 4
    # codes of +-2^j for j in [-3, 3]: exponent field j+7, mantissa 0
    j = rng.integers(-3, 4, size=(rows, H))
    q = (((j + 7) << 3) | (rng.integers(0, 2, size=(rows, H)) << 7)).astype(np.uint8)
    val = np.where(q & 0x80, -1.0, 1.0) * np.exp2(j.astype(np.float64))
    sexp = rng.integers(-4, 5, size=(rows, H // 128))
    sc = np.exp2(sexp).astype(np.float32)
    tm = _routing(rng, T, K, rows, p_neg=0.2)
    w = np.exp2(rng.integers(-3, 1, size=(T, K))).astype(np.float32)
    got, gw = oracle.combine_fp8(q, sc, tm, w, "f32")
    ref = np.zeros((T, H))
    for t in range(T):
        for k in range(K):
            r = tm[t, k]
            if r >= 0:
                ref[t] += float(w[t, k]) * val[r] * np.repeat(sc[r].astype(np.float64), 128)
    assert np.array_equal(got.astype(np.float64), ref)
    assert np.array_equal(gw.astype(np.float64), np.where(tm >= 0, w.astype(np.float64), 0).sum(1))


def test_no_bf16_step_in_the_dequantize():
    """q = 1.125, s = 1 + 2^-10, w = 1: f32(q)*s = 1.125 + 1.125*2^-10 exactly in
    f32; a bf16-rounded dequantize would give 1.125."""
    code = torch.tensor([1.125]).to(torch.float8_e4m3fn).view(torch.uint8).item()
    q = np.full((1, 128), code, np.uint8)
    sc = np.array([[1.0 + 2.0 ** -10]], np.float32)
    got, _ = oracle.combine_fp8(q, sc, np.array([[0]], np.int64), np.array([[1.0]], np.float32), "f32")
    assert np.all(got == np.float32(1.125 + 1.125 * 2.0 ** -10))
    assert np.all(got != np.float32(1.125))


@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
def test_random_against_numpy_float32(out_dt):
    rng = np.random.default_rng(3)
    rows, H, T, K = 30, 512, 21, 6
    q = _codes(rng, (rows, H))
    sc = (rng.random((rows, H // 128)) * 4 + 0.25).astype(np.float32)
    tm = _routing(rng, T, K, rows)
    tm[0] = -1                              # a token with no entry: zero row, weight 0
    tm[1, 0] = rows + 5                     # out of range: skipped
    w = rng.random((T, K)).astype(np.float32)
    got, gw = oracle.combine_fp8(q, sc, tm, w, out_dt)
    dec = _decode(q)
    acc = np.zeros((T, H), np.float32)
    ws = np.zeros(T, np.float32)
    for k in range(K):
        r = tm[:, k]
        ok = (r >= 0) & (r < rows)
        rr = np.where(ok, r, 0)
        v = dec[rr] * np.repeat(sc[rr], 128, axis=1)          # float32 * float32
        p = w[:, k:k + 1] * v
        acc = np.where(ok[:, None], acc + p, acc)
        ws = np.where(ok, ws + w[:, k], ws)
    if out_dt == "bf16":
        exp = torch.from_numpy(acc).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    else:
        exp = acc
    assert np.array_equal(got.view(np.uint8), exp.view(np.uint8))
    assert np.array_equal(gw, ws)
    assert np.all(got[0] == 0) and gw[0] == 0
