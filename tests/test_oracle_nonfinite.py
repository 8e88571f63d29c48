"""Pins of the oracle's handling of non-finite and near-overflow payload values
in the fp8 (e4m3) and fp4 (e2m1) block packs (reading R-nonfinite).

The expected codes below are derived by hand from the format definitions (OCP
e4m3fn: S.1111.110 = 448 is the largest finite value, S.1111.111 is NaN; OCP
e2m1: codes 0..7 are 0, 0.5, 1, 1.5, 2, 3, 4, 6) and from the page fact that
out-of-range values are clamped to the format maximum before conversion.  The
near-overflow cases are also pinned by the power-of-two homogeneity of the
block rule: scaling a block by 2^k leaves every code unchanged and scales the
block scale by exactly 2^k, which an f32 evaluation of x*448 that overflows
would break."""
import os

import numpy as np
import pytest

import oracle
import workloads as W

INF = np.float32(np.inf)
NAN = np.float32(np.nan)


def _golden(key):
    path = os.path.join(os.path.dirname(__file__), "golden", "page_facts.txt")
    for line in open(path):
        if line.startswith(key + " "):
            return line.split()[1]
    raise KeyError(key)


def _bf16(vals):
    """bf16 bit patterns of float32 values that bf16 holds exactly."""
    f = np.asarray(vals, np.float32)
    bits = W.bf16_bits_from_f32(f)
    back = W.f32_from_bf16_bits(bits)
    ok = np.isnan(f) | (back == f)
    assert ok.all(), f[~ok]
    bits[np.isnan(f)] = 0x7FC0        # a positive quiet NaN (torch's conversion sets the sign)
    return bits


def _block(head, fill=0.0, n=128):
    v = np.full(n, fill, np.float32)
    v[:len(head)] = np.asarray(head, np.float32)
    return v


NEG_NAN_BF16 = np.uint16(0xFFC0)   # bf16 NaN with the sign bit set


def test_e4m3_encoder_saturates_and_keeps_nan():
    assert _golden("fp8_out_of_range") == "clamp_to_max"
    big = np.float32([448.0, 449.0, 463.0, 464.0, 480.0, 1e6, 3.0e38, np.inf])
    assert list(oracle.e4m3_encode(big)) == [0x7E] * len(big)
    assert list(oracle.e4m3_encode(-big)) == [0xFE] * len(big)
    nans = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFBFFFFF], np.uint32).view(np.float32)
    assert list(oracle.e4m3_encode(nans)) == [0x7F, 0xFF, 0x7F, 0xFF]


def test_e2m1_encoder_saturates():
    big = np.float32([6.0, 6.5, 7.0, 1e30, np.inf])
    assert list(oracle.e2m1_encode(big)) == [7] * len(big)
    assert list(oracle.e2m1_encode(-big)) == [15] * len(big)
    assert list(oracle.e2m1_encode(np.float32([np.nan]))) == [0]


def test_fp8_block_with_infinities_and_nan_unscaled():
    # finite amax 2 <= 448: scale 1, infinities saturate, NaNs keep their sign
    bits = _bf16(_block([INF, 1.0, -2.0, NAN, 0.0, -INF], fill=0.5))
    bits[4] = NEG_NAN_BF16
    q, s = oracle.fp8_pack_rows(bits[None, :])
    assert s[0, 0] == 1.0
    # 1.0 = 1.0*2^0 -> E=7: 0x38; 2.0 -> E=8: 0x40; 0.5 -> E=6: 0x30
    assert list(q[0, :7]) == [0x7E, 0x38, 0xC0, 0x7F, 0xFF, 0xFE, 0x30]
    assert (q[0, 7:] == 0x30).all()


def test_fp8_block_with_infinities_and_nan_scaled():
    # finite amax 1000 > 448: s = 1000/448; q = 448 * x / 1000
    bits = _bf16(_block([INF, 1000.0, 500.0, NAN, -INF, -250.0]))
    q, s = oracle.fp8_pack_rows(bits[None, :])
    assert s[0, 0] == np.float32(1000.0) / np.float32(448.0)
    # 448 -> 0x7E; 224 = 1.75*2^7 -> E=14, m=6: 0x76; -112 = -1.75*2^6 -> 0xEE
    assert list(q[0, :6]) == [0x7E, 0x7E, 0x76, 0x7F, 0xFE, 0xEE]
    assert (q[0, 6:] == 0x00).all()


def test_fp8_block_without_finite_values():
    v = np.concatenate([np.full(64, INF, np.float32), np.full(64, NAN, np.float32)])
    q, s = oracle.fp8_pack_rows(_bf16(v)[None, :])
    assert s[0, 0] == 1.0
    assert (q[0, :64] == 0x7E).all() and (q[0, 64:] == 0x7F).all()


def test_fp8_block_near_the_bf16_maximum():
    # x*448 overflows f32 for |x| > 2^128/448; the quotient x*448/amax does not
    bits = _bf16(_block([2.0**127, 2.0**126, 1.5 * 2.0**126, -(2.0**120), -(2.0**-100)]))
    q, s = oracle.fp8_pack_rows(bits[None, :])
    assert s[0, 0] == np.float32(2.0**127) / np.float32(448.0)
    # 448 -> 0x7E; 224 -> 0x76; 336 lies halfway between 320 (m=2) and 352 (m=3):
    # even mantissa, 0x7A; -3.5 = -1.75*2^1 -> E=8, m=6: 0xC6; a tiny negative -> -0: 0x80
    assert list(q[0, :5]) == [0x7E, 0x76, 0x7A, 0xC6, 0x80]
    top = _bf16(_block([W.f32_from_bf16_bits(np.uint16(0x7F7F)), 1.0]))   # the bf16 maximum
    q2, _ = oracle.fp8_pack_rows(top[None, :])
    assert q2[0, 0] == 0x7E


@pytest.mark.parametrize("k", [8, 40, 90, 110, 115])
def test_fp8_and_fp4_block_rule_is_power_of_two_homogeneous(k):
    rng = np.random.default_rng(k)
    x = W.normal_x(rng, 16, 512, "bf16")
    x = W.inject_outliers(x, np.arange(0, 16, 2), 1000.0)       # scaled blocks, |x| < 2^13
    xf = W.f32_from_bf16_bits(x)
    assert np.abs(xf).max() < 2.0**13
    xs = W.bf16_bits_from_f32(xf * np.float32(2.0**k))            # exact: exponent shift only
    assert np.array_equal(W.f32_from_bf16_bits(xs), xf * np.float32(2.0**k))
    for pack, m in ((oracle.fp8_pack_rows, 448.0), (oracle.fp4_pack_rows, 6.0)):
        q0, s0 = pack(x)
        q1, s1 = pack(xs)
        blk = np.abs(xf).reshape(16, 4, 128).max(axis=2) > m
        assert blk.any()
        # blocks scaled in both packs: codes unchanged, scale times 2^k exactly
        sel = np.repeat(blk, 128 if pack is oracle.fp8_pack_rows else 64, axis=1)
        assert np.array_equal(q0[sel], q1[sel])
        assert np.array_equal(s1[blk], s0[blk] * np.float32(2.0**k))


def test_fp4_block_with_nan_is_nan_through_its_scale():
    bits = _bf16(_block([NAN, 1.0, 3.0, INF], fill=0.5))
    q, s = oracle.fp4_pack_rows(bits[None, :])
    assert s.view(np.uint32)[0, 0] == 0x7FC00000            # the canonical quiet NaN
    assert (q[0, :64] == 0).all()
    # the decode of that block (code times scale) is NaN everywhere
    dec = oracle.e2m1_decode(np.stack([q[0, :64] & 15, q[0, :64] >> 4], 1).reshape(-1))
    assert np.isnan(dec * s[0, 0]).all()


def test_fp4_block_with_infinities():
    # unscaled (finite amax 3): inf -> 6 (7), -inf -> -6 (15), 1.0 -> 2, 3.0 -> 5, 0.5 -> 1
    bits = _bf16(_block([INF, -INF, 1.0, 3.0], fill=0.5))
    q, s = oracle.fp4_pack_rows(bits[None, :])
    assert s[0, 0] == 1.0
    assert list(q[0, :2]) == [0x7 | (0xF << 4), 0x2 | (0x5 << 4)]
    assert (q[0, 2:64] == 0x11).all()
    # scaled (finite amax 12, s = 2): inf -> 7, 12 -> 6 (7), 3 -> 1.5 (3), -inf -> 15
    bits = _bf16(_block([INF, 12.0, 3.0, -INF]))
    q, s = oracle.fp4_pack_rows(bits[None, :])
    assert s[0, 0] == 2.0
    assert list(q[0, :2]) == [0x7 | (0x7 << 4), 0x3 | (0xF << 4)]
    assert (q[0, 2:64] == 0).all()
    # near the bf16 maximum: 2^127 -> 6 (7), 2^126 -> 3 (5), -2^125 -> -1.5 (0xB)
    bits = _bf16(_block([2.0**127, 2.0**126, -(2.0**125), 0.0]))
    q, s = oracle.fp4_pack_rows(bits[None, :])
    assert s[0, 0] == np.float32(2.0**127) / np.float32(6.0)
    assert list(q[0, :2]) == [0x7 | (0x5 << 4), 0xB | (0x0 << 4)]


def test_nonfinite_rows_through_dispatch_dequant_and_combine():
    """A dispatched row holding infinities and NaNs: the fp8 dequantize gives
    +-448*s at the infinities and NaN at the NaNs, and a combine of such rows
    propagates inf and NaN as f32 arithmetic does."""
    rng = np.random.default_rng(9)
    T, H, K, E = 6, 256, 2, 4
    xf = rng.standard_normal((T, H)).astype(np.float32)
    xf[0, 3], xf[1, 130], xf[2, 7] = np.inf, -np.inf, np.nan
    xf[3, 0] = 1000.0
    xf[3, 1] = np.inf
    x = W.bf16_bits_from_f32(xf)
    x[2, 7] = 0x7FC0
    idx = np.array([[0, 1], [1, 2], [2, 3], [3, 0], [0, 2], [1, 3]], np.int32)
    d = oracle.dispatch(x, "bf16", idx, E, packed_dt="fp8")
    y = W.f32_from_bf16_bits(oracle.fp8_dequant(d["packed"], d["scales"]))
    src = d["packed_src"]
    for row in range(len(src)):
        t = src[row]
        if t == 0:
            assert y[row, 3] == 448.0
        elif t == 1:
            assert y[row, 130] == -448.0
        elif t == 2:
            assert np.isnan(y[row, 7])
        elif t == 3:
            assert y[row, 1] == W.f32_from_bf16_bits(oracle.bf16_encode(
                np.float32([448.0 * (np.float32(1000.0) / np.float32(448.0))])))[0]
    w = np.full((T, K), 0.5, np.float32)
    out, ow = oracle.combine(oracle.fp8_dequant(d["packed"], d["scales"]), "bf16",
                             d["tok_map"], w, "f32")
    assert out[0, 3] == 448.0 and out[1, 130] == -448.0 and np.isnan(out[2, 7])
    assert np.isfinite(np.delete(out[2], 7)).all()


def _f32_rne_exact(q):
    """Round a Fraction to the nearest float32, ties to even, in exact rational
    arithmetic (normal and subnormal results; |q| well inside the f32 range)."""
    from fractions import Fraction
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                                   # now 2^e <= a < 2^(e+1)
    e = max(e, -126)                             # subnormals share the 2^-149 step
    ulp = Fraction(2) ** (e - 23)
    m, rem = divmod(a, ulp)
    if rem > ulp / 2 or (rem == ulp / 2 and m % 2 == 1):
        m += 1
    return np.float32(sign * float(m * ulp))     # m * ulp is exact in float32


def test_fp8_scaled_codes_against_exact_rational_quotients():
    """The scaled branch encodes the correctly rounded f32 value of the exact
    quotient x*448/amax: computed here with fractions and an exact rounding to
    float32, then torch's e4m3 encoder, for blocks whose amax ranges from just
    above 448 to the bf16 maximum (where x*448 itself exceeds the f32 range)."""
    from fractions import Fraction
    import torch
    rng = np.random.default_rng(17)
    rows = []
    for lo, hi in ((9, 12), (20, 60), (100, 120), (120, 127)):
        for _ in range(6):
            with np.errstate(over="ignore"):            # a draw past the f32 range is skipped
                f = rng.standard_normal(128).astype(np.float32)
                f *= np.float32(2.0) ** np.float32(rng.integers(lo, hi + 1))
                f[rng.integers(0, 128)] *= np.float32(-1.9)
            bits = W.bf16_bits_from_f32(f)
            v = W.f32_from_bf16_bits(bits)
            if not np.isfinite(v).all() or np.abs(v).max() <= 448:
                continue
            rows.append(bits)
    x = np.stack(rows)
    q, s = oracle.fp8_pack_rows(x)
    xf = W.f32_from_bf16_bits(x)
    for r in range(x.shape[0]):
        amax = Fraction(float(np.abs(xf[r]).max()))
        quot = np.array([_f32_rne_exact(Fraction(float(v)) * 448 / amax) for v in xf[r]], np.float32)
        ref = torch.from_numpy(quot).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(q[r], ref)
        assert s[r, 0] == _f32_rne_exact(amax / 448)
    assert (np.abs(xf).max(axis=1) > 2.0 ** 119).any()      # some blocks overflow x*448 in f32
