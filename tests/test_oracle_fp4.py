"""Pins of the oracle's fp4 (OCP e2m1) payload: the codec against a brute-force
nearest-value search over the format's eight magnitudes, the row pack against
numpy float32 arithmetic with that search, the fp4 combine against the pinned
bf16 combine and an exact dyadic closed form, and the fp4 dispatch against the
routing of the bf16 dispatch."""
import numpy as np
import pytest

import oracle
import workloads as W

# OCP MX e2m1 magnitudes, codes 0..7 (the format's definition: bias 1, one mantissa bit)
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def brute_e2m1(v):
    """Nearest of the eight magnitudes, ties to the even code, saturating at 6,
    sign kept (also for zero results)."""
    v = np.asarray(v, np.float32).astype(np.float64)
    a = np.abs(v)
    d = np.abs(a[:, None] - E2M1[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = np.where(d == best, np.arange(8)[None, :], 99)
    even = np.where(cand % 2 == 0, cand, 99).min(axis=1)
    code = np.where(even < 99, even, cand.min(axis=1))
    code = np.where(a > 6.0, 7, code)
    return (code | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def test_e2m1_decode_table_and_round_trip():
    codes = np.arange(16, dtype=np.uint8)
    dec = oracle.e2m1_decode(codes)
    assert np.array_equal(dec[:8], E2M1) and np.array_equal(dec[8:], -E2M1)
    assert np.array_equal(oracle.e2m1_encode(dec), codes)


def test_e2m1_encoder_against_brute_force():
    pos = np.arange(0, 0x4181, dtype=np.uint32)                 # every bf16 with |v| <= 16
    bits = np.concatenate([pos, pos | 0x8000]) << 16
    v = bits.astype(np.uint32).view(np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    near = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 100)])
    rng = np.random.default_rng(0)
    rnd = (rng.standard_normal(200000) * 3).astype(np.float32)
    for x in (v, near, -near, rnd):
        assert np.array_equal(oracle.e2m1_encode(x), brute_e2m1(x))


def _pack_ref(x_bits):
    """numpy float32 statement of the block rule with the brute-force encoder."""
    x = W.f32_from_bf16_bits(x_bits)
    rows, H = x.shape
    xb = x.reshape(rows, H // 128, 128)
    amax = np.abs(xb).max(axis=2)
    scaled = amax > np.float32(6.0)
    s = np.where(scaled, amax / np.float32(6.0), np.float32(1.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        qv = np.where(scaled[:, :, None],
                      np.clip((xb * np.float32(6.0)) / amax[:, :, None], -6, 6), xb).astype(np.float32)
    codes = brute_e2m1(qv.reshape(-1)).reshape(rows, H)
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return q, s


def test_fp4_pack_rows_against_numpy():
    rng = np.random.default_rng(1)
    x = W.inject_outliers(W.normal_x(rng, 64, 512, "bf16"), np.arange(0, 64, 5), 1000.0)
    q, s = oracle.fp4_pack_rows(x)
    qr, sr = _pack_ref(x)
    assert np.array_equal(q, qr)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    assert (s > 1).any() and (s == 1).any()
    # the element that sets a scaled block's amax lands on +-6
    dec = oracle.e2m1_decode(np.stack([q & 15, q >> 4], axis=2).reshape(64, 512))
    xf = W.f32_from_bf16_bits(x).reshape(64, 4, 128)
    for r, b in zip(*np.nonzero(s > 1)):
        h = np.abs(xf[r, b]).argmax()
        assert abs(dec[r, b * 128 + h]) == 6.0


def _golden():
    facts = {}
    for line in open(__file__.rsplit("/", 1)[0] + "/golden/page_facts.txt"):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            facts[k] = v
    return facts


def test_fp4_row_bytes_match_the_page():
    """The page's fp4 accumulator path packs 8 codes per i32: hidden/2 bytes and
    hidden/8 dwords per row."""
    g = _golden()
    H = 7168
    q, s = oracle.fp4_pack_rows(np.zeros((1, H), np.uint16))
    assert q.nbytes == H // int(g["fp4_codes_per_byte_inverse"]) == H // 2
    assert q.nbytes // 4 == H // int(g["fp4_codes_per_i32"])


def test_fp4_nibble_order():
    x = np.zeros((1, 128), np.float32)
    x[0, 0], x[0, 1] = 1.0, -4.0                    # codes 2 and 14
    q, s = oracle.fp4_pack_rows(W.bf16_bits_from_f32(x))
    assert q[0, 0] == (2 | (14 << 4)) and s[0, 0] == 1.0


@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
def test_combine_fp4_direct_cast_equals_bf16_combine(out_dt):
    rng = np.random.default_rng(2)
    rows, H, T, K = 30, 256, 19, 4
    q = rng.integers(0, 256, size=(rows, H // 2), dtype=np.uint8)
    codes = np.stack([q & 15, q >> 4], axis=2).reshape(rows, H)
    y = np.where(codes & 8, -1.0, 1.0) * E2M1[codes & 7]               # decoded by the table
    ybits = W.bf16_bits_from_f32(y.astype(np.float32))
    tm = np.stack([rng.permutation(rows)[:K] for _ in range(T)]).astype(np.int64)
    tm[rng.random((T, K)) < 0.1] = -1
    w = rng.random((T, K)).astype(np.float32)
    exp, ew = oracle.combine(ybits, "bf16", tm, w, out_dt)
    got, gw = oracle.combine_fp4(q, None, tm, w, out_dt)
    assert np.array_equal(got.view(np.uint8), exp.view(np.uint8))
    assert np.array_equal(gw, ew)


def test_combine_fp4_scaled_dyadic():
    rng = np.random.default_rng(3)
    rows, H, T, K = 10, 384, 8, 3
    q = rng.integers(0, 256, size=(rows, H // 2), dtype=np.uint8)
    codes = np.stack([q & 15, q >> 4], axis=2).reshape(rows, H)
    val = np.where(codes & 8, -1.0, 1.0) * E2M1[codes & 7]
    sc = np.exp2(rng.integers(-3, 4, size=(rows, H // 128))).astype(np.float32)
    tm = np.stack([rng.permutation(rows)[:K] for _ in range(T)]).astype(np.int64)
    w = np.exp2(rng.integers(-2, 1, size=(T, K))).astype(np.float32)
    got, _ = oracle.combine_fp4(q, sc, tm, w, "f32")
    ref = np.zeros((T, H))
    for t in range(T):
        for k in range(K):
            r = tm[t, k]
            ref[t] += float(w[t, k]) * val[r] * np.repeat(sc[r].astype(np.float64), 128)
    assert np.array_equal(got.astype(np.float64), ref)


def test_fp4_dispatch_rows_and_routing():
    rng = np.random.default_rng(4)
    T, H, K, E = 70, 256, 4, 9
    x = W.inject_outliers(W.normal_x(rng, T, H, "bf16"), np.arange(0, T, 9), 1000.0)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    idx[rng.random((T, K)) < 0.1] = -1
    d = oracle.dispatch(x, "bf16", idx, E, packed_dt="fp4")
    ref = oracle.dispatch(x, "bf16", idx, E)
    for key in ("tok_map", "packed_cnt", "packed_off", "packed_src", "stats"):
        assert np.array_equal(d[key], ref[key]), key
    q, s = _pack_ref(x)
    for row, t in enumerate(d["packed_src"]):
        if t == oracle.POISON_I32:                  # a row no entry took
            assert np.all(d["packed"][row] == oracle.POISON_BYTE)
            continue
        assert np.array_equal(d["packed"][row], q[t])
        assert np.array_equal(d["scales"][row].view(np.uint32), s[t].view(np.uint32))
    rp = oracle.dispatch_replay(x, "bf16", d["tok_map"], d["packed"].shape[0], packed_dt="fp4")
    assert np.array_equal(rp["packed"], d["packed"])
