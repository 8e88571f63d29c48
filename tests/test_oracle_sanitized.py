"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(float-cast-overflow included; host code only) runs every entry point on small
inputs, edge cases and non-finite payloads included, in a child process: no
out-of-bounds access, no undefined arithmetic, no out-of-range float-to-integer
conversion."""
import os
import subprocess
import sys
import textwrap

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

SCRIPT = textwrap.dedent("""
    import sys
    import numpy as np
    sys.path.insert(0, {root!r})
    import oracle
    rng = np.random.default_rng(5)

    def bf16(a):
        return oracle.bf16_encode(a.astype(np.float32))

    for T, H, K, E, cap, rows in [(0, 128, 2, 4, 0, None), (1, 128, 1, 1, 0, None),
                                  (37, 256, 4, 9, 0, None), (50, 128, 3, 5, 4, None),
                                  (64, 128, 8, 16, 0, 100)]:
        idx = rng.integers(-2, E + 2, size=(T, K)).astype(np.int32)
        x = bf16(rng.standard_normal((T, H)) * 300)
        xf = rng.standard_normal((T, H)).astype(np.float32)
        w = rng.random((T, K)).astype(np.float32)
        oracle.route_count(idx, E)
        for pdt in (None, "fp8", "fp4"):
            d = oracle.dispatch(x, "bf16", idx, E, cap=cap, packed_rows=rows, packed_dt=pdt)
            tm = d["tok_map"]
            if pdt is None:
                oracle.combine(d["packed"], "bf16", tm, w, "bf16")
                oracle.dispatch_replay(x, "bf16", tm, d["packed"].shape[0])
            elif pdt == "fp8":
                oracle.combine_fp8(d["packed"], d["scales"], tm, w, "f32")
                oracle.combine_fp8(d["packed"], None, tm, w, "bf16")
                oracle.fp8_dequant(d["packed"], d["scales"])
                q, s = oracle.fp8_pack_rows(x)
                oracle.dispatch(q, "fp8", idx, E, cap=cap, packed_rows=rows, x_scales=s)
                oracle.dispatch_replay(q, "fp8", tm, d["packed"].shape[0], x_scales=s)
            else:
                oracle.combine_fp4(d["packed"], d["scales"], tm, w, "bf16")
                oracle.dispatch_replay(x, "bf16", tm, d["packed"].shape[0], packed_dt="fp4")
        d = oracle.dispatch(xf, "f32", idx, E, cap=cap, packed_rows=rows)
        oracle.combine(d["packed"], "f32", d["tok_map"], w, "f32")
        if E % 4 == 0 and T > 0:
            R = 4
            dd = oracle.dedup_dispatch(xf, "f32", idx, E, R)
            rr = int(dd["recv_cnt"].sum())
            oracle.dedup_combine(dd["packed"], "f32", dd["tok_map"], w, idx, E, R,
                                 dd["rank_slot"], rr, "f32", want_partial=True)
            oracle.dedup_dispatch(x, "bf16", idx, E, R, recv_rows=max(0, rr - 3))
    v = rng.standard_normal(4096).astype(np.float32) * 10
    oracle.e4m3_decode(oracle.e4m3_encode(v))
    # non-finite and near-overflow payloads through every pack and combine
    special = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x7F7F, 0xFF7F, 0x7F00, 0x0001, 0x8000],
                       np.uint16)
    xs = bf16(rng.standard_normal((6, 256)))
    xs.reshape(-1)[rng.integers(0, xs.size, 40)] = rng.choice(special, 40)
    xs[5, :128] = 0x7FC0
    idx = rng.integers(0, 4, size=(6, 2)).astype(np.int32)
    w = rng.random((6, 2)).astype(np.float32)
    for pdt in ("fp8", "fp4"):
        d = oracle.dispatch(xs, "bf16", idx, 4, packed_dt=pdt)
        comb = oracle.combine_fp8 if pdt == "fp8" else oracle.combine_fp4
        comb(d["packed"], d["scales"], d["tok_map"], w, "bf16")
    q, s = oracle.fp8_pack_rows(xs)
    oracle.combine(oracle.fp8_dequant(q, s), "bf16", np.arange(12).reshape(6, 2) % 6, w, "bf16")
    oracle.e4m3_encode(np.float32([np.inf, -np.inf, np.nan, 3e38, -1e30]))
    oracle.e2m1_encode(np.float32([np.inf, -np.inf, np.nan, 3e38, -1e30]))
    oracle.bf16_encode(np.float32([np.inf, -np.inf, np.nan, 3.4e38]))
    oracle.e2m1_decode(oracle.e2m1_encode(np.clip(v, -6, 6)))
    oracle.fp4_pack_rows(bf16(rng.standard_normal((3, 256))))
    print("sanitized oracle: ok")
""")


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_under_asan_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=gnu99", "-ffp-contract=off", "-fno-fast-math",
                    "-fopenmp", "-fsanitize=address,undefined,float-cast-overflow",
                    "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-shared", "-fPIC", "-o", str(lib),
                    os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm"], check=True)
    env = dict(os.environ, MOE_ORACLE_LIB=str(lib), LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", SCRIPT.format(root=ROOT)], env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "sanitized oracle: ok" in r.stdout, r.stderr[-4000:]
