"""Host-side logic of bench.py, on the CPU: the one-GPU refusal, the
algorithmic byte counts the roofline and GB/s figures divide by, the counter
scaling behind the `traffic` field, the kernel-name shortening of the profile
summaries, and that the committed combine profile belongs to the current
combine sources."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr
    assert r.stdout.strip() == "" or not r.stdout.strip().startswith("{")   # no JSON line


def test_headline_algorithmic_bytes(bench):
    """T=8192 H=7168 E=256 K=8, fp8 payload, bf16 expert outputs and output:
    every byte the method must move, each term from the definition."""
    T, H, E, K = 8192, 7168, 256, 8
    N = T * K
    x_read = T * H * 2                       # bf16 token rows, read once
    rows = N * H                             # one e4m3 byte per element per entry
    scales = N * (H // 128) * 4              # one f32 per 128-element block
    idx = N * 4
    tok_map = N * 8
    packed_src = N * 4
    counts = 2 * E * 4                       # packed_cnt and packed_off
    disp = x_read + rows + scales + idx + tok_map + packed_src + counts
    y = N * H * 2                            # bf16 expert outputs gathered once
    out = T * H * 2
    comb = y + out + tok_map + N * 4 + T * 4   # + weights + out_weights
    assert bench.algorithmic_bytes(T, H, K, E, N, fp8=True) == (disp, comb)
    assert comb == 1_057_783_808
    assert disp == 602_933_248


def test_quantized_combine_and_fp4_bytes(bench):
    T, H, E, K = 8192, 7168, 256, 8
    N = T * K
    d8, c8 = bench.algorithmic_bytes(T, H, K, E, N, fp8=True, y_fp8=True)
    d4, c4 = bench.algorithmic_bytes(T, H, K, E, N, fp8=True, y_fp8=True, fp4=True)
    assert c8 - c4 == N * H // 2              # e2m1 rows: half the e4m3 bytes
    assert d8 - d4 == N * H // 2
    assert c8 == N * H + N * (H // 128) * 4 + T * H * 2 + N * 8 + N * 4 + T * 4


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_pmc_summary_scales_by_the_calibration_copy(bench, tmp_path):
    comb = "void moe::(anonymous namespace)::combine_kernel<false, false, 8>(moe::CombineArgs, int, int)"
    copy = "void moe::(anonymous namespace)::copy16_kernel(char const*, char*, long)"
    other = "void moe::(anonymous namespace)::scatter_fp8_kernel<8, 2, false, false>(moe::ScatterArgs, int, int, int)"
    f, w, cf, cw, out = (str(tmp_path / n) for n in ("f.csv", "w.csv", "cf.csv", "cw.csv", "o.json"))
    # counters in KiB per dispatch: the copy moves 1 GiB each way
    _write_csv(f, [{"Kernel_Name": comb, "Counter_Value": 1000.0}, {"Kernel_Name": other, "Counter_Value": 9e9},
                   {"Kernel_Name": comb, "Counter_Value": 3000.0}])
    _write_csv(w, [{"Kernel_Name": comb, "Counter_Value": 500.0}])
    _write_csv(cf, [{"Kernel_Name": copy, "Counter_Value": 524288.0}, {"Kernel_Name": copy, "Counter_Value": 0.0}])
    _write_csv(cw, [{"Kernel_Name": copy, "Counter_Value": 1048576.0}])
    bench.pmc_summary(f, w, cf, cw, out, trace_avg_us=170.0)
    d = json.load(open(out))
    assert d["fetch_bytes_per_unit"] == 2048.0 and d["write_bytes_per_unit"] == 1024.0
    assert d["fetch_bytes_per_launch"] == 2000.0 * 2048
    assert d["write_bytes_per_launch"] == 500.0 * 1024
    assert d["traffic_bytes_per_launch"] == 2000.0 * 2048 + 500.0 * 1024
    assert d["trace_avg_us"] == 170.0 and d["dispatches"] == [2, 1]


@pytest.mark.parametrize("raw,short", [
    ("void moe::(anonymous namespace)::combine_kernel<false, false, 8>(moe::CombineArgs, int, int)",
     "combine_kernel<false, false, 8>"),
    ("void moe::(anonymous namespace)::route_fused_kernel<moe::ExpertKeys>(moe::ExpertKeys, moe::RouteFusedArgs)",
     "route_fused_kernel<ExpertKeys>"),
    ("void moe::(anonymous namespace)::dedup_combine_kernel<true, true, 6, 1>(moe::CombineArgs, int, int)",
     "dedup_combine_kernel<true, true, 6, 1>"),
])
def test_kernel_names_in_summaries(bench, raw, short):
    assert bench._short_kernel(raw) == short


def test_committed_combine_profile_matches_the_sources(bench):
    """The counter and trace figures the bench line quotes were taken on the
    combine kernel as it stands; a change to its sources asks for new runs."""
    d = bench.stored_profile(bench.source_hash(bench.COMBINE_SOURCES))
    assert d, "profiles/combine_skewed_fp8_pmc.json is missing or was taken on other combine sources"
    _, comb = bench.algorithmic_bytes(8192, 7168, 8, 256, 8192 * 8, fp8=True)
    assert 1.0 <= d["traffic_bytes_per_launch"] / comb < 1.02
    assert 150 < d["trace_avg_us"] < 200
    trace = open(os.path.join(ROOT, "profiles", "skewed_fp8_headline_kernel_trace.txt")).read()
    line = next(l for l in trace.splitlines() if l.startswith(bench.HEADLINE_COMBINE))
    assert abs(float(line.split()[-4]) - d["trace_avg_us"]) < 0.01
