"""Launch geometry decides how work is split, never what is computed: the same
calls under the default geometry and under two MOE_GEOM overrides at the ends
of the accepted ranges (1 to 8 workgroups per row, 64 to 256 lane units per
combine workgroup, no cap to 16 workgroups per CU) give the same bytes in every
output.  Each geometry runs in a child process of its own (the variable is read
once per process), one after the other."""
import json
import os
import subprocess
import sys

import pytest

from _gpu_util import note

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import hashlib, json, sys
sys.path.insert(0, ROOT)
import numpy as np
import torch
import combine_moe_route_count_amd as moe
import workloads as W

def h(*ts):
    d = hashlib.sha256()
    for t in ts:
        if t is not None:
            d.update(t.detach().cpu().contiguous().view(torch.uint8).numpy().tobytes())
    return d.hexdigest()[:16]

dev = torch.device("cuda:0")
out = {"geometry": moe.geometry()}
rng = np.random.default_rng(1234)

def idx_of(T, K, E):
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    idx[rng.random((T, K)) < 0.04] = -1
    return torch.from_numpy(idx).to(dev)

# bf16 and f32 copies (compact and padded), combine to bf16 and f32
for dt, T, H, K, E, cap in [("bf16", 2000, 2048, 8, 64, 0), ("f32", 1500, 1024, 4, 32, 300),
                            ("bf16", 700, 7168, 8, 256, 40)]:
    xs = W.normal_x(rng, T, H, dt)
    x = (torch.from_numpy(xs).to(dev) if dt == "f32"
         else torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).to(dev))
    idx = idx_of(T, K, E)
    w = torch.from_numpy(rng.random((T, K)).astype(np.float32)).to(dev)
    o = moe.dispatch(x, idx, E, cap=cap)
    c1, w1 = moe.combine(o.packed, o.tok_map, w, out_dtype=torch.bfloat16)
    c2, _ = moe.combine(o.packed, o.tok_map, w, out_dtype=torch.float32)
    written = torch.sort(o.tok_map[o.tok_map >= 0]).values   # rows no entry owns are never written
    out[f"copy_{dt}_{T}_{H}"] = h(o.packed[written], o.packed_src[written], o.tok_map, o.packed_cnt,
                                  o.packed_off, o.stats, c1, w1, c2)

# e4m3 and e2m1 packs (with scaled blocks), their combines, the pre-quantized dispatch
T, H, K, E = 1500, 7168, 8, 256
xs = W.inject_outliers(W.normal_x(rng, T, H, "bf16"), np.arange(0, T, 7), 1000.0)
x = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).to(dev)
idx = idx_of(T, K, E)
w = torch.from_numpy(rng.random((T, K)).astype(np.float32)).to(dev)
n = None
for name, kw in (("fp8", dict(fp8=True)), ("fp4", dict(fp4=True))):
    o = moe.dispatch(x, idx, E, **kw)
    n = int(o.packed_off[-1].item())
    comb = moe.combine_fp4 if name == "fp4" else moe.combine_fp8
    c, cw = comb(o.packed, o.scales, o.tok_map, w)
    out[name] = h(o.packed[:n], o.scales[:n], o.tok_map, c, cw)
    if name == "fp8":
        q = moe.dispatch_prequant(o.packed[:T].contiguous(), o.scales[:T].contiguous(), idx, E)
        out["prequant"] = h(q.packed[:n], q.scales[:n], q.tok_map)

# dedup: recv copy, expansion, fused and two-stage combines
T, H, K, E, R = 3000, 1024, 6, 64, 8
xs = W.normal_x(rng, T, H, "f32")
x = torch.from_numpy(xs).to(dev)
idx = idx_of(T, K, E)
w = torch.from_numpy(rng.random((T, K)).astype(np.float32)).to(dev)
o = moe.dedup_dispatch(x, idx, E, R)
nr = int(o.recv_off[-1].item())
npk = int(o.packed_off[-1].item())
part = torch.zeros((T * min(K, R), H), dtype=torch.float32, device=dev)
plan = dict(R=R, idx=idx, rank_slot=o.rank_slot, recv_rows=T * min(K, R))
c1, w1 = moe.combine(o.packed, o.tok_map, w, E=E, out_dtype=torch.float32, dedup=plan)
c2, _ = moe.combine(o.packed, o.tok_map, w, E=E, out_dtype=torch.float32, dedup=dict(plan, partial=part))
out["dedup"] = h(o.recv_x[:nr], o.recv_src[:nr], o.rank_slot, o.packed[:npk], o.tok_map, c1, w1, c2,
                 part[:nr])
torch.cuda.synchronize()
print("GEOMETRY-RESULT " + json.dumps(out), flush=True)
"""

GEOMETRIES = {
    "default": None,
    "small": ("combine_chunk_units=64,combine_wgs_per_cu=0,fp8_chunks=1,fp8_wgs_per_cu=0,"
              "copy_chunks=3,copy_wgs_per_cu=7,recv_chunks=1,recv_wgs_per_cu=5,expand_chunks=4,"
              "expand_wgs_per_cu=0"),
    "large": ("combine_chunk_units=160,combine_wgs_per_cu=16,fp8_chunks=8,fp8_wgs_per_cu=3,"
              "copy_chunks=8,copy_wgs_per_cu=16,recv_chunks=8,recv_wgs_per_cu=16,"
              "expand_chunks=8,expand_wgs_per_cu=16"),
}


def _run(name, spec):
    env = dict(os.environ)
    env.pop("MOE_GEOM", None)
    if spec is not None:
        env["MOE_GEOM"] = spec
    note(f"geometry child {name}")
    r = subprocess.run([sys.executable, "-c", f"ROOT = {ROOT!r}\n" + CHILD], capture_output=True,
                       text=True, env=env, timeout=150, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    line = next(l for l in r.stdout.splitlines() if l.startswith("GEOMETRY-RESULT "))
    return json.loads(line[len("GEOMETRY-RESULT "):])


def test_results_do_not_depend_on_the_geometry():
    base = _run("default", None)
    assert "ignored" not in base["geometry"]
    for name in ("small", "large"):
        got = _run(name, GEOMETRIES[name])
        assert got["geometry"] == GEOMETRIES[name], got["geometry"]
        for key, digest in base.items():
            if key != "geometry":
                assert got[key] == digest, (name, key)
