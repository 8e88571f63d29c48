"""Every entry point captured in one HIP graph: the route count, the dedup
dispatch with both dedup combines, the pre-quantized dispatch, its replay and
the e4m3 combine, the e2m1 dispatch with its replay and combine, and the fp8
dequantize.  The graph is replayed four times; before each replay its outputs
are poisoned, and between replays the same calls run eagerly on other output
buffers but the same workspaces.  Every replay and every eager round must give
the bytes of the eager reference, so no call relies on state a replay leaves
(workspace tickets, counters) and nothing in the graph is a memory-set node."""
import numpy as np
import pytest
import torch

import combine_moe_route_count_amd as moe
import workloads as W
from _gpu_util import DEV, dev, dev_bf16, note, poison_

pytestmark = pytest.mark.gpu


def _inputs():
    rng = np.random.default_rng(2024)
    T, K, E, R, H = 1500, 6, 64, 8, 512
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    idx[rng.random((T, K)) < 0.05] = -1
    xf = W.normal_x(rng, T, H, "f32")
    xb = W.inject_outliers(W.normal_x(rng, T, H, "bf16"), np.arange(0, T, 9), 1000.0)
    w = rng.random((T, K)).astype(np.float32)
    return dict(T=T, K=K, E=E, R=R, H=H, idx=dev(idx), xf=dev(xf), xb=dev_bf16(xb), w=dev(w),
                ws_r=moe.workspace(T, K, E, R), ws_p=moe.workspace(T, K, E))


def _outputs(c):
    T, K, E, R, H = c["T"], c["K"], c["E"], c["R"], c["H"]
    rr = T * min(K, R)
    o = {
        "cnt": torch.empty(E, dtype=torch.int32, device=DEV),
        "off": torch.empty(E + 1, dtype=torch.int32, device=DEV),
        "rstats": torch.empty(3, dtype=torch.int32, device=DEV),
        "dd": moe._lib.alloc_dedup(T, H, K, E, R, rr, T * K, torch.float32, DEV),
        "part": torch.empty((rr, H), dtype=torch.float32, device=DEV),
        "c_fused": torch.empty((T, H), dtype=torch.float32, device=DEV),
        "w_fused": torch.empty(T, dtype=torch.float32, device=DEV),
        "c_two": torch.empty((T, H), dtype=torch.float32, device=DEV),
        "w_two": torch.empty(T, dtype=torch.float32, device=DEV),
        "q8": moe._lib.alloc_dispatch(T, H, K, E, T * K, torch.bfloat16, True, DEV),
        "pq": moe._lib.alloc_dispatch(T, H, K, E, T * K, torch.uint8, True, DEV),
        "rp8": torch.empty((T * K, H), dtype=torch.uint8, device=DEV),
        "rp8s": torch.empty((T * K, H // 128), dtype=torch.float32, device=DEV),
        "c8": torch.empty((T, H), dtype=torch.bfloat16, device=DEV),
        "w8": torch.empty(T, dtype=torch.float32, device=DEV),
        "q4": moe._lib.alloc_dispatch(T, H, K, E, T * K, torch.bfloat16, False, DEV, fp4=True),
        "rp4": torch.empty((T * K, H // 2), dtype=torch.uint8, device=DEV),
        "rp4s": torch.empty((T * K, H // 128), dtype=torch.float32, device=DEV),
        "c4": torch.empty((T, H), dtype=torch.float32, device=DEV),
        "w4": torch.empty(T, dtype=torch.float32, device=DEV),
        "deq": torch.empty((T * K, H), dtype=torch.bfloat16, device=DEV),
    }
    return o


def _tensors(o):
    for k, v in o.items():
        if isinstance(v, torch.Tensor):
            yield k, v
        else:
            for f in ("recv_x", "recv_cnt", "recv_off", "recv_src", "rank_slot", "packed", "scales",
                      "packed_cnt", "packed_off", "packed_src", "tok_map", "stats"):
                t = getattr(v, f, None)
                if t is not None:
                    yield f"{k}.{f}", t


def _poison(o):
    for _, t in _tensors(o):
        poison_(t)


def _run(c, o):
    E, R = c["E"], c["R"]
    moe.route_count(c["idx"], E, cnt=o["cnt"], off=o["off"], stats=o["rstats"], ws=c["ws_p"])
    dd = o["dd"]
    moe.dedup_dispatch(c["xf"], c["idx"], E, R, out=dd, ws=c["ws_r"])
    rr = dd.recv_x.shape[0]
    plan = dict(R=R, idx=c["idx"], rank_slot=dd.rank_slot, recv_rows=rr)
    moe.combine(dd.packed, dd.tok_map, c["w"], E=E, out_dtype=torch.float32, dedup=plan,
                out=o["c_fused"], out_weights=o["w_fused"])
    moe.combine(dd.packed, dd.tok_map, c["w"], E=E, out_dtype=torch.float32,
                dedup=dict(plan, partial=o["part"]), out=o["c_two"], out_weights=o["w_two"])
    q8 = o["q8"]
    moe.dispatch(c["xb"], c["idx"], E, fp8=True, out=q8, ws=c["ws_p"])
    T = c["T"]
    pq = o["pq"]
    moe.dispatch_prequant(q8.packed[:T], q8.scales[:T], c["idx"], E, out=pq, ws=c["ws_p"])
    moe.dispatch_replay(q8.packed[:T], pq.tok_map, o["rp8"], scales=o["rp8s"], x_scales=q8.scales[:T])
    moe.combine_fp8(pq.packed, pq.scales, pq.tok_map, c["w"], out=o["c8"], out_weights=o["w8"])
    q4 = o["q4"]
    moe.dispatch(c["xb"], c["idx"], E, fp4=True, out=q4, ws=c["ws_p"])
    moe.dispatch_replay(c["xb"], q4.tok_map, o["rp4"], scales=o["rp4s"], fp4=True)
    moe.combine_fp4(q4.packed, q4.scales, q4.tok_map, c["w"], out_dtype=torch.float32, out=o["c4"],
                    out_weights=o["w4"])
    moe.fp8_dequant(q8.packed, q8.scales, o["deq"])


def _assert_same(a, b, what):
    for (k, x), (_, y) in zip(_tensors(a), _tensors(b)):
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.uint8 else x,
                           y.view(torch.uint8) if y.dtype != torch.uint8 else y), f"{what}: {k}"


def test_every_entry_point_in_one_graph():
    c = _inputs()
    ref, g_out, e_out = _outputs(c), _outputs(c), _outputs(c)
    _poison(ref)
    note("graph: eager reference")
    _run(c, ref)
    torch.cuda.synchronize()
    cs = torch.cuda.Stream(DEV)
    cs.wait_stream(torch.cuda.current_stream(DEV))
    _poison(g_out)
    torch.cuda.synchronize()
    note("graph: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            _run(c, g_out)
    torch.cuda.synchronize()
    for rep in range(4):
        _poison(g_out)
        torch.cuda.synchronize()
        note(f"graph: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        _assert_same(g_out, ref, f"replay {rep}")
        _poison(e_out)
        _run(c, e_out)           # eager calls on the same workspaces between replays
        torch.cuda.synchronize()
        _assert_same(e_out, ref, f"eager round {rep}")
