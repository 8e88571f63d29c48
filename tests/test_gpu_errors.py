"""Failed calls on a real device: every entry point, given one bad argument
next to real device buffers, returns its documented status and a message, and
after the device has drained every buffer still holds the bytes it held
before the call (an error enqueues nothing and changes no buffer)."""
import pytest
import torch

import combine_moe_route_count_amd as moe
from combine_moe_route_count_amd import _lib as L
from _gpu_util import DEV, note

pytestmark = pytest.mark.gpu

INVALID, UNSUPPORTED, WORKSPACE = L.MOE_ERR_INVALID_ARG, L.MOE_ERR_UNSUPPORTED, L.MOE_ERR_WORKSPACE
T, K, E, H, R = 300, 4, 64, 256, 8


@pytest.fixture(scope="module")
def bufs():
    g = torch.Generator().manual_seed(3)
    def rnd(n):
        return torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).to(DEV)
    b = {
        "x": rnd(T * H * 4), "idx": torch.randint(0, E, (T * K,), dtype=torch.int32, generator=g).to(DEV),
        "packed": rnd(T * K * H * 4), "scales": rnd(T * K * (H // 128) * 4), "cnt": rnd(E * 4),
        "off": rnd((E + 1) * 4), "src": rnd(T * K * 4), "tm": rnd(T * K * 8), "stats": rnd(12),
        "out": rnd(T * H * 4), "ow": rnd(T * 4), "w": rnd(T * K * 4), "recv": rnd(T * R * H * 4),
        "rcnt": rnd(R * 4), "roff": rnd((R + 1) * 4), "rsrc": rnd(T * R * 4), "rslot": rnd(T * R * 4),
        "ws": rnd(moe.workspace_size(T, K, E, R) + 4096),
    }
    # a valid routing map, so no failing combine could read past y even if it ran
    tm = torch.arange(T * K, dtype=torch.int64, device=DEV)
    b["tm"].view(torch.int64).copy_(tm)
    torch.cuda.synchronize()
    return b


def p(t, off=0):
    return t.data_ptr() + off


def _expect(bufs, status, fn):
    before = {k: v.clone() for k, v in bufs.items()}
    torch.cuda.synchronize()
    st = fn()
    msg = L.load().moe_last_error().decode()
    torch.cuda.synchronize()
    assert st == status, (st, msg)
    assert msg
    for k, v in bufs.items():
        assert torch.equal(v, before[k]), f"buffer {k} changed by a failed call ({msg})"


def _disp(b, **kw):
    a = dict(x=p(b["x"]), x_dt=L.MOE_BF16, T=T, H=H, idx=p(b["idx"]), K=K, E=E, cap=0, rows=T * K,
             packed=p(b["packed"]), pdt=L.MOE_BF16, scales=None, pc=p(b["cnt"]), po=p(b["off"]),
             ps=p(b["src"]), tm=p(b["tm"]), st=p(b["stats"]), ws=p(b["ws"]),
             wsb=moe.workspace_size(T, K, E))
    a.update(kw)
    return lambda: L.load().moe_dispatch(
        a["x"], a["x_dt"], a["T"], a["H"], a["idx"], a["K"], a["E"], a["cap"], a["rows"],
        a["packed"], a["pdt"], a["scales"], a["pc"], a["po"], a["ps"], a["tm"], a["st"], a["ws"],
        a["wsb"], None)


DISPATCH_CASES = {
    "ws_short": (WORKSPACE, dict(wsb=1024)),
    "ws_unaligned": (WORKSPACE, dict(ws="+16")),
    "K0": (INVALID, dict(K=0)),
    "E1025": (INVALID, dict(E=1025)),
    "H12": (INVALID, dict(H=12)),
    "fp8_from_f32": (UNSUPPORTED, dict(x_dt=L.MOE_F32, pdt=L.MOE_FP8_E4M3, scales="scales")),
    "fp8_without_scales": (INVALID, dict(pdt=L.MOE_FP8_E4M3)),
    "x_unaligned": (INVALID, dict(x="+2")),
    "tok_map_unaligned": (INVALID, dict(tm="+4")),
    "rows_past_int32": (INVALID, dict(rows=1 << 31)),
}


@pytest.mark.parametrize("case", list(DISPATCH_CASES))
def test_dispatch_error_changes_nothing(bufs, case):
    status, kw = DISPATCH_CASES[case]
    kw = dict(kw)
    for k, v in list(kw.items()):     # "+n": the buffer's own pointer moved by n bytes
        if isinstance(v, str):
            kw[k] = p(bufs[k], int(v[1:])) if v.startswith("+") else p(bufs[v])
    note(f"failing dispatch {case}")
    _expect(bufs, status, _disp(bufs, **kw))


def test_other_entry_points_errors_change_nothing(bufs):
    lib = L.load()
    b = bufs
    ws_b = moe.workspace_size(T, K, E, R)
    note("failing combine / quantized combines / dedup / replay / prequant / noalloc / route count")
    cases = [
        (INVALID, lambda: lib.moe_combine(p(b["packed"]), L.MOE_BF16, 1 << 31, H, p(b["tm"]), p(b["w"]),
                                          T, K, E, None, p(b["out"]), L.MOE_BF16, p(b["ow"]), None)),
        (INVALID, lambda: lib.moe_combine(p(b["packed"]), L.MOE_BF16, T * K, H, p(b["tm"]), p(b["w"]),
                                          T, 17, E, None, p(b["out"]), L.MOE_BF16, p(b["ow"]), None)),
        (UNSUPPORTED, lambda: lib.moe_combine(p(b["packed"]), L.MOE_FP8_E4M3, T * K, H, p(b["tm"]),
                                              p(b["w"]), T, K, E, None, p(b["out"]), L.MOE_BF16,
                                              p(b["ow"]), None)),
        (INVALID, lambda: lib.moe_combine_fp8(p(b["packed"]), p(b["scales"]), T * K, 64, p(b["tm"]),
                                              p(b["w"]), T, K, p(b["out"]), L.MOE_BF16, p(b["ow"]),
                                              None)),
        (INVALID, lambda: lib.moe_combine_fp4(p(b["packed"]), p(b["scales"]), T * K, 64, p(b["tm"]),
                                              p(b["w"]), T, K, p(b["out"]), L.MOE_BF16, p(b["ow"]),
                                              None)),
        (INVALID, lambda: lib.moe_dedup_dispatch(
            p(b["x"]), L.MOE_F32, T, H, p(b["idx"]), K, E, 7, p(b["recv"]), T * R, p(b["rcnt"]),
            p(b["roff"]), p(b["rsrc"]), p(b["rslot"]), 0, T * K, p(b["packed"]), p(b["cnt"]),
            p(b["off"]), p(b["src"]), p(b["tm"]), p(b["stats"]), p(b["ws"]), ws_b, None)),
        (WORKSPACE, lambda: lib.moe_dedup_dispatch(
            p(b["x"]), L.MOE_F32, T, H, p(b["idx"]), K, E, R, p(b["recv"]), T * R, p(b["rcnt"]),
            p(b["roff"]), p(b["rsrc"]), p(b["rslot"]), 0, T * K, p(b["packed"]), p(b["cnt"]),
            p(b["off"]), p(b["src"]), p(b["tm"]), p(b["stats"]), p(b["ws"]), 256, None)),
        (INVALID, lambda: lib.moe_dispatch_replay(p(b["x"]), L.MOE_BF16, None, T, H, p(b["tm"]), K,
                                                  T * K, p(b["packed"]), L.MOE_F32, None, None)),
        (INVALID, lambda: lib.moe_dispatch_prequant(
            p(b["x"]), None, T, H, p(b["idx"]), K, E, 0, T * K, p(b["packed"]), p(b["scales"]),
            p(b["cnt"]), p(b["off"]), p(b["src"]), p(b["tm"]), p(b["stats"]), p(b["ws"]), ws_b, None)),
        (WORKSPACE, lambda: lib.moe_dispatch_noalloc(
            p(b["x"]), L.MOE_BF16, 104641, H, p(b["idx"]), 8, 256, 0, 837128, p(b["packed"]),
            L.MOE_BF16, None, p(b["cnt"]), p(b["off"]), p(b["src"]), p(b["tm"]), p(b["stats"]), None)),
        (INVALID, lambda: lib.moe_route_count(p(b["idx"]), T, K, E, None, p(b["off"]), p(b["stats"]),
                                              p(b["ws"]), ws_b, None)),
        (INVALID, lambda: lib.moe_fp8_dequant(p(b["packed"]), p(b["scales"]), T, 64, p(b["out"]), None)),
        (INVALID, lambda: lib.moe_copy16(p(b["x"]), p(b["out"]), 24, None)),
    ]
    for status, fn in cases:
        _expect(bufs, status, fn)
