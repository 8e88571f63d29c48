"""Host-only checks of the C ABI: the library loads, exports every function the
header declares, sizes its workspace, and rejects bad arguments with the
documented status before enqueueing anything.

The calls run in a child process that sees no GPU (ROCR_VISIBLE_DEVICES=-1), so
even a validation bug could not launch a kernel on a device."""
import os
import re
import subprocess
import sys
import textwrap

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_route.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ["moe_route_count", "moe_dispatch", "moe_combine", "moe_dedup_dispatch",
              "moe_fp8_dequant", "moe_workspace_size", "moe_last_error", "moe_version"]:
        assert n in names, n


CHILD = textwrap.dedent(r"""
import ctypes, json, sys
sys.path.insert(0, ROOT)
from combine_moe_route_count_amd import _lib as L
lib = L.load()
res = {}
res["exports"] = {n: hasattr(lib, n) for n in NAMES}
res["version"] = lib.moe_version()
res["geometry"] = lib.moe_geometry().decode()
res["ws"] = [lib.moe_workspace_size(*a) for a in [(8192, 8, 256, 0), (8192, 8, 256, 0),
             (16384, 6, 64, 8), (0, 1, 1, 0), (1, 16, 1024, 0), (-1, 8, 8, 0)]]
P = ctypes.c_void_p
A = P(0x100000)       # aligned stand-in pointers: never dereferenced, every case fails a check
A8 = P(0x100008)
A4 = P(0x100004)
ws_need = lib.moe_workspace_size(100, 4, 16, 0)
WS = P(0x200000)

def disp(**kw):
    a = dict(x=A, x_dt=0, T=100, H=64, idx=A, K=4, E=16, cap=0, rows=400, packed=A, pdt=0,
             scales=None, pc=A, po=None, ps=A, tm=A, st=None, ws=WS, wsb=ws_need)
    a.update(kw)
    st = lib.moe_dispatch(a["x"], a["x_dt"], a["T"], a["H"], a["idx"], a["K"], a["E"], a["cap"],
                          a["rows"], a["packed"], a["pdt"], a["scales"], a["pc"], a["po"], a["ps"],
                          a["tm"], a["st"], a["ws"], a["wsb"], None)
    return [st, lib.moe_last_error().decode()]

res["dispatch"] = {
    "K0": disp(K=0), "K17": disp(K=17), "E0": disp(E=0), "E1025": disp(E=1025),
    "Tneg": disp(T=-1), "H12": disp(H=12), "Hzero": disp(H=0),
    "fp8_H64": disp(pdt=2, scales=A, H=64),
    "fp8_from_f32": disp(pdt=2, x_dt=1, scales=A, H=128),
    "fp8_no_scales": disp(pdt=2, H=128),
    "scales_not_fp8": disp(scales=A),
    "dtype_mix": disp(pdt=1),
    "bad_dtype": disp(x_dt=7),
    "x_null": disp(x=None), "x_unaligned": disp(x=A8), "packed_unaligned": disp(packed=A8),
    "idx_null": disp(idx=None), "tok_map_null": disp(tm=None), "tok_map_unaligned": disp(tm=A4),
    "pc_null": disp(pc=None), "ps_null": disp(ps=None),
    "cap_neg": disp(cap=-1), "rows_neg": disp(rows=-1), "rows_huge": disp(rows=1 << 31),
    "TK_overflow": disp(T=1 << 28, K=16),
    "ws_small": disp(wsb=ws_need - 1), "ws_null": disp(ws=None),
    "ws_unaligned": disp(ws=P(0x200010)),
}

def comb(**kw):
    a = dict(y=A, ydt=0, yr=10, H=64, tm=A, w=A, T=5, K=2, E=8, dd=None, out=A, odt=0, ow=None)
    a.update(kw)
    st = lib.moe_combine(a["y"], a["ydt"], a["yr"], a["H"], a["tm"], a["w"], a["T"], a["K"], a["E"],
                         a["dd"], a["out"], a["odt"], a["ow"], None)
    return [st, lib.moe_last_error().decode()]

bad_plan = L.DedupPlan(3, 0x100000, 0x100000, 10, None)
res["combine"] = {
    "K0": comb(K=0), "H7": comb(H=7), "y_fp8": comb(ydt=2), "out_fp8": comb(odt=2),
    "y_null": comb(y=None), "tm_null": comb(tm=None), "w_null": comb(w=None),
    "out_unaligned": comb(out=A8), "y_rows_neg": comb(yr=-1), "y_rows_huge": comb(yr=1 << 31),
    "y_rows_2p32": comb(yr=1 << 32),
    "dd_R_not_divisor": comb(dd=ctypes.byref(bad_plan)),
}

def dd(**kw):
    a = dict(x=A, xdt=1, T=50, H=64, idx=A, K=6, E=64, R=8, rx=A, rr=300, rc=A, ro=A, rs=A, rsl=A,
             cap=0, pr=300, px=A, pc=A, po=None, ps=A, tm=A, st=None, ws=WS,
             wsb=lib.moe_workspace_size(50, 6, 64, 8))
    a.update(kw)
    st = lib.moe_dedup_dispatch(a["x"], a["xdt"], a["T"], a["H"], a["idx"], a["K"], a["E"], a["R"],
                                a["rx"], a["rr"], a["rc"], a["ro"], a["rs"], a["rsl"], a["cap"],
                                a["pr"], a["px"], a["pc"], a["po"], a["ps"], a["tm"], a["st"],
                                a["ws"], a["wsb"], None)
    return [st, lib.moe_last_error().decode()]

res["dedup"] = {
    "R0": dd(R=0), "R33": dd(R=33), "R_not_divisor": dd(R=7), "recv_null": dd(rx=None),
    "rank_slot_null": dd(rsl=None), "ws_small": dd(wsb=100), "recv_rows_neg": dd(rr=-1),
    "fp8": dd(xdt=2),
}
res["dequant"] = {
    "H64": [lib.moe_fp8_dequant(A, A, 4, 64, A, None), lib.moe_last_error().decode()],
    "rows_neg": [lib.moe_fp8_dequant(A, A, -1, 128, A, None), lib.moe_last_error().decode()],
    "scales_null": [lib.moe_fp8_dequant(A, None, 4, 128, A, None), lib.moe_last_error().decode()],
}
res["copy16"] = {
    "bytes_odd": [lib.moe_copy16(A, P(0x300000), 24, None), lib.moe_last_error().decode()],
    "bytes_neg": [lib.moe_copy16(A, P(0x300000), -16, None), lib.moe_last_error().decode()],
    "src_null": [lib.moe_copy16(None, P(0x300000), 32, None), lib.moe_last_error().decode()],
    "unaligned": [lib.moe_copy16(A8, P(0x300000), 32, None), lib.moe_last_error().decode()],
    "overlap": [lib.moe_copy16(A, P(0x100010), 64, None), lib.moe_last_error().decode()],
}
def c8(**kw):
    a = dict(q=A, sc=A, yr=10, H=128, tm=A, w=A, T=5, K=2, out=A, odt=0, ow=None)
    a.update(kw)
    st = lib.moe_combine_fp8(a["q"], a["sc"], a["yr"], a["H"], a["tm"], a["w"], a["T"], a["K"],
                             a["out"], a["odt"], a["ow"], None)
    return [st, lib.moe_last_error().decode()]

def c4(**kw):
    a = dict(q=A, sc=A, yr=10, H=128, tm=A, w=A, T=5, K=2, out=A, odt=0, ow=None)
    a.update(kw)
    st = lib.moe_combine_fp4(a["q"], a["sc"], a["yr"], a["H"], a["tm"], a["w"], a["T"], a["K"],
                             a["out"], a["odt"], a["ow"], None)
    return [st, lib.moe_last_error().decode()]

res["combine_fp4"] = {"H64": c4(H=64), "K0": c4(K=0), "out_fp4": c4(odt=3), "q_unaligned": c4(q=A8),
                      "y_rows_huge": c4(yr=1 << 31)}
res["dispatch"]["fp4_from_f32"] = disp(x_dt=1, pdt=3, scales=A, H=128)
res["dispatch"]["fp4_no_scales"] = disp(pdt=3, H=128)
res["dispatch"]["fp4_H64"] = disp(pdt=3, scales=A, H=64)
res["dispatch"]["bad_packed_dtype"] = disp(pdt=9)
res["combine_fp8"] = {
    "H64": c8(H=64), "K0": c8(K=0), "K17": c8(K=17), "out_fp8": c8(odt=2), "q_null": c8(q=None),
    "q_unaligned": c8(q=A8), "scales_unaligned": c8(sc=P(0x100002)), "tm_null": c8(tm=None),
    "out_unaligned": c8(out=A8), "Tneg": c8(T=-1), "y_rows_neg": c8(yr=-1),
    "y_rows_huge": c8(yr=1 << 31),
}
def rp(**kw):
    a = dict(x=A, xdt=0, xs=None, T=5, H=128, tm=A, K=2, rows=10, px=A, pdt=0, ps=None)
    a.update(kw)
    st = lib.moe_dispatch_replay(a["x"], a["xdt"], a["xs"], a["T"], a["H"], a["tm"], a["K"], a["rows"],
                                 a["px"], a["pdt"], a["ps"], None)
    return [st, lib.moe_last_error().decode()]

def pq(**kw):
    a = dict(x=A, xs=A, T=100, H=128, idx=A, K=4, E=16, cap=0, rows=400, px=A, ps=A, pc=A, po=None,
             psrc=A, tm=A, st=None, ws=WS, wsb=ws_need)
    a.update(kw)
    st = lib.moe_dispatch_prequant(a["x"], a["xs"], a["T"], a["H"], a["idx"], a["K"], a["E"], a["cap"],
                                   a["rows"], a["px"], a["ps"], a["pc"], a["po"], a["psrc"], a["tm"],
                                   a["st"], a["ws"], a["wsb"], None)
    return [st, lib.moe_last_error().decode()]

res["replay"] = {
    "K0": rp(K=0), "Tneg": rp(T=-1), "tm_null": rp(tm=None), "tm_unaligned": rp(tm=A4),
    "dtype_mix": rp(pdt=1), "fp8_no_scales": rp(pdt=2), "f32_to_fp8": rp(xdt=1, pdt=2, ps=A),
    "prequant_no_xscales": rp(xdt=2, pdt=2, ps=A), "xscales_not_fp8": rp(xs=A),
    "fp8_H64": rp(pdt=2, ps=A, H=64), "x_unaligned": rp(x=A8), "rows_neg": rp(rows=-1),
}
res["prequant"] = {
    "xs_null": pq(xs=None), "H64": pq(H=64), "ps_null": pq(ps=None), "K0": pq(K=0),
    "ws_small": pq(wsb=ws_need - 1), "idx_null": pq(idx=None), "xs_unaligned": pq(xs=P(0x100002)),
}
res["dispatch"]["fp8_input"] = disp(x_dt=2, pdt=2, scales=A, H=128)

def na(**kw):
    a = dict(x=A, x_dt=0, T=100, H=64, idx=A, K=4, E=16, cap=0, rows=400, packed=A, pdt=0,
             scales=None, pc=A, po=None, ps=A, tm=A, st=None)
    a.update(kw)
    st = lib.moe_dispatch_noalloc(a["x"], a["x_dt"], a["T"], a["H"], a["idx"], a["K"], a["E"],
                                  a["cap"], a["rows"], a["packed"], a["pdt"], a["scales"], a["pc"],
                                  a["po"], a["ps"], a["tm"], a["st"], None)
    return [st, lib.moe_last_error().decode()]

res["noalloc"] = {
    "too_big_E256": na(T=104641, K=8, E=256, rows=837128), "too_big_E1024": na(T=65536, K=8, E=1024),
    "K0": na(K=0), "E1025": na(E=1025), "H12": na(H=12), "x_null": na(x=None),
    "fp8_input": na(x_dt=2, pdt=2, scales=A, H=128), "pc_null": na(pc=None),
    "tok_map_unaligned": na(tm=A4), "fp8_no_scales": na(pdt=2, H=128),
}
res["route"] = {
    "cnt_null": [lib.moe_route_count(A, 10, 2, 4, None, A, None, WS, 1 << 20, None),
                 lib.moe_last_error().decode()],
    "ws_small": [lib.moe_route_count(A, 10, 2, 4, A, A, None, WS, 0, None),
                 lib.moe_last_error().decode()],
}
# moe_last_error is per thread: two threads fail differently, then each reads
# its own text after both have failed; a thread that never failed reads ""
import threading
bar = threading.Barrier(2)
thr = {}
def _fail(name, kw):
    st = disp(**kw)[0]
    bar.wait()
    thr[name] = [st, lib.moe_last_error().decode()]
def _fresh():
    thr["fresh"] = lib.moe_last_error().decode()
ts = [threading.Thread(target=_fail, args=("K", dict(K=0))),
      threading.Thread(target=_fail, args=("E", dict(E=0))), threading.Thread(target=_fresh)]
for t in ts:
    t.start()
for t in ts:
    t.join()
res["threads"] = thr
print(json.dumps(res))
""")


def _run_child():
    env = dict(os.environ, ROCR_VISIBLE_DEVICES="-1", HIP_VISIBLE_DEVICES="-1")
    code = f"ROOT = {ROOT!r}\nNAMES = {_declared_functions()!r}\n" + CHILD
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    import json
    return json.loads(r.stdout.strip().splitlines()[-1])


_RES = None


def _res():
    global _RES
    if _RES is None:
        _RES = _run_child()
    return _RES


def test_library_exports_every_declared_function():
    ex = _res()["exports"]
    assert ex and all(ex.values()), ex


def test_workspace_size():
    ws = _res()["ws"]
    assert ws[0] == ws[1] > 0          # deterministic
    assert ws[2] > 0 and ws[3] > 0 and ws[4] > 0
    assert ws[5] == 0                  # invalid sizes give 0
    assert all(w % 256 == 0 for w in ws)
    assert _res()["version"] >> 16 == 1 and _res()["version"] & 0xFFFF >= 2


INVALID, UNSUPPORTED, WORKSPACE = -1, -2, -3


def test_dispatch_argument_errors():
    d = _res()["dispatch"]
    expect_ws = {"ws_small", "ws_null", "ws_unaligned"}
    for case, (st, msg) in d.items():
        if case in expect_ws:
            assert st == WORKSPACE, (case, st, msg)
        elif case in ("fp8_from_f32", "fp4_from_f32"):
            assert st == UNSUPPORTED, (case, st, msg)
        else:
            assert st == INVALID, (case, st, msg)
        assert msg, case


def test_combine_argument_errors():
    for case, (st, msg) in _res()["combine"].items():
        assert st == (UNSUPPORTED if case == "y_fp8" else INVALID), (case, st, msg)
        assert msg


def test_dedup_and_helpers_argument_errors():
    for case, (st, msg) in _res()["dedup"].items():
        assert st == (WORKSPACE if case == "ws_small" else INVALID), (case, st, msg)
    for case, (st, msg) in _res()["dequant"].items():
        assert st == INVALID, (case, st, msg)
    for case, (st, msg) in _res()["replay"].items():
        assert st == (UNSUPPORTED if case == "f32_to_fp8" else INVALID) and msg, (case, st, msg)
    for case, (st, msg) in _res()["prequant"].items():
        assert st == (WORKSPACE if case == "ws_small" else INVALID) and msg, (case, st, msg)
    for case, (st, msg) in _res()["combine_fp4"].items():
        assert st == INVALID and msg, (case, st, msg)
    for case, (st, msg) in _res()["combine_fp8"].items():
        assert st == INVALID and msg, (case, st, msg)
    for case, (st, msg) in _res()["copy16"].items():
        assert st == INVALID and msg, (case, st, msg)
    r = _res()["route"]
    assert r["cnt_null"][0] == INVALID and r["ws_small"][0] == WORKSPACE


def test_noalloc_dispatch_argument_errors():
    """The static-workspace dispatch rejects sizes past its 4 MiB array and bad
    arguments on the host, before it looks anything up on a device."""
    for case, (st, msg) in _res()["noalloc"].items():
        want = WORKSPACE if case.startswith("too_big") else INVALID
        assert st == want and msg, (case, st, msg)
    assert "static" in _res()["noalloc"]["too_big_E256"][1]


def test_last_error_is_per_thread():
    t = _res()["threads"]
    assert t["K"][0] == INVALID and "K=0" in t["K"][1], t
    assert t["E"][0] == INVALID and "E=0" in t["E"][1], t
    assert t["fresh"] == "", t


DEFAULT_GEOMETRY = ("combine_chunk_units=256,combine_wgs_per_cu=5,fp8_chunks=2,fp8_wgs_per_cu=8,"
                    "copy_chunks=1,copy_wgs_per_cu=0,recv_chunks=2,recv_wgs_per_cu=0,"
                    "expand_chunks=1,expand_wgs_per_cu=4")


def test_default_geometry():
    assert _res()["geometry"] == DEFAULT_GEOMETRY


def test_geometry_override_and_rejects():
    """MOE_GEOM overrides keys in range and lists everything else as ignored."""
    code = ("import sys\nsys.path.insert(0, %r)\nfrom combine_moe_route_count_amd import _lib\n"
            "print(_lib.load().moe_geometry().decode())" % ROOT)
    env = dict(os.environ, ROCR_VISIBLE_DEVICES="-1", HIP_VISIBLE_DEVICES="-1",
               MOE_GEOM="combine_chunk_units=224,copy_chunks=2,bogus=3,fp8_chunks=99,"
                        "expand_wgs_per_cu=x,,combine_wgs_per_cu=0,recv_chunks,fp8_wgs_per_cu=2,"
                        "combine_chunk_units=32")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    got = r.stdout.strip().splitlines()[-1]
    want = (DEFAULT_GEOMETRY.replace("combine_chunk_units=256", "combine_chunk_units=224")
            .replace("copy_chunks=1", "copy_chunks=2")
            .replace("combine_wgs_per_cu=5", "combine_wgs_per_cu=0")
            + "; ignored: bogus=3,fp8_chunks=99,expand_wgs_per_cu=x,recv_chunks,fp8_wgs_per_cu=2,"
              "combine_chunk_units=32")
    assert got == want, got
