"""CPU oracle for the MoE route-count / dispatch / combine path (numpy front end).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may use this package; the GPU library never does.  The
arithmetic lives in moe_oracle.c (plain C, built with gcc -ffp-contract=off);
this module allocates numpy outputs, fills the ones that may be left partly
untouched with a poison pattern, and calls it through ctypes.

Every function cites, in moe_oracle.c, the passage of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

BF16, F32, FP8, FP4 = 0, 1, 2, 3
DT = {"bf16": BF16, "f32": F32, "fp8": FP8, "fp4": FP4}
NP_DT = {BF16: np.uint16, F32: np.float32, FP8: np.uint8, FP4: np.uint8}


def _row_width(dt, H):
    """Array width of one packed row of H elements (fp4: two codes per byte)."""
    return {BF16: H, F32: H, FP8: H, FP4: H // 2}[dt]


def _quantized(dt):
    return dt in (FP8, FP4)

# Poison written into outputs before a call, so a row or slot that a call does
# not own can be told apart from one it wrote.
POISON_BYTE = 0xA5
POISON_I32 = -7

_lib = None


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-std=gnu99", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-shared", "-fPIC", "-o", _LIB_PATH, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def _load():
    """The compiled oracle; MOE_ORACLE_LIB names another build of the same
    source (the sanitizer test loads one built with ASan and UBSan)."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("MOE_ORACLE_LIB")
    if not path:
        path = _LIB_PATH
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build()
    lib = ctypes.CDLL(path)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sigs = {
        "oracle_route_count": [P, I64, I32, I32, P, P, P],
        "oracle_dispatch": [P, I32, P, I64, I64, P, I32, I32, I64, I64, P, I32, P, P, P, P, P, P],
        "oracle_dispatch_replay": [P, I32, P, I64, I64, P, I32, I64, P, I32, P],
        "oracle_combine": [P, I32, I64, I64, P, P, I64, I32, P, I32, P],
        "oracle_combine_fp8": [P, P, I64, I64, P, P, I64, I32, P, I32, P],
        "oracle_combine_fp4": [P, P, I64, I64, P, P, I64, I32, P, I32, P],
        "oracle_e2m1_encode": [P, I64, P],
        "oracle_e2m1_decode": [P, I64, P],
        "oracle_fp4_pack_rows": [P, I64, I64, P, P],
        "oracle_dedup_dispatch": [P, I32, I64, I64, P, I32, I32, I32, P, I64, P, P, P, P, I64,
                                  I64, P, P, P, P, P, P],
        "oracle_dedup_combine": [P, I32, I64, I64, P, P, P, I64, I32, I32, I32, P, I64, P, P,
                                 I32, P],
        "oracle_fp8_dequant": [P, P, I64, I64, P],
        "oracle_expert_scale": [P, I64, I32, P, P, P, P],
        "oracle_bf16_encode": [P, I64, P],
        "oracle_e4m3_encode": [P, I64, P],
        "oracle_e4m3_decode": [P, I64, P],
        "oracle_fp8_pack_rows": [P, I64, I64, P, P],
    }
    for name, argt in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = argt
        fn.restype = ctypes.c_int if not name.endswith(("encode", "decode", "pack_rows")) else None
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def set_threads(n: int) -> None:
    """Set the OpenMP thread count used by the copy / pack / combine loops."""
    _load()
    omp = ctypes.CDLL("libgomp.so.1")
    omp.omp_set_num_threads(ctypes.c_int(int(n)))


def get_threads() -> int:
    _load()
    omp = ctypes.CDLL("libgomp.so.1")
    omp.omp_get_max_threads.restype = ctypes.c_int
    return int(omp.omp_get_max_threads())


def route_count(idx: np.ndarray, E: int):
    """(cnt int32 [E], off int32 [E+1], stats int32 [3])."""
    idx = _c(idx, np.int32)
    T, K = idx.shape
    cnt = np.empty(E, np.int32)
    off = np.empty(E + 1, np.int32)
    stats = np.zeros(3, np.int32)
    _load().oracle_route_count(_p(idx), T, K, E, _p(cnt), _p(off), _p(stats))
    return cnt, off, stats


def _rows_needed(idx, E, cap):
    T, K = idx.shape
    return E * cap if cap > 0 else T * K


def dispatch(x: np.ndarray, x_dt: str, idx: np.ndarray, E: int, cap: int = 0,
             packed_rows: int | None = None, packed_dt: str | None = None,
             x_scales: np.ndarray | None = None) -> dict:
    """Plain dispatch.  x: uint16 bf16 bits, float32, or (x_dt "fp8") uint8 e4m3
    codes with x_scales f32 [T,H/128] [T,H].  Returns a dict of packed [rows,H]
    (poisoned where not written), scales f32 [rows,H/128] (fp8 only), packed_cnt
    [E], packed_off [E+1], packed_src [rows] (poisoned where not written),
    tok_map int64 [T,K], stats [3]."""
    idx = _c(idx, np.int32)
    T, K = idx.shape
    xd = DT[x_dt]
    pd = DT[packed_dt or x_dt]
    if pd != xd and not (_quantized(pd) and xd == BF16):
        raise ValueError("packed dtype must equal x dtype, or be fp8/fp4 from bf16")
    if (xd == FP8) != (x_scales is not None):
        raise ValueError("x_scales go with fp8 input, and only with it")
    xs = None if x_scales is None else _c(x_scales, np.float32)
    x = _c(x, NP_DT[xd])
    H = x.shape[1]
    rows = _rows_needed(idx, E, cap) if packed_rows is None else int(packed_rows)
    packed = np.full((rows, _row_width(pd, H)), POISON_BYTE, np.uint8).view(NP_DT[pd]) \
        if pd in (FP8, FP4) else \
        np.full((rows, H * (2 if pd == BF16 else 4)), POISON_BYTE, np.uint8).view(NP_DT[pd])
    scales = np.full((rows, H // 128 * 4), POISON_BYTE, np.uint8).view(np.float32) if _quantized(pd) else None
    packed_cnt = np.empty(E, np.int32)
    packed_off = np.empty(E + 1, np.int32)
    packed_src = np.full(rows, POISON_I32, np.int32)
    tok_map = np.empty((T, K), np.int64)
    stats = np.zeros(3, np.int32)
    _load().oracle_dispatch(_p(x), xd, _p(xs), T, H, _p(idx), K, E, cap, rows, _p(packed), pd,
                            _p(scales), _p(packed_cnt), _p(packed_off), _p(packed_src),
                            _p(tok_map), _p(stats))
    return dict(packed=packed, scales=scales, packed_cnt=packed_cnt, packed_off=packed_off,
                packed_src=packed_src, tok_map=tok_map, stats=stats)


def dispatch_replay(x: np.ndarray, x_dt: str, tok_map: np.ndarray, packed_rows: int,
                    packed_dt: str | None = None, x_scales: np.ndarray | None = None) -> dict:
    """Replay dispatch on a cached tok_map [T,K]: packed [rows,H] and (fp8)
    scales [rows,H/128], poisoned where not written."""
    tok_map = _c(tok_map, np.int64)
    T, K = tok_map.shape
    xd = DT[x_dt]
    pd = DT[packed_dt or x_dt]
    if pd != xd and not (_quantized(pd) and xd == BF16):
        raise ValueError("packed dtype must equal x dtype, or be fp8/fp4 from bf16")
    if (xd == FP8) != (x_scales is not None):
        raise ValueError("x_scales go with fp8 input, and only with it")
    xs = None if x_scales is None else _c(x_scales, np.float32)
    x = _c(x, NP_DT[xd])
    H = x.shape[1]
    rows = int(packed_rows)
    packed = np.full((rows, _row_width(pd, H)), POISON_BYTE, np.uint8).view(NP_DT[pd]) \
        if pd in (FP8, FP4) else \
        np.full((rows, H * (2 if pd == BF16 else 4)), POISON_BYTE, np.uint8).view(NP_DT[pd])
    scales = np.full((rows, H // 128 * 4), POISON_BYTE, np.uint8).view(np.float32) if _quantized(pd) else None
    _load().oracle_dispatch_replay(_p(x), xd, _p(xs), T, H, _p(tok_map), K, rows, _p(packed), pd,
                                   _p(scales))
    return dict(packed=packed, scales=scales)


def combine(y: np.ndarray, y_dt: str, tok_map: np.ndarray, w: np.ndarray, out_dt: str):
    """(out [T,H] bf16 bits or f32, out_weights f32 [T])."""
    yd, od = DT[y_dt], DT[out_dt]
    y = _c(y, NP_DT[yd])
    tok_map = _c(tok_map, np.int64)
    w = _c(w, np.float32)
    T, K = tok_map.shape
    y_rows, H = y.shape
    out = np.empty((T, H), NP_DT[od])
    ow = np.empty(T, np.float32)
    _load().oracle_combine(_p(y), yd, y_rows, H, _p(tok_map), _p(w), T, K, _p(out), od, _p(ow))
    return out, ow


def combine_fp8(q: np.ndarray, scales, tok_map: np.ndarray, w: np.ndarray, out_dt: str):
    """Combine of fp8 expert outputs: q uint8 [rows,H] e4m3 codes, scales f32
    [rows,H/128] or None (direct cast).  (out [T,H] bf16 bits or f32, out_weights [T])."""
    od = DT[out_dt]
    q = _c(q, np.uint8)
    sc = None if scales is None else _c(scales, np.float32)
    tok_map = _c(tok_map, np.int64)
    w = _c(w, np.float32)
    T, K = tok_map.shape
    y_rows, H = q.shape
    assert H % 128 == 0 and (sc is None or sc.shape == (y_rows, H // 128))
    out = np.empty((T, H), NP_DT[od])
    ow = np.empty(T, np.float32)
    _load().oracle_combine_fp8(_p(q), _p(sc), y_rows, H, _p(tok_map), _p(w), T, K, _p(out), od,
                               _p(ow))
    return out, ow


def combine_fp4(q: np.ndarray, scales, tok_map: np.ndarray, w: np.ndarray, out_dt: str):
    """Combine of fp4 expert outputs: q uint8 [rows,H/2] (two e2m1 codes per byte,
    element 2i in the low nibble), scales f32 [rows,H/128] or None."""
    od = DT[out_dt]
    q = _c(q, np.uint8)
    sc = None if scales is None else _c(scales, np.float32)
    tok_map = _c(tok_map, np.int64)
    w = _c(w, np.float32)
    T, K = tok_map.shape
    y_rows, Hh = q.shape
    H = 2 * Hh
    assert H % 128 == 0 and (sc is None or sc.shape == (y_rows, H // 128))
    out = np.empty((T, H), NP_DT[od])
    ow = np.empty(T, np.float32)
    _load().oracle_combine_fp4(_p(q), _p(sc), y_rows, H, _p(tok_map), _p(w), T, K, _p(out), od,
                               _p(ow))
    return out, ow


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """Encode values to e2m1 codes (0..15), round to nearest even, saturating at 6
    (infinities included); NaN gives code 0."""
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().oracle_e2m1_encode(_p(v), v.size, _p(out))
    return out


def e2m1_decode(c: np.ndarray) -> np.ndarray:
    c = _c(c, np.uint8)
    out = np.empty(c.shape, np.float32)
    _load().oracle_e2m1_decode(_p(c), c.size, _p(out))
    return out


def fp4_pack_rows(x_bf16: np.ndarray):
    """Blockwise fp4 pack of bf16 rows: (q uint8 [rows,H/2], s f32 [rows,H/128])."""
    x = _c(x_bf16, np.uint16)
    rows, H = x.shape
    q = np.empty((rows, H // 2), np.uint8)
    s = np.empty((rows, H // 128), np.float32)
    _load().oracle_fp4_pack_rows(_p(x), rows, H, _p(q), _p(s))
    return q, s


def dedup_dispatch(x: np.ndarray, x_dt: str, idx: np.ndarray, E: int, R: int,
                   recv_rows: int | None = None, cap: int = 0,
                   packed_rows: int | None = None) -> dict:
    """Dedup dispatch over R virtual ranks; returns the recv buffers and the
    same packed outputs as dispatch()."""
    idx = _c(idx, np.int32)
    T, K = idx.shape
    xd = DT[x_dt]
    x = _c(x, NP_DT[xd])
    H = x.shape[1]
    eb = 4 if xd == F32 else 2
    rr = T * min(K, R) if recv_rows is None else int(recv_rows)
    rows = _rows_needed(idx, E, cap) if packed_rows is None else int(packed_rows)
    recv_x = np.full((rr, H * eb), POISON_BYTE, np.uint8).view(NP_DT[xd])
    packed = np.full((rows, H * eb), POISON_BYTE, np.uint8).view(NP_DT[xd])
    recv_cnt = np.empty(R, np.int32)
    recv_off = np.empty(R + 1, np.int32)
    recv_src = np.full(rr, POISON_I32, np.int32)
    rank_slot = np.empty((T, R), np.int32)
    packed_cnt = np.empty(E, np.int32)
    packed_off = np.empty(E + 1, np.int32)
    packed_src = np.full(rows, POISON_I32, np.int32)
    tok_map = np.empty((T, K), np.int64)
    stats = np.zeros(3, np.int32)
    _load().oracle_dedup_dispatch(_p(x), xd, T, H, _p(idx), K, E, R, _p(recv_x), rr, _p(recv_cnt),
                                  _p(recv_off), _p(recv_src), _p(rank_slot), cap, rows,
                                  _p(packed), _p(packed_cnt), _p(packed_off), _p(packed_src),
                                  _p(tok_map), _p(stats))
    return dict(recv_x=recv_x, recv_cnt=recv_cnt, recv_off=recv_off, recv_src=recv_src,
                rank_slot=rank_slot, packed=packed, packed_cnt=packed_cnt, packed_off=packed_off,
                packed_src=packed_src, tok_map=tok_map, stats=stats)


def dedup_combine(y: np.ndarray, y_dt: str, tok_map: np.ndarray, w: np.ndarray, idx: np.ndarray,
                  E: int, R: int, rank_slot: np.ndarray, recv_rows: int, out_dt: str,
                  want_partial: bool = False):
    """(out, out_weights, partial or None)."""
    yd, od = DT[y_dt], DT[out_dt]
    y = _c(y, NP_DT[yd])
    tok_map = _c(tok_map, np.int64)
    w = _c(w, np.float32)
    idx = _c(idx, np.int32)
    rank_slot = _c(rank_slot, np.int32)
    T, K = tok_map.shape
    y_rows, H = y.shape
    out = np.empty((T, H), NP_DT[od])
    ow = np.empty(T, np.float32)
    partial = np.full((recv_rows, H * 4), POISON_BYTE, np.uint8).view(np.float32) \
        if want_partial else None
    _load().oracle_dedup_combine(_p(y), yd, y_rows, H, _p(tok_map), _p(w), _p(idx), T, K, E, R,
                                 _p(rank_slot), recv_rows, _p(partial), _p(out), od, _p(ow))
    return out, ow, partial


def fp8_dequant(q: np.ndarray, scales: np.ndarray) -> np.ndarray:
    q = _c(q, np.uint8)
    scales = _c(scales, np.float32)
    rows, H = q.shape
    y = np.empty((rows, H), np.uint16)
    _load().oracle_fp8_dequant(_p(q), _p(scales), rows, H, _p(y))
    return y


def expert_scale(packed: np.ndarray, packed_cnt: np.ndarray, packed_off: np.ndarray,
                 c: np.ndarray) -> np.ndarray:
    """Decode-workload expert stand-in: y = bf16(c_e * x) per packed row of expert e.
    Rows outside every expert segment are left zero."""
    packed = _c(packed, np.uint16)
    rows, H = packed.shape
    y = np.zeros((rows, H), np.uint16)
    E = len(packed_cnt)
    _load().oracle_expert_scale(_p(packed), H, E, _p(_c(packed_cnt, np.int32)),
                                _p(_c(packed_off, np.int32)), _p(_c(c, np.float32)), _p(y))
    return y


def bf16_encode(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_bf16_encode(_p(v), v.size, _p(out))
    return out


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Encode values to OCP e4m3fn bytes (round to nearest even; magnitudes above
    448, infinities included, saturate to +-448; NaN gives S.1111.111)."""
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().oracle_e4m3_encode(_p(v), v.size, _p(out))
    return out


def e4m3_decode(b: np.ndarray) -> np.ndarray:
    b = _c(b, np.uint8)
    out = np.empty(b.shape, np.float32)
    _load().oracle_e4m3_decode(_p(b), b.size, _p(out))
    return out


def fp8_pack_rows(x_bf16: np.ndarray):
    """Blockwise fp8 pack of bf16 rows: (q uint8 [rows,H], s f32 [rows,H/128])."""
    x = _c(x_bf16, np.uint16)
    rows, H = x.shape
    q = np.empty((rows, H), np.uint8)
    s = np.empty((rows, H // 128), np.float32)
    _load().oracle_fp8_pack_rows(_p(x), rows, H, _p(q), _p(s))
    return q, s
