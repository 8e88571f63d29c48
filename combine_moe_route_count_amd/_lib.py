"""ctypes binding of libmoe_route.so (argument marshalling only).

Every step of the path runs in the library's HIP kernels; this module only
turns torch tensors into pointers and sizes, allocates outputs the caller did
not pass, and raises MoeError on a non-OK status.  The library must be built
(python -m combine_moe_route_count_amd.build); loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_route.so")

MOE_BF16, MOE_F32, MOE_FP8_E4M3, MOE_FP4_E2M1 = 0, 1, 2, 3
MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int
_SZ = ctypes.c_size_t


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"moe status {status}: {msg}")
        self.status = status


class DedupPlan(ctypes.Structure):
    _fields_ = [("R", ctypes.c_int), ("idx", _P), ("rank_slot", _P), ("recv_rows", _I64),
                ("partial", _P)]


_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the library once (MOE_ROUTE_LIB overrides the in-tree path);
    raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("MOE_ROUTE_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m combine_moe_route_count_amd.build`")
    lib = ctypes.CDLL(path)
    lib.moe_version.restype = ctypes.c_int
    lib.moe_version.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_geometry.restype = ctypes.c_char_p
    lib.moe_geometry.argtypes = []
    lib.moe_workspace_size.restype = _SZ
    lib.moe_workspace_size.argtypes = [_I64, _I32, _I32, _I32]
    lib.moe_route_count.argtypes = [_P, _I64, _I32, _I32, _P, _P, _P, _P, _SZ, _P]
    lib.moe_dispatch.argtypes = [_P, _I32, _I64, _I64, _P, _I32, _I32, _I64, _I64, _P, _I32, _P,
                                 _P, _P, _P, _P, _P, _P, _SZ, _P]
    lib.moe_combine.argtypes = [_P, _I32, _I64, _I64, _P, _P, _I64, _I32, _I32,
                                ctypes.POINTER(DedupPlan), _P, _I32, _P, _P]
    lib.moe_dedup_dispatch.argtypes = [_P, _I32, _I64, _I64, _P, _I32, _I32, _I32, _P, _I64, _P,
                                       _P, _P, _P, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                       _P]
    lib.moe_fp8_dequant.argtypes = [_P, _P, _I64, _I64, _P, _P]
    lib.moe_copy16.argtypes = [_P, _P, _I64, _P]
    lib.moe_combine_fp8.argtypes = [_P, _P, _I64, _I64, _P, _P, _I64, _I32, _P, _I32, _P, _P]
    lib.moe_dispatch_prequant.argtypes = [_P, _P, _I64, _I64, _P, _I32, _I32, _I64, _I64, _P, _P,
                                          _P, _P, _P, _P, _P, _P, _SZ, _P]
    lib.moe_dispatch_replay.argtypes = [_P, _I32, _P, _I64, _I64, _P, _I32, _I64, _P, _I32, _P, _P]
    lib.moe_combine_fp4.argtypes = [_P, _P, _I64, _I64, _P, _P, _I64, _I32, _P, _I32, _P, _P]
    lib.moe_dispatch_noalloc.argtypes = [_P, _I32, _I64, _I64, _P, _I32, _I32, _I64, _I64, _P,
                                         _I32, _P, _P, _P, _P, _P, _P, _P]
    for fn in ("moe_route_count", "moe_dispatch", "moe_combine", "moe_dedup_dispatch",
               "moe_fp8_dequant", "moe_copy16", "moe_combine_fp8", "moe_dispatch_prequant",
               "moe_dispatch_replay", "moe_combine_fp4", "moe_dispatch_noalloc"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, load().moe_last_error().decode())


# The marshalling below runs on every call, and decode-sized calls take a few
# microseconds on the GPU: pointers go to ctypes as plain ints, and the current
# stream comes from torch's raw-handle query where it exists (the public
# Stream object costs about a microsecond more per call).
def ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device):
    if _raw_stream is not None:
        index = device.index if isinstance(device, torch.device) else None
        return _raw_stream(torch.cuda.current_device() if index is None else index)
    return torch.cuda.current_stream(device).cuda_stream


_DTYPE_CODES = {torch.bfloat16: MOE_BF16, torch.float32: MOE_F32, torch.uint8: MOE_FP8_E4M3,
                torch.float8_e4m3fn: MOE_FP8_E4M3}


def dtype_code(dt: torch.dtype) -> int:
    code = _DTYPE_CODES.get(dt)
    if code is None:
        raise ValueError(f"unsupported dtype {dt}")
    return code


def version() -> int:
    return load().moe_version()


def geometry() -> str:
    """The launch geometry in use ("key=value,..."; MOE_GEOM overrides it)."""
    return load().moe_geometry().decode()


def workspace_size(T: int, K: int, E: int, R: int = 0) -> int:
    return int(load().moe_workspace_size(T, K, E, R))


def workspace(T: int, K: int, E: int, R: int = 0, device="cuda") -> torch.Tensor:
    """A device workspace for these sizes (256-byte aligned, needs no initialisation)."""
    n = max(workspace_size(T, K, E, R), 1)
    buf = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + n]


def _ws(ws, T, K, E, R, device):
    return workspace(T, K, E, R, device) if ws is None else ws


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def route_count(idx: torch.Tensor, E: int, cnt=None, off=None, stats=None, ws=None):
    """cnt int32 [E], off int32 [E+1], stats int32 [3]."""
    T, K = idx.shape
    dev = idx.device
    cnt = torch.empty(E, dtype=torch.int32, device=dev) if cnt is None else cnt
    off = torch.empty(E + 1, dtype=torch.int32, device=dev) if off is None else off
    stats = torch.empty(3, dtype=torch.int32, device=dev) if stats is None else stats
    ws = _ws(ws, T, K, E, 0, dev)
    _check(load().moe_route_count(ptr(idx), T, K, E, ptr(cnt), ptr(off), ptr(stats), ptr(ws),
                                  ws.numel(), _stream(dev)))
    return cnt, off, stats


@dataclasses.dataclass
class DispatchOut:
    packed: torch.Tensor
    scales: Optional[torch.Tensor]
    packed_cnt: torch.Tensor
    packed_off: torch.Tensor
    packed_src: torch.Tensor
    tok_map: torch.Tensor
    stats: torch.Tensor


def alloc_dispatch(T, H, K, E, packed_rows, x_dtype, fp8, device, fp4=False) -> DispatchOut:
    """Output buffers of a dispatch; fp4 rows hold two e2m1 codes per byte."""
    q = fp8 or fp4
    pdt = torch.uint8 if q else x_dtype
    return DispatchOut(
        packed=torch.empty((packed_rows, H // 2 if fp4 else H), dtype=pdt, device=device),
        scales=torch.empty((packed_rows, H // 128), dtype=torch.float32, device=device) if q else None,
        packed_cnt=torch.empty(E, dtype=torch.int32, device=device),
        packed_off=torch.empty(E + 1, dtype=torch.int32, device=device),
        packed_src=torch.empty(packed_rows, dtype=torch.int32, device=device),
        tok_map=torch.empty((T, K), dtype=torch.int64, device=device),
        stats=torch.empty(3, dtype=torch.int32, device=device))


def dispatch(x: torch.Tensor, idx: torch.Tensor, E: int, cap: int = 0,
             packed_rows: Optional[int] = None, fp8: bool = False,
             out: Optional[DispatchOut] = None, ws=None, fp4: bool = False) -> DispatchOut:
    """Count, scan, slot and scatter x [T,H] (bf16 or f32) into per-expert rows.
    fp8=True packs bf16 to blockwise e4m3 with f32 scales per 128 elements;
    fp4=True to e2m1, two codes per byte, with the same scale blocks."""
    T, H = x.shape
    K = idx.shape[1]
    if packed_rows is None:
        packed_rows = E * cap if cap > 0 else T * K
    dev = x.device
    o = alloc_dispatch(T, H, K, E, packed_rows, x.dtype, fp8, dev, fp4) if out is None else out
    ws = _ws(ws, T, K, E, 0, dev)
    pdt = MOE_FP4_E2M1 if fp4 else (MOE_FP8_E4M3 if fp8 else dtype_code(x.dtype))
    _check(load().moe_dispatch(ptr(x), dtype_code(x.dtype), T, H, ptr(idx), K, E, cap,
                               packed_rows, ptr(o.packed), pdt, ptr(o.scales), ptr(o.packed_cnt),
                               ptr(o.packed_off), ptr(o.packed_src), ptr(o.tok_map), ptr(o.stats),
                               ptr(ws), ws.numel(), _stream(dev)))
    return o


def dispatch_noalloc(x: torch.Tensor, idx: torch.Tensor, E: int, cap: int = 0,
                     packed_rows: Optional[int] = None, fp8: bool = False,
                     out: Optional[DispatchOut] = None, fp4: bool = False) -> DispatchOut:
    """dispatch() through moe_dispatch_noalloc: no workspace argument; the
    library's static per-GPU workspace is used (out must be given by callers
    that cannot allocate)."""
    T, H = x.shape
    K = idx.shape[1]
    if packed_rows is None:
        packed_rows = E * cap if cap > 0 else T * K
    dev = x.device
    o = alloc_dispatch(T, H, K, E, packed_rows, x.dtype, fp8, dev, fp4) if out is None else out
    pdt = MOE_FP4_E2M1 if fp4 else (MOE_FP8_E4M3 if fp8 else dtype_code(x.dtype))
    _check(load().moe_dispatch_noalloc(ptr(x), dtype_code(x.dtype), T, H, ptr(idx), K, E, cap,
                                       packed_rows, ptr(o.packed), pdt, ptr(o.scales),
                                       ptr(o.packed_cnt), ptr(o.packed_off), ptr(o.packed_src),
                                       ptr(o.tok_map), ptr(o.stats), _stream(dev)))
    return o


def dispatch_prequant(x_q: torch.Tensor, x_scales: torch.Tensor, idx: torch.Tensor, E: int,
                      cap: int = 0, packed_rows: Optional[int] = None,
                      out: Optional[DispatchOut] = None, ws=None) -> DispatchOut:
    """Dispatch of pre-quantized input: x_q uint8 [T,H] e4m3 codes, x_scales f32
    [T,H/128]; codes and scale rows are forwarded unchanged."""
    T, H = x_q.shape
    K = idx.shape[1]
    if packed_rows is None:
        packed_rows = E * cap if cap > 0 else T * K
    dev = x_q.device
    o = alloc_dispatch(T, H, K, E, packed_rows, torch.uint8, True, dev) if out is None else out
    ws = _ws(ws, T, K, E, 0, dev)
    _check(load().moe_dispatch_prequant(ptr(x_q), ptr(x_scales), T, H, ptr(idx), K, E, cap,
                                        packed_rows, ptr(o.packed), ptr(o.scales),
                                        ptr(o.packed_cnt), ptr(o.packed_off), ptr(o.packed_src),
                                        ptr(o.tok_map), ptr(o.stats), ptr(ws), ws.numel(),
                                        _stream(dev)))
    return o


def dispatch_replay(x: torch.Tensor, tok_map: torch.Tensor, packed: torch.Tensor,
                    scales: Optional[torch.Tensor] = None,
                    x_scales: Optional[torch.Tensor] = None, fp4: bool = False) -> torch.Tensor:
    """Move the rows of x [T,H] into packed along a cached tok_map [T,K] (no
    routing).  packed uint8 with x bf16 packs to fp8 (fp4=True: e2m1, [rows,H/2])
    with scales out; x uint8 with x_scales is pre-quantized fp8 input."""
    T, H = x.shape
    K = tok_map.shape[1]
    dev = x.device
    x_dt = MOE_FP8_E4M3 if x.dtype == torch.uint8 else dtype_code(x.dtype)
    pdt = MOE_FP4_E2M1 if fp4 else (MOE_FP8_E4M3 if packed.dtype == torch.uint8
                                     else dtype_code(packed.dtype))
    _check(load().moe_dispatch_replay(ptr(x), x_dt, ptr(x_scales), T, H, ptr(tok_map), K,
                                      packed.shape[0], ptr(packed), pdt, ptr(scales),
                                      _stream(dev)))
    return packed


def combine(y: torch.Tensor, tok_map: torch.Tensor, w: torch.Tensor, E: int = 0,
            out_dtype: torch.dtype = torch.bfloat16, dedup: Optional[dict] = None,
            out: Optional[torch.Tensor] = None, out_weights: Optional[torch.Tensor] = None,
            want_weights: bool = True):
    """out [T,H] = sum_k w[t,k] * y[tok_map[t,k]] in f32, ascending k (or grouped
    per virtual rank when `dedup` = dict(R, idx, rank_slot, recv_rows[, partial]))."""
    y_rows, H = y.shape
    T, K = tok_map.shape
    dev = y.device
    out = torch.empty((T, H), dtype=out_dtype, device=dev) if out is None else out
    if want_weights and out_weights is None:
        out_weights = torch.empty(T, dtype=torch.float32, device=dev)
    plan = None
    if dedup is not None:
        plan = DedupPlan(int(dedup["R"]), dedup["idx"].data_ptr(), dedup["rank_slot"].data_ptr(),
                         int(dedup["recv_rows"]),
                         dedup["partial"].data_ptr() if dedup.get("partial") is not None else None)
    _check(load().moe_combine(ptr(y), dtype_code(y.dtype), y_rows, H, ptr(tok_map), ptr(w), T, K,
                              E, ctypes.byref(plan) if plan is not None else None, ptr(out),
                              dtype_code(out.dtype), ptr(out_weights), _stream(dev)))
    return out, out_weights


def combine_fp8(q: torch.Tensor, scales: Optional[torch.Tensor], tok_map: torch.Tensor,
                w: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                out: Optional[torch.Tensor] = None, out_weights: Optional[torch.Tensor] = None,
                want_weights: bool = True):
    """Combine of fp8 expert outputs: q uint8 [rows,H] e4m3 codes, scales f32
    [rows,H/128] or None (direct cast); out [T,H] = sum_k w * (f32(q) * s)."""
    y_rows, H = q.shape
    T, K = tok_map.shape
    dev = q.device
    out = torch.empty((T, H), dtype=out_dtype, device=dev) if out is None else out
    if want_weights and out_weights is None:
        out_weights = torch.empty(T, dtype=torch.float32, device=dev)
    _check(load().moe_combine_fp8(ptr(q), ptr(scales), y_rows, H, ptr(tok_map), ptr(w), T, K,
                                  ptr(out), dtype_code(out.dtype), ptr(out_weights), _stream(dev)))
    return out, out_weights


def combine_fp4(q: torch.Tensor, scales: Optional[torch.Tensor], tok_map: torch.Tensor,
                w: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                out: Optional[torch.Tensor] = None, out_weights: Optional[torch.Tensor] = None,
                want_weights: bool = True):
    """Combine of fp4 expert outputs: q uint8 [rows,H/2] (two e2m1 codes per
    byte), scales f32 [rows,H/128] or None; out [T,H] = sum_k w * (f32(q) * s)."""
    y_rows, Hh = q.shape
    H = 2 * Hh
    T, K = tok_map.shape
    dev = q.device
    out = torch.empty((T, H), dtype=out_dtype, device=dev) if out is None else out
    if want_weights and out_weights is None:
        out_weights = torch.empty(T, dtype=torch.float32, device=dev)
    _check(load().moe_combine_fp4(ptr(q), ptr(scales), y_rows, H, ptr(tok_map), ptr(w), T, K,
                                  ptr(out), dtype_code(out.dtype), ptr(out_weights), _stream(dev)))
    return out, out_weights


@dataclasses.dataclass
class DedupOut:
    recv_x: torch.Tensor
    recv_cnt: torch.Tensor
    recv_off: torch.Tensor
    recv_src: torch.Tensor
    rank_slot: torch.Tensor
    packed: torch.Tensor
    packed_cnt: torch.Tensor
    packed_off: torch.Tensor
    packed_src: torch.Tensor
    tok_map: torch.Tensor
    stats: torch.Tensor


def alloc_dedup(T, H, K, E, R, recv_rows, packed_rows, dtype, device) -> DedupOut:
    return DedupOut(
        recv_x=torch.empty((recv_rows, H), dtype=dtype, device=device),
        recv_cnt=torch.empty(R, dtype=torch.int32, device=device),
        recv_off=torch.empty(R + 1, dtype=torch.int32, device=device),
        recv_src=torch.empty(recv_rows, dtype=torch.int32, device=device),
        rank_slot=torch.empty((T, R), dtype=torch.int32, device=device),
        packed=torch.empty((packed_rows, H), dtype=dtype, device=device),
        packed_cnt=torch.empty(E, dtype=torch.int32, device=device),
        packed_off=torch.empty(E + 1, dtype=torch.int32, device=device),
        packed_src=torch.empty(packed_rows, dtype=torch.int32, device=device),
        tok_map=torch.empty((T, K), dtype=torch.int64, device=device),
        stats=torch.empty(3, dtype=torch.int32, device=device))


def dedup_dispatch(x: torch.Tensor, idx: torch.Tensor, E: int, R: int,
                   recv_rows: Optional[int] = None, cap: int = 0,
                   packed_rows: Optional[int] = None, out: Optional[DedupOut] = None,
                   ws=None) -> DedupOut:
    """One row copy per unique (token, virtual rank), then local expansion."""
    T, H = x.shape
    K = idx.shape[1]
    if recv_rows is None:
        recv_rows = T * min(K, R)
    if packed_rows is None:
        packed_rows = E * cap if cap > 0 else T * K
    dev = x.device
    o = alloc_dedup(T, H, K, E, R, recv_rows, packed_rows, x.dtype, dev) if out is None else out
    ws = _ws(ws, T, K, E, R, dev)
    _check(load().moe_dedup_dispatch(
        ptr(x), dtype_code(x.dtype), T, H, ptr(idx), K, E, R, ptr(o.recv_x), recv_rows,
        ptr(o.recv_cnt), ptr(o.recv_off), ptr(o.recv_src), ptr(o.rank_slot), cap, packed_rows,
        ptr(o.packed), ptr(o.packed_cnt), ptr(o.packed_off), ptr(o.packed_src), ptr(o.tok_map),
        ptr(o.stats), ptr(ws), ws.numel(), _stream(dev)))
    return o


def fp8_dequant(q: torch.Tensor, scales: torch.Tensor, y: Optional[torch.Tensor] = None):
    """y = bf16(f32(q) * scale of its 128-element block)."""
    rows, H = q.shape
    y = torch.empty((rows, H), dtype=torch.bfloat16, device=q.device) if y is None else y
    _check(load().moe_fp8_dequant(ptr(q), ptr(scales), rows, H, ptr(y), _stream(q.device)))
    return y


def copy16(src: torch.Tensor, dst: torch.Tensor) -> torch.Tensor:
    """dst <- src bytes with the library's 16-byte streaming copy (the copy ceiling)."""
    n = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() >= n
    _check(load().moe_copy16(ptr(src), ptr(dst), n, _stream(src.device)))
    return dst
