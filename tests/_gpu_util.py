"""Helpers shared by the GPU parity tests: host <-> device conversion, output
poisoning, and a runner that calls the HIP library and the oracle on the same
seeded inputs."""
import sys

import numpy as np
import torch

import combine_moe_route_count_amd as moe
import oracle

DEV = "cuda"


def note(msg: str) -> None:
    """Name the case on stdout before a GPU step, so a crash can be placed."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def dev_x(x: np.ndarray, dtype: str) -> torch.Tensor:
    return dev_bf16(x) if dtype == "bf16" else dev(x.astype(np.float32))


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def poison_(t) -> None:
    if t is None:
        return
    if t.dtype in (torch.int32, torch.int64):
        t.fill_(oracle.POISON_I32)
    else:
        t.view(torch.uint8).fill_(oracle.POISON_BYTE)


def gpu_dispatch(x_dev, idx_np, E, cap=0, packed_rows=None, fp8=False, fp4=False):
    T, H = x_dev.shape
    K = idx_np.shape[1]
    if packed_rows is None:
        packed_rows = E * cap if cap > 0 else T * K
    o = moe._lib.alloc_dispatch(T, H, K, E, packed_rows, x_dev.dtype, fp8, DEV, fp4=fp4)
    for t in (o.packed, o.scales, o.packed_src, o.tok_map, o.packed_cnt, o.packed_off, o.stats):
        poison_(t)
    moe.dispatch(x_dev, dev(idx_np.astype(np.int32)), E, cap=cap, packed_rows=packed_rows,
                 fp8=fp8, out=o, fp4=fp4)
    torch.cuda.synchronize()
    return o


def assert_dispatch_equal(o, ref, fp8=False, check_rows=True):
    np.testing.assert_array_equal(host(o.tok_map), ref["tok_map"], err_msg="tok_map")
    np.testing.assert_array_equal(host(o.packed_cnt), ref["packed_cnt"], err_msg="packed_cnt")
    np.testing.assert_array_equal(host(o.packed_off), ref["packed_off"], err_msg="packed_off")
    np.testing.assert_array_equal(host(o.packed_src), ref["packed_src"], err_msg="packed_src")
    np.testing.assert_array_equal(host(o.stats), ref["stats"], err_msg="stats")
    if check_rows:
        got = host(o.packed).view(np.uint8)
        exp = ref["packed"].view(np.uint8)
        if not np.array_equal(got, exp):
            bad = np.nonzero(np.any(got != exp, axis=1))[0]
            raise AssertionError(f"packed rows differ: {len(bad)} rows, first {bad[:8]}")
        if fp8:
            np.testing.assert_array_equal(host(o.scales).view(np.uint32),
                                          ref["scales"].view(np.uint32), err_msg="scales")


def bf16_ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in representable bf16 steps (monotone integer mapping of the bits)."""
    def key(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)
    return np.abs(key(a_bits) - key(b_bits))
