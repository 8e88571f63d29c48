"""moe_dispatch_noalloc (the routing workspace is the library's static per-GPU
array) against moe_dispatch (the caller's workspace) through the C ABI: every
output bitwise equal, on two calls in a row with the second one smaller, for
each payload, for the one-launch and the two-launch routing, and at the
largest size the static workspace holds."""
import numpy as np
import pytest
import torch

import combine_moe_route_count_amd as moe
import workloads as W
from _gpu_util import DEV, dev, dev_bf16, host, note, poison_

pytestmark = pytest.mark.gpu


def _idx(rng, T, K, E):
    idx = rng.integers(0, E, size=(T, K)).astype(np.int32)
    idx[rng.random((T, K)) < 0.03] = -1
    return idx


def _both(x, idx_np, E, cap, rows, fp8, fp4):
    T, H = x.shape
    K = idx_np.shape[1]
    outs = []
    for fn in ("dispatch", "dispatch_noalloc"):
        o = moe._lib.alloc_dispatch(T, H, K, E, rows, x.dtype, fp8, DEV, fp4=fp4)
        for t in (o.packed, o.scales, o.packed_src, o.tok_map, o.packed_cnt, o.packed_off,
                  o.stats):
            poison_(t)
        getattr(moe, fn)(x, dev(idx_np), E, cap=cap, packed_rows=rows, fp8=fp8, fp4=fp4, out=o)
        outs.append(o)
    torch.cuda.synchronize()
    a, b = outs
    for name in ("tok_map", "packed_cnt", "packed_off", "packed_src", "stats", "packed"):
        ga, gb = host(getattr(a, name)), host(getattr(b, name))
        assert np.array_equal(ga.view(np.uint8), gb.view(np.uint8)), name
    if a.scales is not None:
        assert np.array_equal(host(a.scales).view(np.uint32), host(b.scales).view(np.uint32))
    return a


# (payload, first T, second T, K, E, H, layout): the second call is smaller; T*K
# <= 1024 takes the one-launch dispatch, larger sizes the two-launch routing
CASES = [
    ("bf16", 3000, 1100, 8, 256, 512, "compact"),
    ("bf16", 2000, 40, 4, 64, 256, "padded"),
    ("f32", 1500, 700, 6, 32, 128, "compact"),
    ("fp8", 2500, 300, 8, 256, 1024, "compact"),
    ("fp8", 900, 100, 8, 128, 7168, "padded"),
    ("fp4", 2100, 257, 8, 256, 512, "compact"),
]


@pytest.mark.parametrize("payload,T1,T2,K,E,H,layout", CASES)
def test_noalloc_equals_dispatch_twice(payload, T1, T2, K, E, H, layout):
    rng = np.random.default_rng(T1 + T2 + K + H)
    for T in (T1, T2):
        idx = _idx(rng, T, K, E)
        dt = "f32" if payload == "f32" else "bf16"
        xs = W.normal_x(rng, T, H, dt)
        x = dev(xs.astype(np.float32)) if dt == "f32" else dev_bf16(xs)
        flat = idx.ravel()
        cnt = np.bincount(flat[flat >= 0], minlength=E)
        cap = int(cnt.max()) if layout == "padded" else 0
        rows = E * cap if cap else T * K
        note(f"noalloc {payload} T={T} K={K} E={E} H={H} {layout}")
        _both(x, idx, E, cap, rows, payload == "fp8", payload == "fp4")


def test_noalloc_at_the_static_workspace_limit():
    """T*K = 837120 entries at E = 256: the largest routing the 4 MiB array
    holds; then a small call again."""
    rng = np.random.default_rng(5)
    for T, K, E, H in [(104640, 8, 256, 64), (33, 8, 256, 64)]:
        assert moe.workspace_size(T, K, E) <= 4 << 20
        idx = _idx(rng, T, K, E)
        x = dev_bf16(W.normal_x(rng, T, H, "bf16"))
        note(f"noalloc limit T={T} K={K} E={E} H={H}")
        _both(x, idx, E, 0, T * K, False, False)
    assert moe.workspace_size(104641, 8, 256) > 4 << 20


def test_noalloc_dispatch_captured_in_a_graph():
    """The callers it is for include code under graph capture: a captured
    moe_dispatch_noalloc, replayed three times with eager calls on other
    inputs in between, writes what moe_dispatch writes on the same input."""
    rng = np.random.default_rng(9)
    T, K, E, H = 1500, 8, 64, 512
    idx_a, idx_b = _idx(rng, T, K, E), _idx(rng, 700, K, E)
    xa = dev_bf16(W.normal_x(rng, T, H, "bf16"))
    xb = dev_bf16(W.normal_x(rng, 700, H, "bf16"))
    ia, ib = dev(idx_a), dev(idx_b)
    # rows past the valid entries are never written: both outputs start poisoned
    ref = moe._lib.alloc_dispatch(T, H, K, E, T * K, xa.dtype, True, DEV)
    for t in (ref.packed, ref.scales, ref.packed_src, ref.tok_map, ref.packed_cnt, ref.packed_off,
              ref.stats):
        poison_(t)
    moe.dispatch(xa, ia, E, fp8=True, out=ref)
    o = moe._lib.alloc_dispatch(T, H, K, E, T * K, xa.dtype, True, DEV)
    moe.dispatch_noalloc(xa, ia, E, fp8=True, out=o)      # the first call on the device, eager
    torch.cuda.synchronize()
    note("noalloc graph capture")
    cs = torch.cuda.Stream(DEV)
    cs.wait_stream(torch.cuda.current_stream(DEV))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            moe.dispatch_noalloc(xa, ia, E, fp8=True, out=o)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (o.packed, o.scales, o.packed_src, o.tok_map, o.packed_cnt, o.packed_off, o.stats):
            poison_(t)
        g.replay()
        torch.cuda.synchronize()
        for name in ("tok_map", "packed_cnt", "packed_off", "packed_src", "stats", "packed"):
            assert torch.equal(getattr(o, name), getattr(ref, name)), (rep, name)
        assert torch.equal(o.scales.view(torch.int32), ref.scales.view(torch.int32)), rep
        moe.dispatch_noalloc(xb, ib, E, fp8=True)          # eager work on the same array between replays
        torch.cuda.synchronize()


def test_noalloc_from_two_host_threads_on_one_stream():
    """Two host threads share the static array through one stream: the library
    enqueues each call's launches as one unit, so the stream orders whole calls
    and each thread's outputs equal moe_dispatch of its own input (without that,
    one call's scatter could run after the other call's routing had replaced
    its routing results in the array)."""
    import threading
    rng = np.random.default_rng(21)
    K, E, H = 8, 128, 256
    work = []
    for T in (1800, 90):     # a multi-tile and a one-launch dispatch
        idx = _idx(rng, T, K, E)
        x = dev_bf16(W.normal_x(rng, T, H, "bf16"))
        ref = moe._lib.alloc_dispatch(T, H, K, E, T * K, x.dtype, True, DEV)
        o = moe._lib.alloc_dispatch(T, H, K, E, T * K, x.dtype, True, DEV)
        for t in (ref.packed, ref.scales, ref.packed_src, ref.tok_map, ref.packed_cnt,
                  ref.packed_off, ref.stats, o.packed, o.scales, o.packed_src, o.tok_map,
                  o.packed_cnt, o.packed_off, o.stats):
            poison_(t)
        i = dev(idx)
        moe.dispatch(x, i, E, fp8=True, out=ref)
        work.append((x, i, o, ref))
    torch.cuda.synchronize()
    note("noalloc two host threads, one stream")
    errors = []

    shared = torch.cuda.Stream(DEV)
    shared.wait_stream(torch.cuda.current_stream(DEV))

    def run(x, i, o):
        try:
            torch.cuda.set_device(0)
            with torch.cuda.stream(shared):
                for _ in range(20):
                    moe.dispatch_noalloc(x, i, E, fp8=True, out=o)
        except Exception as e:   # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=run, args=(x, i, o)) for x, i, o, _ in work]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads) and not errors, errors
    torch.cuda.synchronize()
    for _, _, o, ref in work:
        for name in ("tok_map", "packed_cnt", "packed_off", "packed_src", "stats", "packed"):
            assert torch.equal(getattr(o, name), getattr(ref, name)), name
        assert torch.equal(o.scales.view(torch.int32), ref.scales.view(torch.int32))
