"""Build libmoe_route.so for gfx950 with hipcc (in-tree, no JIT cache).

python -m combine_moe_route_count_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe_route.so")

SOURCES = ["api.cpp", "geometry.cpp", "route.hip", "scatter.hip", "combine.hip", "route_fused.hip",
           "scratch.hip"]
HEADERS = ["device_common.hpp", "internal.hpp", "route_device.hpp", "rows_device.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -ffp-contract=off: every multiply and add is rounded separately (the combine
# order contract).  Packed fp32 ALU ops are disabled for the device code.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libmoe_route.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


C_SMOKE_SRC = os.path.join(ROOT, "tests", "c_abi_smoke.c")
C_SMOKE_BIN = os.path.join(ROOT, "tests", "c_abi_smoke")


def build_c_abi_smoke(verbose: bool = False) -> str:
    """Compile the plain-C user of the ABI (tests/c_abi_smoke.c) against the
    built library, with gcc: no HIP device code, only the runtime's C API."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    cmd = ["gcc", "-std=gnu99", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           C_SMOKE_SRC, "-o", C_SMOKE_BIN, "-L", HERE, "-lmoe_route",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../combine_moe_route_count_amd",
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed for {C_SMOKE_SRC}:\n{r.stdout}\n{r.stderr}")
    return C_SMOKE_BIN


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
