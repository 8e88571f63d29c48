"""The host side of the C ABI (api.cpp: argument checks, workspace carving,
launch sequencing) built with AddressSanitizer and UndefinedBehaviorSanitizer
and linked with the device objects of the normal build, then put through the
host-only ABI tests in a child process.  No GPU is touched: those tests call
only the paths that fail or return before any launch."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CLANG = "/opt/rocm/llvm/bin/clang++"
DEVICE_OBJECTS = ["route.hip.o", "scatter.hip.o", "combine.hip.o", "route_fused.hip.o",
                  "scratch.hip.o", "geometry.cpp.o"]


def test_abi_host_code_under_asan_ubsan(tmp_path):
    objs = [os.path.join(ROOT, "_build", o) for o in DEVICE_OBJECTS]
    if not os.path.exists(CLANG) or not all(os.path.exists(o) for o in objs):
        pytest.skip("needs the ROCm clang and the objects of a prior build()")
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("clang sanitizer runtime not installed")
    rocm = os.path.dirname(os.path.dirname(os.path.dirname(CLANG)))
    api_o = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libmoe_route_san.so")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    subprocess.run([CLANG, "-O1", "-g", "-std=c++17", "-fPIC", "-fvisibility=hidden", *san,
                    "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
                    "-c", os.path.join(ROOT, "combine_moe_route_count_amd", "csrc", "api.cpp"),
                    "-o", api_o], check=True)
    subprocess.run([CLANG, "-shared", "-fPIC", *san, "-shared-libsan", "-o", lib, api_o, *objs,
                    "-L", os.path.join(rocm, "lib"), "-lamdhip64",
                    "-Wl,-rpath," + os.path.join(rocm, "lib")], check=True)
    env = dict(os.environ, MOE_ROUTE_LIB=lib, LD_PRELOAD=rt,
               LD_LIBRARY_PATH=os.path.dirname(rt) + ":" + os.environ.get("LD_LIBRARY_PATH", ""),
               ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_abi_host.py"),
                        "-q", "-p", "no:cacheprovider"], env=env, capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "runtime error" not in out and "AddressSanitizer" not in out, \
        out[-4000:]
