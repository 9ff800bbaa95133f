"""The library's host code (argument validation, shape rules, workspace
layouts) built with g++ under the address and undefined-behaviour
sanitizers and run without a GPU: tests/host/host_check.cpp stands in for
the kernel launchers, records what each call would hand to its kernel and
checks it -- grids that cover every row, splits and chunk counts the
kernels are built for, 32-bit buffer offsets below 2^31 at their edges,
workspace and no-allocation scratch regions in bounds and disjoint."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "vector_quantized_decode_amd", "csrc")
HIP_INCLUDE = "/opt/rocm/include"


def test_host_code_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(HIP_INCLUDE):
        pytest.skip("g++ or the HIP headers are not available")
    exe = str(tmp_path / "host_check")
    build = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE, "-I", os.path.join(ROOT, "include"),
             os.path.join(CSRC, "vq_api.cpp"), os.path.join(CSRC, "vq_shapes.cpp"),
             os.path.join(ROOT, "tests", "host", "host_check.cpp"), "-o", exe]
    r = subprocess.run(build, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "host checks passed" in r.stdout
