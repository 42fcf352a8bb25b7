"""The C ABI from plain C: tests/abi_c_check.c includes include/moe_route.h as C11 (gcc), links
libmoe_route.so and checks the status codes of calls that fail validation, so no GPU is needed."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

PKG = os.path.join(ROOT, "combine_moe_route_03_amd")


def test_header_compiles_as_c_and_the_library_links(tmp_path):
    gcc = shutil.which("gcc")
    lib = os.path.join(PKG, "libmoe_route.so")
    if gcc is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("gcc or the ROCm headers are missing")
    assert os.path.exists(lib), "build the library first (__graft_entry__.build())"
    exe = str(tmp_path / "abi_c_check")
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-Werror=implicit-function-declaration",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "abi_c_check.c"), "-L", PKG, "-lmoe_route",
           f"-Wl,-rpath,{PKG}", "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "ok" in run.stdout
