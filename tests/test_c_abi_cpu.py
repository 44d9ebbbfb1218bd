"""The library from plain C: tests/c_abi_check.c is compiled with gcc against
include/bi.h only (no HIP compiler, no torch) and linked to libbi.so, then run;
it exercises validation, status strings, workspace sizes and the plan, none of
which reach a GPU."""
import os
import shutil
import subprocess

import pytest

import deterministic_invariant_gemm_amd as dig

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_c_caller(tmp_path):
    if not os.path.exists(dig.LIB_PATH):
        pytest.skip("libbi.so is not built")
    exe = tmp_path / "c_abi_check"
    libdir = os.path.dirname(dig.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "c_abi_check.c"), "-o", str(exe),
           "-L", libdir, "-lbi", f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi ok" in r.stdout
