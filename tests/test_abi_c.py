"""The header is usable from C and C++: tests/abi_check.c compiles against
include/gtattn.h with gcc (C11) and g++ (C++17), links libgtattn.so and checks
argument rejections that return before any device work (CPU only)."""
import os
import shutil
import subprocess

import pytest

import sparse_graph_attention_amd as gt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.parametrize("compiler,flags", [("gcc", ["-std=c11", "-x", "c"]), ("g++", ["-std=c++17", "-x", "c++"])])
def test_c_caller(tmp_path, compiler, flags):
    if shutil.which(compiler) is None:
        pytest.skip("%s not installed" % compiler)
    gt.lib()  # builds the library if it is missing
    libdir = os.path.dirname(gt._build.LIB)
    exe = str(tmp_path / "abi_check")
    cmd = [compiler, *flags, "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), os.path.join(ROOT, "tests", "abi_check.c"), "-x", "none",
           "-o", exe, "-L", libdir, "-lgtattn", "-Wl,-rpath," + libdir]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
