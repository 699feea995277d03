"""The boundary is a C ABI: a plain C11 program (tests/c_abi_check.c)
compiles against include/mbrow_ln.h with gcc, links against the library and
gets the documented status codes back from host-side validation (CPU only:
nothing it calls reaches a GPU)."""
import os
import shutil
import subprocess

import pytest

import memory_bound_row_amd as mb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_program_compiles_links_and_validates(tmp_path):
    mb.lib()   # the library is built
    exe = tmp_path / "c_abi_check"
    libdir = os.path.dirname(mb.LIB_PATH)
    cmd = ["gcc", "-std=c11", "-Wall", "-Werror=implicit-function-declaration",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", os.path.join(ROOT, "tests", "c_abi_check.c"),
           "-L", libdir, "-lmbrow_ln", "-Wl,-rpath," + libdir, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("OK")
