"""A plain C11 program (tests/c_abi_run.c) runs the kernels through the C ABI
alone: hipMalloc'd buffers, ln_fwd, bias_dropout_residual_ln_fwd with the
mask written out, ln_bwd_dx with its partials and ln_bwd_dgamma_dbeta on the
ready partials.  It writes its inputs and outputs to a file; here they are
checked against the float64 oracle (the mask bit for bit)."""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import memory_bound_row_amd as mb
from gpu_helpers import FMT, case, check_bwd, check_fused, check_fwd

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def c_program(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    mb.lib()
    exe = str(tmp_path_factory.mktemp("c_abi") / "c_abi_run")
    libdir = os.path.dirname(mb.LIB_PATH)
    cmd = ["gcc", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "c_abi_run.c"), "-L", libdir, "-lmbrow_ln",
           "-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath," + libdir,
           "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("rows,cols,seed", [(64, 768, 1), (37, 1001, 2), (300, 4104, 3)])
def test_plain_c_caller_runs_the_kernels(orc, c_program, tmp_path, rows, cols, seed):
    case(f"plain C caller fp32 {rows}x{cols}")
    out = str(tmp_path / "out.bin")
    r = subprocess.run([c_program, str(rows), str(cols), str(seed), out], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    raw = open(out, "rb").read()
    n, c = rows * cols, cols
    sizes = [n, n, n, c, c, c, n, rows, rows, n, n, rows, rows, n, c, c]
    f = np.frombuffer(raw[:4 * sum(sizes)], dtype=np.float32)
    parts, o = [], 0
    for k in sizes:
        parts.append(torch.from_numpy(f[o:o + k].copy()))
        o += k
    mask = torch.from_numpy(np.frombuffer(raw[4 * sum(sizes):], dtype=np.uint8).copy())
    assert mask.numel() == n
    x, res, dy, g, b, bias, y, mean, rstd, z, y2, mean2, rstd2, dx, dg, db = parts
    x, res, dy, y, z, y2, dx = (t.view(rows, cols) for t in (x, res, dy, y, z, y2, dx))
    fmt = FMT[torch.float32]
    check_fwd(orc, x, g, b, y, mean, rstd, fmt, name="c.fwd")
    inp = {"x": x, "bias": bias, "residual": res, "gamma": g, "beta": b}
    check_fused(orc, inp, 0.1, 12345, z, y2, mean2, rstd2, mask.view(rows, cols), fmt,
                name="c.fused")
    check_bwd(orc, dy, x, g, mean, rstd, dx, dg, db, fmt, name="c.bwd")
