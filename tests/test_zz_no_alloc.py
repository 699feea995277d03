"""ln_bwd_noalloc, the backward for callers that cannot allocate: its column
partials live in the library's static device scratch.  Checked through the C
ABI against the existing workspace path (ln_bwd_dx with a workspace, then the
fold), bit for bit since the kernels are shared, and against the float64
oracle; two calls in a row, the second on a smaller input, so that the
scratch's leftover contents from the first call cannot leak into the second.
Runs alone in a fresh process and after every other test."""
import numpy as np
import pytest
import torch

import memory_bound_row_amd as mb
from memory_bound_row_amd import synth
from gpu_helpers import EPS, FMT, case, check_bwd, dev

pytestmark = pytest.mark.gpu


def _inputs(rows, cols, dtype, seed):
    inp = dev(synth.layer_inputs(rows, cols, dtype, seed=seed,
                                 names=("x", "gamma", "beta", "dy")))
    _, mean, rstd = mb.ln_fwd(inp["x"], inp["gamma"], inp["beta"], EPS)
    return inp, mean, rstd


def _noalloc(inp, mean, rstd):
    rows, cols = inp["x"].shape
    dx = torch.empty_like(inp["x"])
    dg = torch.empty(cols, dtype=torch.float32, device="cuda")
    db = torch.empty(cols, dtype=torch.float32, device="cuda")
    mb.ln_bwd_noalloc(inp["dy"], inp["x"], inp["gamma"], mean, rstd, dx=dx, dgamma=dg, dbeta=db)
    return dx, dg, db


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_noalloc_matches_workspace_path_twice(orc, dtype):
    shapes = [(8192, 1280), (300, 1000)]          # the second call is smaller
    for i, (rows, cols) in enumerate(shapes):
        case(f"ln_bwd_noalloc call {i} {dtype} {rows}x{cols}")
        inp, mean, rstd = _inputs(rows, cols, dtype, seed=40 + i)
        got = _noalloc(inp, mean, rstd)
        want = mb.ln_bwd(inp["dy"], inp["x"], inp["gamma"], mean, rstd)
        torch.cuda.synchronize()
        for name, a, b in zip(("dx", "dgamma", "dbeta"), got, want):
            assert torch.equal(a, b), f"{name} differs from the workspace path ({rows}x{cols})"
        check_bwd(orc, inp["dy"], inp["x"], inp["gamma"], mean, rstd, *got, FMT[dtype],
                  name=f"noalloc.{i}")


def test_noalloc_rejects_shapes_beyond_the_scratch():
    case("ln_bwd_noalloc beyond its scratch")
    rows, cols = 512, 16384                       # 256 partitions x 2 x 16384 x 4 B = 32 MiB
    assert mb.ln_bwd_workspace_bytes(rows, cols) > mb.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((rows, cols), dtype=torch.bfloat16, device="cuda")
    g = torch.ones(cols, dtype=torch.bfloat16, device="cuda")
    st = torch.zeros(rows, dtype=torch.float32, device="cuda")
    dx = torch.full_like(x, 7.0)
    dg = torch.full((cols,), 7.0, dtype=torch.float32, device="cuda")
    db = torch.full((cols,), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError, match="LN_ERR_SCRATCH"):
        mb.ln_bwd_noalloc(x, x, g, st, st, dx=dx, dgamma=dg, dbeta=db)
    torch.cuda.synchronize()
    assert torch.all(dx == 7.0) and torch.all(dg == 7.0) and torch.all(db == 7.0)
