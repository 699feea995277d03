"""GPU properties beyond parity: run-to-run bit reproducibility, fused vs
standalone partials, compositions of the calls, in-place and unaligned
buffers, guard bands around outputs, and HIP-graph replay."""
import numpy as np
import pytest
import torch

import memory_bound_row_amd as mb
from memory_bound_row_amd import synth

from gpu_helpers import EPS, FMT, case, check_bwd, check_fwd, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _default_path():
    mb.debug_force_path(0)
    yield
    mb.debug_force_path(0)


def test_determinism_config3_100_runs():
    case("determinism ln_bwd bf16 16384x1024 x100")
    inp = dev(synth.layer_inputs(16384, 1024, torch.bfloat16, seed=0,
                                 names=("x", "gamma", "beta", "dy")))
    y, mean, rstd = mb.ln_fwd(inp["x"], inp["gamma"], inp["beta"], EPS)
    ws = mb.workspace(16384, 1024, "cuda")
    dx0, dg0, db0 = [t.clone() for t in mb.ln_bwd(inp["dy"], inp["x"], inp["gamma"], mean, rstd,
                                                   workspace_buf=ws)]
    y0, m0, r0 = y.clone(), mean.clone(), rstd.clone()
    for _ in range(100):
        y, mean, rstd = mb.ln_fwd(inp["x"], inp["gamma"], inp["beta"], EPS, y=y, mean=mean,
                                  rstd=rstd)
        dx, dg, db = mb.ln_bwd(inp["dy"], inp["x"], inp["gamma"], mean, rstd, workspace_buf=ws)
        torch.cuda.synchronize()
        assert torch.equal(dg, dg0) and torch.equal(db, db0)
        assert torch.equal(dx, dx0) and torch.equal(y, y0)
        assert torch.equal(mean, m0) and torch.equal(rstd, r0)


@pytest.mark.parametrize("dtype,rows,cols", [(torch.bfloat16, 8192, 1280),
                                              (torch.float32, 4096, 16384),
                                              (torch.float16, 1000, 999)])
def test_fused_and_standalone_partials_identical(dtype, rows, cols):
    case(f"partials fused vs standalone {dtype} {rows}x{cols}")
    inp = dev(synth.layer_inputs(rows, cols, dtype, seed=1, names=("x", "gamma", "beta", "dy")))
    y, mean, rstd = mb.ln_fwd(inp["x"], inp["gamma"], inp["beta"], EPS)
    ws1 = mb.workspace(rows, cols, "cuda")
    ws2 = mb.workspace(rows, cols, "cuda")
    mb.ln_bwd_dx(inp["dy"], inp["x"], inp["gamma"], mean, rstd, workspace=ws1)
    g1, b1 = mb.ln_bwd_dgamma_dbeta(ws1, rows, cols, dtype, partials_ready=True)
    g2, b2 = mb.ln_bwd_dgamma_dbeta(ws2, rows, cols, dtype, partials_ready=False,
                                    dy=inp["dy"], x=inp["x"], mean=mean, rstd=rstd)
    torch.cuda.synchronize()
    assert torch.equal(ws1, ws2)
    assert torch.equal(g1, g2) and torch.equal(b1, b2)


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16],
                         ids=["f32", "f16", "bf16"])
def test_fused_p0_equals_plain_layernorm_of_z(dtype):
    case(f"fused p=0 == ln_fwd(z) {dtype} 300x1280")
    inp = dev(synth.layer_inputs(300, 1280, dtype, seed=2))
    z, y, mean, rstd, mask = mb.bias_dropout_residual_ln_fwd(
        inp["x"], inp["bias"], inp["residual"], inp["gamma"], inp["beta"], 0.0, 7, EPS,
        want_mask=True)
    y2, mean2, rstd2 = mb.ln_fwd(z, inp["gamma"], inp["beta"], EPS)
    torch.cuda.synchronize()
    assert torch.all(mask == 1)
    assert torch.equal(y, y2) and torch.equal(mean, mean2) and torch.equal(rstd, rstd2)
    # p = 0: z is residual + (x + bias) rounded once
    ref = (inp["residual"].float() + (inp["x"].float() + inp["bias"].float())).to(dtype)
    assert torch.equal(z, ref)


def test_fused_p_nonzero_equals_plain_layernorm_of_z():
    case("fused p=0.1 y == ln_fwd(z) bf16 8192x1280")
    inp = dev(synth.layer_inputs(8192, 1280, torch.bfloat16, seed=0))
    z, y, mean, rstd, _ = mb.bias_dropout_residual_ln_fwd(
        inp["x"], inp["bias"], inp["residual"], inp["gamma"], inp["beta"], 0.1, 0, EPS)
    y2, mean2, rstd2 = mb.ln_fwd(z, inp["gamma"], inp["beta"], EPS)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(mean, mean2) and torch.equal(rstd, rstd2)


def test_mask_independent_of_dtype_and_of_mask_output():
    case("mask across dtypes 64x1000 p=0.25 seed 99")
    masks = []
    for dtype in (torch.float32, torch.float16, torch.bfloat16):
        inp = dev(synth.layer_inputs(64, 1000, dtype, seed=5))
        z, y, _, _, mask = mb.bias_dropout_residual_ln_fwd(
            inp["x"], inp["bias"], inp["residual"], inp["gamma"], inp["beta"], 0.25, 99, EPS,
            want_mask=True)
        z2, y2, _, _, none = mb.bias_dropout_residual_ln_fwd(
            inp["x"], inp["bias"], inp["residual"], inp["gamma"], inp["beta"], 0.25, 99, EPS,
            stats=False)
        torch.cuda.synchronize()
        assert none is None
        assert torch.equal(z, z2) and torch.equal(y, y2)
        masks.append(mask.cpu())
    assert torch.equal(masks[0], masks[1]) and torch.equal(masks[0], masks[2])


def test_in_place_forward_and_backward(orc):
    case("in place y=x and dx=dy bf16 513x1280")
    inp = dev(synth.layer_inputs(513, 1280, torch.bfloat16, seed=6,
                                 names=("x", "gamma", "beta", "dy")))
    y_ref, mean, rstd = mb.ln_fwd(inp["x"], inp["gamma"], inp["beta"], EPS)
    dx_ref, dg_ref, db_ref = mb.ln_bwd(inp["dy"], inp["x"], inp["gamma"], mean, rstd)
    x = inp["x"].clone()
    mb.ln_fwd(x, inp["gamma"], inp["beta"], EPS, y=x, mean=mean, rstd=rstd)
    dy = inp["dy"].clone()
    ws = mb.workspace(513, 1280, "cuda")
    mb.ln_bwd_dx(dy, inp["x"], inp["gamma"], mean, rstd, dx=dy, workspace=ws)
    dg, db = mb.ln_bwd_dgamma_dbeta(ws, 513, 1280, torch.bfloat16, partials_ready=True)
    torch.cuda.synchronize()
    assert torch.equal(x, y_ref) and torch.equal(dy, dx_ref)
    assert torch.equal(dg, dg_ref) and torch.equal(db, db_ref)


def test_unaligned_buffers_take_the_scalar_path(orc):
    # tensors that start 2 bytes past a 16-byte boundary
    rows, cols, dtype = 41, 1280, torch.bfloat16
    case(f"unaligned {dtype} {rows}x{cols}")
    inp = synth.layer_inputs(rows, cols, dtype, seed=8, names=("x", "gamma", "beta", "dy"))

    def shifted(t):
        buf = torch.empty(t.numel() + 8, dtype=t.dtype, device="cuda")
        v = buf[1:1 + t.numel()].view(t.shape)
        v.copy_(t.to("cuda"))
        return v
    x, g, b, dy = (shifted(inp[k]) for k in ("x", "gamma", "beta", "dy"))
    assert x.data_ptr() % 16 == 2
    y = shifted(torch.zeros(rows, cols, dtype=dtype))
    y, mean, rstd = mb.ln_fwd(x, g, b, EPS, y=y)
    dx = shifted(torch.zeros(rows, cols, dtype=dtype))
    dx, dg, db = mb.ln_bwd(dy, x, g, mean, rstd, dx=dx)
    torch.cuda.synchronize()
    check_fwd(orc, x, g, b, y, mean, rstd, FMT[dtype])
    check_bwd(orc, dy, x, g, mean, rstd, dx, dg, db, FMT[dtype])


@pytest.mark.parametrize("dtype,cols", [(torch.bfloat16, 1280), (torch.float32, 999),
                                        (torch.float16, 16384)])
def test_guard_bands_untouched(dtype, cols):
    rows = 77
    case(f"guard bands {dtype} {rows}x{cols}")
    inp = dev(synth.layer_inputs(rows, cols, dtype, seed=10))
    pad = 4096

    def banded(shape, dt):
        n = int(np.prod(shape))
        buf = torch.full((n + 2 * pad,), 77, dtype=dt, device="cuda")
        return buf, buf[pad:pad + n].view(shape)

    outs = {}
    for name, shape, dt in (("z", (rows, cols), dtype), ("y", (rows, cols), dtype),
                            ("mean", (rows,), torch.float32), ("rstd", (rows,), torch.float32),
                            ("mask", (rows, cols), torch.uint8),
                            ("dx", (rows, cols), dtype), ("dg", (cols,), torch.float32),
                            ("db", (cols,), torch.float32)):
        outs[name] = banded(shape, dt)
    ws_n = mb.ln_bwd_workspace_bytes(rows, cols) // 4
    ws_buf = torch.full((ws_n + 2 * pad,), 77, dtype=torch.float32, device="cuda")
    ws = ws_buf[pad:pad + ws_n]
    mb.bias_dropout_residual_ln_fwd(
        inp["x"], inp["bias"], inp["residual"], inp["gamma"], inp["beta"], 0.1, 3, EPS,
        residual_out=outs["z"][1], y=outs["y"][1], mean=outs["mean"][1], rstd=outs["rstd"][1],
        mask_out=outs["mask"][1])
    mb.ln_bwd_dx(inp["dy"], outs["z"][1], inp["gamma"], outs["mean"][1], outs["rstd"][1],
                 dx=outs["dx"][1], workspace=ws)
    mb.ln_bwd_dgamma_dbeta(ws, rows, cols, dtype, partials_ready=True, dgamma=outs["dg"][1],
                           dbeta=outs["db"][1])
    torch.cuda.synchronize()
    for name, (buf, _) in list(outs.items()) + [("ws", (ws_buf, ws))]:
        head, tail = buf[:pad], buf[-pad:]
        assert torch.all(head == 77) and torch.all(tail == 77), name


def test_graph_capture_replay(orc):
    rows, cols, dtype = 2048, 1280, torch.bfloat16
    case(f"graph capture fused fwd + bwd + fold {dtype} {rows}x{cols}")
    inp = dev(synth.layer_inputs(rows, cols, dtype, seed=11))
    z = torch.empty_like(inp["x"])
    y = torch.empty_like(inp["x"])
    dx = torch.empty_like(inp["x"])
    mean = torch.empty(rows, device="cuda")
    rstd = torch.empty(rows, device="cuda")
    dg = torch.empty(cols, device="cuda")
    db = torch.empty(cols, device="cuda")
    ws = mb.workspace(rows, cols, "cuda")

    def step():
        mb.bias_dropout_residual_ln_fwd(inp["x"], inp["bias"], inp["residual"], inp["gamma"],
                                        inp["beta"], 0.1, 21, EPS, residual_out=z, y=y,
                                        mean=mean, rstd=rstd)
        mb.ln_bwd_dx(inp["dy"], z, inp["gamma"], mean, rstd, dx=dx, workspace=ws)
        mb.ln_bwd_dgamma_dbeta(ws, rows, cols, dtype, partials_ready=True, dgamma=dg, dbeta=db)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (z, y, mean, rstd, dx, dg, db)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for k in range(4):
        for t in (z, y, mean, rstd, dx, dg, db):
            t.fill_(-1)                     # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((z, y, mean, rstd, dx, dg, db), eager):
            assert torch.equal(a, b), k
    check_bwd(orc, inp["dy"], z, inp["gamma"], mean, rstd, dx, dg, db, FMT[dtype])
