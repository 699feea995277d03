"""GPU parity of bias_dropout_residual_ln_bwd -- the LayerNorm backward fused
with the backward of the bias + dropout + residual prologue -- against the
float64 oracle, and its identities with the other entry points."""
import pytest
import torch

import memory_bound_row_amd as mb
from memory_bound_row_amd import synth
from gpu_helpers import EPS, FMT, case, check_dropout_bwd, dev

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.float16, torch.bfloat16]
DROP_LAYOUTS_F32 = [(16, 1), (16, 2), (16, 4), (32, 1), (32, 2), (32, 3), (32, 4), (64, 1),
                    (64, 2), (64, 3), (64, 4), (64, 5), (64, 6), (128, 4), (256, 4), (512, 4)]
DROP_LAYOUTS_16 = [(16, 1), (16, 2), (32, 1), (32, 2), (32, 3), (64, 1), (64, 2), (64, 3),
                   (128, 2), (256, 2), (512, 2)]


def forward(rows, cols, dtype, p, seed, data_seed=0):
    """Stored inputs and the fused forward's outputs, plus a gradient reaching
    z from its other uses (drawn like dy, from the next data seed)."""
    inp = dev(synth.layer_inputs(rows, cols, dtype, seed=data_seed))
    z, y, mean, rstd, mask = mb.bias_dropout_residual_ln_fwd(
        inp["x"], inp["bias"], inp["residual"], inp["gamma"], inp["beta"], p, seed, EPS,
        want_mask=True)
    ez = dev(synth.layer_inputs(rows, cols, dtype, seed=data_seed + 1, names=("dy",)))["dy"]
    return inp, z, mean, rstd, mask, ez


def backward(inp, z, mean, rstd, p, seed, ez):
    return mb.bias_dropout_residual_ln_bwd(inp["dy"], z, inp["gamma"], mean, rstd, p, seed,
                                           dz_extra=ez)


def check(orc, inp, z, mean, rstd, p, seed, ez, outs, name):
    dres, dx, dg, db, dbias = outs
    torch.cuda.synchronize()
    check_dropout_bwd(orc, inp["dy"], ez, z, inp["gamma"], mean, rstd, p, seed, dres, dx, dg,
                      db, dbias, FMT[z.dtype], name=name)


@pytest.mark.parametrize("extra", [True, False])
def test_metric_shape(orc, extra):
    case(f"prologue backward 8192x1280 bf16 p=0.1 dz_extra={extra}")
    inp, z, mean, rstd, _, ez = forward(8192, 1280, torch.bfloat16, 0.1, 0)
    ez = ez if extra else None
    check(orc, inp, z, mean, rstd, 0.1, 0, ez, backward(inp, z, mean, rstd, 0.1, 0, ez),
          "drop_bwd.8192x1280")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("cols", [1, 7, 8, 100, 1000, 1280, 2048, 4104, 8192])
def test_small_shapes(orc, dtype, cols):
    rows = 300 if cols <= 2048 else 40   # several partitions and a ragged last block
    case(f"prologue backward {rows}x{cols} {dtype}")
    inp, z, mean, rstd, _, ez = forward(rows, cols, dtype, 0.1, 5)
    check(orc, inp, z, mean, rstd, 0.1, 5, ez, backward(inp, z, mean, rstd, 0.1, 5, ez),
          f"drop_bwd.{rows}x{cols}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_forced_layouts(orc, dtype):
    layouts = DROP_LAYOUTS_F32 if dtype == torch.float32 else DROP_LAYOUTS_16
    e = 4 if dtype == torch.float32 else 8
    try:
        for g, v in layouts:
            cols = g * v * e - e              # one slot short of full: idle lanes
            case(f"prologue backward forced {g}x{v} cols={cols} {dtype}")
            mb.debug_force_path(g, v)
            inp, z, mean, rstd, _, ez = forward(70, cols, dtype, 0.25, 11)
            check(orc, inp, z, mean, rstd, 0.25, 11, ez,
                  backward(inp, z, mean, rstd, 0.25, 11, ez), f"drop_bwd.{g}x{v}")
    finally:
        mb.debug_force_path(0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_per_element_path(orc, dtype):
    case(f"prologue backward per-element path 200x1000 {dtype}")
    try:
        mb.debug_force_path(0, 0, scalar=True)
        inp, z, mean, rstd, _, ez = forward(200, 1000, dtype, 0.1, 3)
        check(orc, inp, z, mean, rstd, 0.1, 3, ez, backward(inp, z, mean, rstd, 0.1, 3, ez),
              "drop_bwd.scalar")
    finally:
        mb.debug_force_path(0)


def test_p_zero_passes_dz_through():
    case("prologue backward p=0")
    inp, z, mean, rstd, _, ez = forward(256, 1280, torch.bfloat16, 0.0, 0)
    dres, dx, _, _, dbias = backward(inp, z, mean, rstd, 0.0, 0, ez)
    torch.cuda.synchronize()
    # keep everything, scale 1: dx is dz itself
    assert torch.equal(dx, dres)


def test_matches_layernorm_backward():
    """Without dz_extra, dresidual is the LayerNorm's dx and dgamma/dbeta are
    the LayerNorm backward's, bit for bit (same layout, same partitions, same
    expressions and fold order)."""
    for dtype, cols, layout in ((torch.bfloat16, 1280, (64, 3)), (torch.float32, 768, (64, 3)),
                                (torch.float16, 4096, (512, 2))):
        case(f"prologue backward vs LayerNorm backward {dtype} {cols}")
        inp, z, mean, rstd, _, _ = forward(1000, cols, dtype, 0.1, 1)
        try:
            if layout[0] <= 64:
                mb.debug_force_path(*layout)
            dres, _, dg, db, _ = backward(inp, z, mean, rstd, 0.1, 1, None)
            dx_ln, dg_ln, db_ln = mb.ln_bwd(inp["dy"], z, inp["gamma"], mean, rstd)
            torch.cuda.synchronize()
        finally:
            mb.debug_force_path(0)
        if layout[0] <= 64:
            assert torch.equal(dres, dx_ln)
            assert torch.equal(dg, dg_ln) and torch.equal(db, db_ln)
        else:
            # different layouts: same values within float32 rounding
            assert torch.allclose(dg, dg_ln, rtol=1e-5, atol=1e-4)


def test_dropped_positions_follow_the_forward_mask():
    case("prologue backward mask consistency")
    inp, z, mean, rstd, mask, ez = forward(512, 1280, torch.float32, 0.3, 99)
    dres, dx, _, _, _ = backward(inp, z, mean, rstd, 0.3, 99, ez)
    torch.cuda.synchronize()
    m = mask.bool()
    assert torch.all(dx[~m] == 0)
    nz = dres != 0
    assert torch.all(dx[m & nz] != 0)
    # kept positions: dz / (1 - p) in float32, rounded to fp32 storage
    ratio = (dx[m & nz] / dres[m & nz]).double()
    assert torch.allclose(ratio, torch.full_like(ratio, 1.0 / (1.0 - 0.3)), rtol=1e-6)


def test_deterministic():
    case("prologue backward determinism")
    inp, z, mean, rstd, _, ez = forward(16384, 1024, torch.bfloat16, 0.1, 2)
    ref = backward(inp, z, mean, rstd, 0.1, 2, ez)
    torch.cuda.synchronize()
    for _ in range(20):
        out = backward(inp, z, mean, rstd, 0.1, 2, ez)
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_in_place():
    case("prologue backward in place")
    inp, z, mean, rstd, _, ez = forward(300, 1280, torch.bfloat16, 0.1, 4)
    ref = backward(inp, z, mean, rstd, 0.1, 4, ez)
    dy2, z2 = inp["dy"].clone(), z.clone()
    out = mb.bias_dropout_residual_ln_bwd(dy2, z2, inp["gamma"], mean, rstd, 0.1, 4,
                                          dz_extra=ez, dresidual=dy2, dx=z2)
    torch.cuda.synchronize()
    assert out[0].data_ptr() == dy2.data_ptr() and out[1].data_ptr() == z2.data_ptr()
    for a, b in zip(out, ref):
        assert torch.equal(a, b)


def test_seed_changes_mask():
    case("prologue backward seeds")
    inp, z, mean, rstd, _, ez = forward(256, 1024, torch.bfloat16, 0.5, 7)
    _, dx_a, _, _, _ = backward(inp, z, mean, rstd, 0.5, 7, ez)
    _, dx_b, _, _, _ = backward(inp, z, mean, rstd, 0.5, 8, ez)
    torch.cuda.synchronize()
    a, b = dx_a == 0, dx_b == 0
    # p = 0.5: about half the positions differ between independent masks
    frac = (a != b).float().mean().item()
    assert 0.4 < frac < 0.6, frac


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows,cols", [(8192, 1280), (37, 1001)])
def test_two_stage_calls_equal_the_combined_call(dtype, rows, cols):
    # bias_dropout_residual_ln_bwd_dx then _fold give the combined call's bits
    case(f"prologue backward split stages {dtype} {rows}x{cols}")
    inp, z, mean, rstd, _, ez = forward(rows, cols, dtype, 0.1, 21)
    want = backward(inp, z, mean, rstd, 0.1, 21, ez)
    ws = mb.dropout_workspace(rows, cols, z.device)
    dres, dx = mb.bias_dropout_residual_ln_bwd_dx(inp["dy"], z, inp["gamma"], mean, rstd, 0.1,
                                                  21, workspace=ws, dz_extra=ez)
    dg, db, dbias = mb.bias_dropout_residual_ln_bwd_fold(ws, rows, cols)
    torch.cuda.synchronize()
    for name, a, b in zip(("dresidual", "dx", "dgamma", "dbeta", "dbias"),
                          (dres, dx, dg, db, dbias), want):
        assert torch.equal(a, b), name
