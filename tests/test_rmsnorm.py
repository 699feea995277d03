"""GPU parity of the fused residual add + RMSNorm forward and backward
(add_rmsnorm_fwd / add_rmsnorm_bwd) against the float64 oracle."""
import numpy as np
import pytest
import torch

import memory_bound_row_amd as mb
from memory_bound_row_amd import synth
from gpu_helpers import FMT, case, check_rmsnorm_bwd, check_rmsnorm_fwd, dev, f64

pytestmark = pytest.mark.gpu

RMS_EPS = 1e-6
DTYPES = [torch.float32, torch.float16, torch.bfloat16]
LAYOUTS_F32 = [(16, 1), (16, 2), (16, 4), (16, 8), (32, 1), (32, 2), (32, 3), (32, 4), (32, 5),
               (32, 6), (32, 7), (32, 8), (64, 1), (64, 2), (64, 3), (64, 4), (64, 5), (64, 6),
               (64, 7), (64, 8), (128, 4), (256, 4), (512, 4), (1024, 4)]
LAYOUTS_16 = [(16, 1), (16, 2), (16, 4), (32, 1), (32, 2), (32, 3), (32, 4), (32, 5), (64, 1),
              (64, 2), (64, 3), (64, 4), (64, 5), (128, 4), (256, 4), (512, 4)]


def inputs(rows, cols, dtype, seed, **kw):
    inp = dev(synth.layer_inputs(rows, cols, dtype, seed=seed,
                                 names=("x", "residual", "gamma", "dy"), **kw))
    ez = dev(synth.layer_inputs(rows, cols, dtype, seed=seed + 1, names=("dy",)))["dy"]
    return inp, ez


def run(orc, rows, cols, dtype, seed, residual=True, extra=True, name="rms", **kw):
    """Forward and backward on the GPU, each checked against the oracle."""
    inp, ez = inputs(rows, cols, dtype, seed, **kw)
    res = inp["residual"] if residual else None
    z, y, rstd = mb.add_rmsnorm_fwd(inp["x"], inp["gamma"], RMS_EPS, residual=res)
    ez = ez if extra else None
    dz, dg = mb.add_rmsnorm_bwd(inp["dy"], z, inp["gamma"], rstd, dz_extra=ez)
    torch.cuda.synchronize()
    check_rmsnorm_fwd(orc, inp["x"], res, inp["gamma"], z, y, rstd, FMT[dtype], RMS_EPS,
                      name=name)
    check_rmsnorm_bwd(orc, inp["dy"], ez, z, inp["gamma"], rstd, dz, dg, FMT[dtype],
                      name=f"{name}_bwd")
    return inp, z, y, rstd, dz, dg


@pytest.mark.parametrize("extra", [True, False])
def test_llama_prefill_shape(orc, extra):
    # one layer's add + RMSNorm of a 2048-token prefill at d = 4096 (the
    # Llama-3-8B prefill of the roofline page's worked example)
    case(f"add+rmsnorm 2048x4096 bf16 dz_extra={extra}")
    run(orc, 2048, 4096, torch.bfloat16, 0, extra=extra, name="rms.2048x4096")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("cols", [1, 7, 8, 100, 1000, 1280, 2048, 4096, 4104, 16384])
def test_small_shapes(orc, dtype, cols):
    rows = 300 if cols <= 4096 else 40   # several partitions and a ragged last block
    case(f"add+rmsnorm {rows}x{cols} {dtype}")
    run(orc, rows, cols, dtype, 5, name=f"rms.{rows}x{cols}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_without_residual(orc, dtype):
    case(f"plain rmsnorm 300x1280 {dtype}")
    inp, z, _, _, _, _ = run(orc, 300, 1280, dtype, 8, residual=False, extra=False,
                             name="rms.plain")
    assert z.data_ptr() == inp["x"].data_ptr()   # z is x itself


@pytest.mark.parametrize("dtype", DTYPES)
def test_forced_layouts(orc, dtype):
    layouts = LAYOUTS_F32 if dtype == torch.float32 else LAYOUTS_16
    e = 4 if dtype == torch.float32 else 8
    try:
        for g, v in layouts:
            cols = g * v * e - e              # one slot short of full: idle lanes
            case(f"add+rmsnorm forced {g}x{v} cols={cols} {dtype}")
            mb.debug_force_path(g, v)
            run(orc, 70, cols, dtype, 11, name=f"rms.{g}x{v}")
    finally:
        mb.debug_force_path(0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_per_element_path(orc, dtype):
    case(f"add+rmsnorm per-element path 200x1000 {dtype}")
    try:
        mb.debug_force_path(0, 0, scalar=True)
        run(orc, 200, 1000, dtype, 3, name="rms.scalar")
    finally:
        mb.debug_force_path(0)


def test_unaligned_rows(orc):
    # 1001 bf16 values per row: rows are not 16-byte aligned
    case("add+rmsnorm 129x1001 bf16 (per-element path by alignment)")
    run(orc, 129, 1001, torch.bfloat16, 4, name="rms.1001")


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_outliers(orc, dtype):
    """Activation outliers of 300: 300^2 = 90000 overflows fp16, so a sum of
    squares kept in fp16 would zero the row; the float32 sum keeps it."""
    case(f"add+rmsnorm outliers 256x4096 {dtype}")
    _, _, y, rstd, _, _ = run(orc, 256, 4096, dtype, 6, name="rms.outliers",
                              outlier_frac=1e-3)
    assert torch.isfinite(y).all() and torch.isfinite(rstd).all()
    assert (y != 0).float().mean().item() > 0.99


def test_in_place(orc):
    case("add+rmsnorm in place")
    inp, ez = inputs(300, 1280, torch.bfloat16, 9)
    z_ref, y_ref, rs_ref = mb.add_rmsnorm_fwd(inp["x"], inp["gamma"], RMS_EPS,
                                              residual=inp["residual"])
    dz_ref, dg_ref = mb.add_rmsnorm_bwd(inp["dy"], z_ref, inp["gamma"], rs_ref, dz_extra=ez)
    x2, r2, dy2 = inp["x"].clone(), inp["residual"].clone(), inp["dy"].clone()
    z, y, rs = mb.add_rmsnorm_fwd(x2, inp["gamma"], RMS_EPS, residual=r2, residual_out=r2,
                                  y=x2)
    dz, dg = mb.add_rmsnorm_bwd(dy2, z, inp["gamma"], rs, dz_extra=ez, dz=dy2)
    torch.cuda.synchronize()
    assert z.data_ptr() == r2.data_ptr() and y.data_ptr() == x2.data_ptr()
    assert dz.data_ptr() == dy2.data_ptr()
    for a, b in ((z, z_ref), (y, y_ref), (rs, rs_ref), (dz, dz_ref), (dg, dg_ref)):
        assert torch.equal(a, b)


def test_stats_not_kept(orc):
    case("add+rmsnorm without rstd")
    inp, _ = inputs(64, 4096, torch.bfloat16, 2)
    z, y, rstd = mb.add_rmsnorm_fwd(inp["x"], inp["gamma"], RMS_EPS,
                                    residual=inp["residual"], stats=False)
    z2, y2, _ = mb.add_rmsnorm_fwd(inp["x"], inp["gamma"], RMS_EPS, residual=inp["residual"])
    torch.cuda.synchronize()
    assert rstd is None and torch.equal(y, y2) and torch.equal(z, z2)


def test_empty():
    inp, _ = inputs(4, 64, torch.bfloat16, 0)
    x0 = inp["x"][:0]
    z, y, rstd = mb.add_rmsnorm_fwd(x0, inp["gamma"], RMS_EPS, residual=inp["residual"][:0])
    dz, dg = mb.add_rmsnorm_bwd(inp["dy"][:0], z, inp["gamma"], rstd)
    torch.cuda.synchronize()
    assert y.shape == (0, 64) and dz.shape == (0, 64)
    assert torch.equal(dg, torch.zeros_like(dg))


def test_one_column_row(orc):
    # m = 1: y = gamma * z / sqrt(z^2 + eps) and dx = rstd*eps*rstd^2*g -> tiny
    case("add+rmsnorm 300x1 fp32")
    _, z, y, rstd, dz, _ = run(orc, 300, 1, torch.float32, 12, extra=False, name="rms.m1")
    z64 = f64(z)[:, 0]
    assert np.all(np.abs(f64(y)[:, 0]) <= 1.5 * (np.abs(z64) / np.sqrt(z64 ** 2 + RMS_EPS))
                  + 1e-6)


def test_deterministic():
    case("add+rmsnorm determinism")
    inp, ez = inputs(16384, 1024, torch.bfloat16, 2)
    z, _, rstd = mb.add_rmsnorm_fwd(inp["x"], inp["gamma"], RMS_EPS, residual=inp["residual"])
    ref = mb.add_rmsnorm_bwd(inp["dy"], z, inp["gamma"], rstd, dz_extra=ez)
    torch.cuda.synchronize()
    for _ in range(20):
        out = mb.add_rmsnorm_bwd(inp["dy"], z, inp["gamma"], rstd, dz_extra=ez)
        torch.cuda.synchronize()
        assert torch.equal(out[0].view(torch.int16), ref[0].view(torch.int16))
        assert torch.equal(out[1], ref[1])
