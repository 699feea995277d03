"""Row isolation under non-finite inputs (GPU).

A few rows of each input hold +Inf, NaN or -Inf in one element.  Every other
row -- including rows that share a wave, a workgroup and a reduction tree
with a poisoned one -- must still equal the float64 oracle under the usual
tolerance, and each poisoned row must be finite exactly where the oracle's
is: a reduction that mixed rows, or masked another row's lanes by
multiplying with 0, would spread the NaN.  The column sums show the same
separation: dbeta sums dy alone and stays finite and exact, while dgamma
(which sums dy * xhat) is non-finite in every column, as in the oracle.
Where a -Inf is a legal value (a masked score for the softmax, a logit of
probability 0), the row stays finite and is checked like the others; in the
fused forward a poisoned element that the mask drops adds exactly 0.
"""
import math

import numpy as np
import pytest
import torch

import memory_bound_row_amd as mb
from memory_bound_row_amd import synth
from oracle import compare as cmp
from gpu_helpers import (EPS, FMT, assert_reports, case, check_bwd, check_fwd,
                         check_rmsnorm_fwd, check_softmax_bwd, check_softmax_fwd, check_xent,
                         dev, f64)

pytestmark = pytest.mark.gpu

ROWS = 48
POISON = ((5, 3, np.inf), (17, -1, np.nan), (30, 0, -np.inf))   # (row, column, value)


def poison(t):
    for r, c, v in POISON:
        t[r, c] = v


def split(ref):
    """Rows where the oracle's output is finite throughout, and the rest."""
    ok = np.isfinite(ref.reshape(ref.shape[0], -1)).all(axis=1)
    return np.nonzero(ok)[0].tolist(), np.nonzero(~ok)[0].tolist()


def same_finiteness(name, got, ref):
    g = f64(got).reshape(ref.shape)
    bad = np.isfinite(g) != np.isfinite(ref)
    assert not bad.any(), f"{name}: {int(bad.sum())} elements differ in finiteness"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("cols", [64, 1000, 1280, 4096])
def test_layernorm(orc, dtype, cols):
    case(f"LayerNorm fwd + bwd with non-finite rows {ROWS}x{cols} {dtype}")
    inp = dev(synth.layer_inputs(ROWS, cols, dtype, seed=31, names=("x", "gamma", "beta", "dy")))
    x = inp["x"]
    poison(x)
    y, mean, rstd = mb.ln_fwd(x, inp["gamma"], inp["beta"], EPS)
    dx, dg, db = mb.ln_bwd(inp["dy"], x, inp["gamma"], mean, rstd)
    torch.cuda.synchronize()
    y_ref, _, _ = orc.ln_fwd(f64(x), f64(inp["gamma"]), f64(inp["beta"]), EPS)
    good, bad = split(y_ref)
    assert sorted(bad) == sorted(r for r, _, _ in POISON)
    g = torch.as_tensor(good, device="cuda")
    check_fwd(orc, x[g], inp["gamma"], inp["beta"], y[g], mean[g], rstd[g], FMT[dtype],
              name="nonfinite.ln")
    same_finiteness("nonfinite.ln.y", y[bad], y_ref[bad])
    # dx from the stored statistics of each row (non-finite in the poisoned ones)
    check_bwd(orc, inp["dy"][g], x[g], inp["gamma"], mean[g], rstd[g], dx[g], None, None,
              FMT[dtype], name="nonfinite.ln_bwd")
    dx_ref = orc.ln_bwd_dx(f64(inp["dy"])[bad], f64(x)[bad], f64(inp["gamma"]),
                           f64(mean)[bad], f64(rstd)[bad])
    same_finiteness("nonfinite.ln_bwd.dx", dx[bad], dx_ref)
    dg_ref, db_ref, _, sb = orc.ln_bwd_params(f64(inp["dy"]), f64(x), f64(mean), f64(rstd))
    same_finiteness("nonfinite.dgamma", dg, dg_ref)
    assert not np.isfinite(dg_ref).any()
    assert_reports(cmp.check_colsum("nonfinite.dbeta", f64(db), db_ref, sb, ROWS, FMT[dtype]))


@pytest.mark.parametrize("dtype,cols", [(torch.float32, 20000), (torch.float32, 65536),
                                        (torch.bfloat16, 40000)])
def test_layernorm_staged_rows(orc, dtype, cols):
    # rows staged in LDS; fp32 65536: the last column lies past the stage, in
    # the slots whose statistics pass 1 keeps apart
    case(f"staged LayerNorm fwd with non-finite rows {ROWS}x{cols} {dtype}")
    inp = dev(synth.layer_inputs(ROWS, cols, dtype, seed=33, names=("x", "gamma", "beta")))
    x = inp["x"]
    poison(x)
    y, mean, rstd = mb.ln_fwd(x, inp["gamma"], inp["beta"], EPS)
    torch.cuda.synchronize()
    y_ref, _, _ = orc.ln_fwd(f64(x), f64(inp["gamma"]), f64(inp["beta"]), EPS)
    good, bad = split(y_ref)
    assert sorted(bad) == sorted(r for r, _, _ in POISON)
    g = torch.as_tensor(good, device="cuda")
    check_fwd(orc, x[g], inp["gamma"], inp["beta"], y[g], mean[g], rstd[g], FMT[dtype],
              name="nonfinite.staged")
    same_finiteness("nonfinite.staged.y", y[bad], y_ref[bad])


@pytest.fixture(params=[False, True], ids=["registers", "two_pass"])
def two_pass(request):
    """The register-resident kernels, or the two-pass long-row path forced
    at these widths."""
    mb.debug_force_two_pass(request.param)
    yield request.param
    mb.debug_force_two_pass(False)


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
@pytest.mark.parametrize("cols", [64, 1000, 4096])
def test_softmax(orc, dtype, cols, two_pass):
    case(f"softmax fwd + bwd with non-finite rows {ROWS}x{cols} {dtype} two_pass={two_pass}")
    d = dev(synth.layer_inputs(ROWS, cols, dtype, seed=32, names=("x", "dy")))
    x = d["x"]
    poison(x)
    y, _ = mb.attn_softmax_fwd(x, 0.5)
    dx = mb.attn_softmax_bwd(d["dy"], y, 0.5)
    torch.cuda.synchronize()
    y_ref = orc.attn_softmax_fwd(f64(x), scale=0.5, mask=None, rows_per_mask=1, causal=False)
    good, bad = split(y_ref)
    assert sorted(bad) == [5, 17]          # the -Inf score is a masked key
    g = torch.as_tensor(good, device="cuda")
    check_softmax_fwd(orc, x[g], y[g], None, FMT[dtype], scale=0.5, name="nonfinite.sm")
    same_finiteness("nonfinite.sm.y", y[bad], y_ref[bad])
    check_softmax_bwd(orc, d["dy"][g], y[g], dx[g], FMT[dtype], scale=0.5,
                      name="nonfinite.sm_bwd")
    dx_ref = orc.attn_softmax_bwd(f64(d["dy"])[bad], f64(y)[bad], keep=None, p=0.0, scale=0.5)
    same_finiteness("nonfinite.sm_bwd.dx", dx[bad], dx_ref)


@pytest.mark.parametrize("cols", [1280, 4096])
def test_add_rmsnorm(orc, cols):
    case(f"add + RMSNorm fwd with non-finite rows {ROWS}x{cols} bf16")
    dt = torch.bfloat16
    d = dev(synth.layer_inputs(ROWS, cols, dt, seed=33, names=("x", "residual", "gamma")))
    x = d["x"]
    poison(x)
    z, y, rstd = mb.add_rmsnorm_fwd(x, d["gamma"], 1e-6, residual=d["residual"])
    torch.cuda.synchronize()
    y_ref, rs_ref = orc.rmsnorm_fwd(f64(z), f64(d["gamma"]), 1e-6)
    good, bad = split(y_ref)
    assert sorted(bad) == sorted(r for r, _, _ in POISON)
    g = torch.as_tensor(good, device="cuda")
    check_rmsnorm_fwd(orc, x[g], d["residual"][g], d["gamma"], z[g], y[g], rstd[g], FMT[dt],
                      1e-6, name="nonfinite.rms")
    # an infinite element: rstd = 0, the rest of its row exactly 0, the element NaN
    same_finiteness("nonfinite.rms.y", y[bad], y_ref[bad])
    same_finiteness("nonfinite.rms.rstd", rstd[bad], rs_ref[bad])
    yb, rb = f64(y[bad]), y_ref[bad]
    both = np.isfinite(yb) & np.isfinite(rb)
    assert np.array_equal(yb[both], rb[both])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("cols", [1000, 50257, 120000, 200000])
def test_cross_entropy(orc, dtype, cols, two_pass):
    # 120000 fp32 and 200000 bf16 columns: rows held in registers and LDS
    # (column -1 of a poisoned row lies in an LDS slot)
    case(f"cross-entropy with non-finite rows {ROWS}x{cols} {dtype} two_pass={two_pass}")
    x = dev(synth.layer_inputs(ROWS, cols, dtype, seed=34, names=("x",)))["x"]
    poison(x)
    lab = torch.randint(0, cols, (ROWS,), device="cuda",
                        generator=torch.Generator(device="cuda").manual_seed(35))
    loss, dx = mb.cross_entropy_fwd_bwd(x, lab, label_smoothing=0.1, grad_scale=1.0)
    torch.cuda.synchronize()
    loss_ref, dx_ref = orc.cross_entropy(f64(x), lab.cpu().numpy(), 0.1, 1.0, grad=True)
    bad = sorted(r for r, _, _ in POISON)
    good = [r for r in range(ROWS) if r not in bad]
    check_xent(orc, x, lab, cols, 0.1, 1.0, loss, dx, FMT[dtype], rows_sel=good,
               name="nonfinite.xent")
    # a -Inf logit has probability 0: the smoothed loss is +Inf, the gradient finite
    same_finiteness("nonfinite.xent.loss", loss[bad], loss_ref[bad])
    same_finiteness("nonfinite.xent.dx", dx[bad], dx_ref[bad])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("cols", [64, 1280])
def test_fused_forward(orc, dtype, cols):
    """A dropped element contributes exactly 0 whatever its value: a poisoned
    row whose poisoned element the mask drops stays finite (z = residual
    there), one whose element is kept turns non-finite."""
    case(f"fused forward with non-finite rows {ROWS}x{cols} {dtype}")
    p, seed = 0.5, 4242
    d = dev(synth.layer_inputs(ROWS, cols, dtype, seed=36,
                               names=("x", "residual", "bias", "gamma", "beta")))
    x = d["x"]
    # every row poisoned at its own column, so some elements are kept and some dropped
    for r in range(ROWS):
        x[r, (7 * r) % cols] = (np.inf, np.nan, -np.inf)[r % 3]
    z, y, mean, rstd, _ = mb.bias_dropout_residual_ln_fwd(x, d["bias"], d["residual"],
                                                          d["gamma"], d["beta"], p, seed, EPS)
    torch.cuda.synchronize()
    keep = orc.dropout_keep(seed, p, ROWS, cols)
    z_ref = orc.bias_dropout_residual(f64(x), f64(d["bias"]), f64(d["residual"]), keep, p)
    good, bad = split(z_ref)
    hit = keep[np.arange(ROWS), (7 * np.arange(ROWS)) % cols] == 1
    assert bad == np.nonzero(hit)[0].tolist() and len(good) > 0 and len(bad) > 0
    g = torch.as_tensor(good, device="cuda")
    assert_reports(cmp.check_elementwise("nonfinite.fused.z", f64(z)[good], z_ref[good],
                                         FMT[dtype]))
    check_fwd(orc, z[g], d["gamma"], d["beta"], y[g], mean[g], rstd[g], FMT[dtype],
              name="nonfinite.fused.ln")
    same_finiteness("nonfinite.fused.z", z[bad], z_ref[bad])
    y_ref, _, _ = orc.ln_fwd(f64(z)[bad], f64(d["gamma"]), f64(d["beta"]), EPS)
    same_finiteness("nonfinite.fused.y", y[bad], y_ref)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("cols", [64, 1280])
def test_prologue_backward(orc, dtype, cols):
    """Poisoned rows of z: their dz is non-finite throughout, their dx only
    where the mask keeps; dbias is non-finite exactly in the columns where a
    poisoned row is kept, dgamma everywhere, dbeta nowhere."""
    case(f"prologue backward with non-finite rows {ROWS}x{cols} {dtype}")
    p, seed = 0.3, 99
    d = dev(synth.layer_inputs(ROWS, cols, dtype, seed=37,
                               names=("x", "residual", "gamma", "beta", "dy")))
    z, ez = d["x"], d["residual"]
    poison(z)
    _, mean, rstd = mb.ln_fwd(z, d["gamma"], d["beta"], EPS)
    dres, dx, dg, db, dbias = mb.bias_dropout_residual_ln_bwd(d["dy"], z, d["gamma"], mean,
                                                              rstd, p, seed, dz_extra=ez)
    torch.cuda.synchronize()
    dy64, z64, g64 = f64(d["dy"]), f64(z), f64(d["gamma"])
    mu64, rs64, ez64 = f64(mean), f64(rstd), f64(ez)
    dz_ref = orc.ln_bwd_dx(dy64, z64, g64, mu64, rs64) + ez64
    scale = orc.ln_bwd_dx_scale(dy64, z64, g64, mu64, rs64) + np.abs(ez64)
    keep = orc.dropout_keep(seed, p, ROWS, cols)
    dx_ref, dbias_ref, sbias = orc.dropout_residual_bwd(dz_ref, keep, p)
    good, bad = split(dz_ref)
    assert sorted(bad) == sorted(r for r, _, _ in POISON)
    s = 1.0 / (1.0 - np.float64(np.float32(p)))
    dx_scale = np.where(keep == 1, scale * s, 0.0)
    fmt = FMT[dtype]
    assert_reports(
        cmp.check_elementwise("nonfinite.drop.dresidual", f64(dres)[good], dz_ref[good], fmt,
                              term_scale=scale[good], row_len=cols),
        cmp.check_elementwise("nonfinite.drop.dx", f64(dx)[good], dx_ref[good], fmt,
                              term_scale=dx_scale[good], row_len=cols))
    same_finiteness("nonfinite.drop.dresidual", dres[bad], dz_ref[bad])
    same_finiteness("nonfinite.drop.dx", dx[bad], dx_ref[bad])
    assert np.all(f64(dx)[keep == 0] == 0.0)
    same_finiteness("nonfinite.drop.dbias", dbias, dbias_ref)
    fin = np.isfinite(dbias_ref)
    k = 4 + math.ceil(math.log2(max(cols, 2)))
    bias_err = np.sum(k * 2.0 ** -24 * np.where(np.isfinite(dx_scale), dx_scale, 0.0), axis=0)
    reps = []
    if fin.any():
        reps.append(cmp.check_colsum("nonfinite.drop.dbias", f64(dbias)[fin], dbias_ref[fin],
                                     sbias[fin], ROWS, fmt, term_err=bias_err[fin]))
    dg_ref, db_ref, _, sb = orc.ln_bwd_params(dy64, z64, mu64, rs64)
    same_finiteness("nonfinite.drop.dgamma", dg, dg_ref)
    reps.append(cmp.check_colsum("nonfinite.drop.dbeta", f64(db), db_ref, sb, ROWS, fmt))
    assert_reports(*reps)


@pytest.mark.parametrize("cols", [1280, 4096])
def test_add_rmsnorm_backward(orc, cols):
    """An infinite element of z: rstd = 0, so its row's xhat is NaN at that
    element and 0 elsewhere; dz is non-finite across the row, dgamma only in
    the poisoned columns."""
    case(f"add + RMSNorm bwd with non-finite rows {ROWS}x{cols} bf16")
    dt = torch.bfloat16
    d = dev(synth.layer_inputs(ROWS, cols, dt, seed=38, names=("x", "residual", "gamma", "dy")))
    z0, ez = d["x"], d["residual"]
    z0[5, 3] = np.inf
    z0[30, 0] = -np.inf
    z, _, rstd = mb.add_rmsnorm_fwd(z0, d["gamma"], 1e-6)
    dz, dg = mb.add_rmsnorm_bwd(d["dy"], z, d["gamma"], rstd, dz_extra=ez)
    torch.cuda.synchronize()
    dy64, z64, g64, rs64, ez64 = f64(d["dy"]), f64(z), f64(d["gamma"]), f64(rstd), f64(ez)
    dx_ref, dg_ref, sg = orc.rmsnorm_bwd(dy64, z64, g64, rs64)
    dz_ref = dx_ref + ez64
    good, bad = split(dz_ref)
    assert bad == [5, 30]
    g = g64 * dy64
    with np.errstate(invalid="ignore"):   # inf * 0 in the poisoned rows
        xh = z64 * rs64[:, None]
        scale = rs64[:, None] * (np.abs(g) + np.abs(xh) * np.sum(np.abs(g * xh), axis=1,
                                                                  keepdims=True) / cols)
    scale = scale + np.abs(ez64)
    assert_reports(cmp.check_elementwise("nonfinite.rms_bwd.dz", f64(dz)[good], dz_ref[good],
                                         cmp.BF16, term_scale=scale[good], row_len=cols))
    same_finiteness("nonfinite.rms_bwd.dz", dz[bad], dz_ref[bad])
    same_finiteness("nonfinite.rms_bwd.dgamma", dg, dg_ref)
    fin = np.isfinite(dg_ref)
    assert sorted(np.nonzero(~fin)[0].tolist()) == [0, 3]
    assert_reports(cmp.check_colsum("nonfinite.rms_bwd.dgamma", f64(dg)[fin], dg_ref[fin],
                                    sg[fin], ROWS, cmp.BF16))
