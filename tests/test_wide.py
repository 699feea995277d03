"""GPU parity of the LDS-staged LayerNorm path: rows wider than the register
layouts (more than 16384 columns) staged in one workgroup's LDS ("02 · llmc/
的 CUDA kernel 层" §3.1), forward, fused forward and backward, against the
float64 oracle; the same kernels forced onto narrow and ragged rows; the
rows past the stage's capacity that are read again from global memory."""
import numpy as np
import pytest
import torch

import memory_bound_row_amd as mb
from memory_bound_row_amd import synth
from gpu_helpers import (EPS, FMT, assert_reports, case, check_bwd, check_fused, check_fwd, dev,
                         f64)
from oracle import compare as cmp

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.float16, torch.bfloat16]
IDS = ["f32", "f16", "bf16"]
# widest backward row per dtype (LN_MAX_COLS_BWD_*)
MAX_BWD = {torch.float32: 19968, torch.float16: 32768, torch.bfloat16: 32768}


@pytest.fixture(autouse=True)
def _default_path():
    mb.debug_force_staged(False)
    yield
    mb.debug_force_staged(False)


def fwd_bwd(rows, cols, dtype, seed, x_mean=0.0, bwd=True):
    inp = dev(synth.layer_inputs(rows, cols, dtype, seed=seed, x_mean=x_mean))
    y, mean, rstd = mb.ln_fwd(inp["x"], inp["gamma"], inp["beta"], EPS)
    out = None
    if bwd:
        out = mb.ln_bwd(inp["dy"], inp["x"], inp["gamma"], mean, rstd)
    torch.cuda.synchronize()
    return inp, y, mean, rstd, out


@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
@pytest.mark.parametrize("cols", [16385, 16392, 20000, 32768, 39936, 40000, 65535, 65536])
def test_forward_wide(orc, dtype, cols):
    # fp32 rows past 39936 columns overflow the stage and are read again
    rows = 20
    case(f"staged ln_fwd {dtype} {rows}x{cols}")
    inp, y, mean, rstd, _ = fwd_bwd(rows, cols, dtype, seed=cols, bwd=False)
    check_fwd(orc, inp["x"], inp["gamma"], inp["beta"], y, mean, rstd, FMT[dtype],
              strict=dtype == torch.float32)


@pytest.mark.parametrize("dtype,cols", [(d, c) for d in DTYPES
                                        for c in (16385, 16392, 19968, 20000, 32768)
                                        if c <= MAX_BWD[d]])
def test_backward_wide(orc, dtype, cols):
    rows = 300                                  # 256 partitions, some with two rows
    case(f"staged ln_fwd+ln_bwd {dtype} {rows}x{cols}")
    inp, y, mean, rstd, (dx, dg, db) = fwd_bwd(rows, cols, dtype, seed=cols + 1)
    check_fwd(orc, inp["x"], inp["gamma"], inp["beta"], y, mean, rstd, FMT[dtype])
    check_bwd(orc, inp["dy"], inp["x"], inp["gamma"], mean, rstd, dx, dg, db, FMT[dtype],
              strict=dtype == torch.float32)


@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
@pytest.mark.parametrize("cols", [16392, 32768, 65536, 40001])
@pytest.mark.parametrize("seed", [0, 2 ** 63 + 5])
def test_fused_forward_wide(orc, dtype, cols, seed):
    rows = 12
    case(f"staged bias_dropout_residual_ln_fwd {dtype} {rows}x{cols} seed {seed}")
    inp = dev(synth.layer_inputs(rows, cols, dtype, seed=cols + 2))
    z, y, mean, rstd, mask = mb.bias_dropout_residual_ln_fwd(
        inp["x"], inp["bias"], inp["residual"], inp["gamma"], inp["beta"], 0.1, seed, EPS,
        want_mask=True)
    torch.cuda.synchronize()
    check_fused(orc, inp, 0.1, seed, z, y, mean, rstd, mask, FMT[dtype])


@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
@pytest.mark.parametrize("cols", [20000, 65536])
def test_fused_forward_wide_keep_bits(orc, dtype, cols):
    # x = 0.75, bias = 0.25, residual = 0: z shows every keep bit the kernel applied
    rows, p, seed = 9, 0.25, 77
    case(f"staged fused keep bits {dtype} {rows}x{cols}")
    x = torch.full((rows, cols), 0.75, dtype=dtype, device="cuda")
    res = torch.zeros_like(x)
    bias = torch.full((cols,), 0.25, dtype=dtype, device="cuda")
    ones, zeros = torch.ones_like(bias), torch.zeros_like(bias)
    z, _, _, _, _ = mb.bias_dropout_residual_ln_fwd(x, bias, res, ones, zeros, p, seed,
                                                    stats=False)
    torch.cuda.synchronize()
    got = (z.float() != 0).cpu().numpy().astype(np.uint8)
    assert np.array_equal(got, orc.dropout_keep(seed, p, rows, cols))


@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
@pytest.mark.parametrize("cols", [1, 7, 8, 64, 100, 1000, 1001, 1280, 4104])
def test_staged_path_forced_on_narrow_rows(orc, dtype, cols):
    # the staged kernels on rows the register layouts would take: tiny rows
    # leave most of the 1024 lanes idle; ragged widths take the per-element path
    rows = 37
    case(f"forced staged path {dtype} {rows}x{cols}")
    mb.debug_force_staged(True)
    inp = dev(synth.layer_inputs(rows, cols, dtype, seed=cols + 3))
    y, mean, rstd = mb.ln_fwd(inp["x"], inp["gamma"], inp["beta"], EPS)
    dx, dg, db = mb.ln_bwd(inp["dy"], inp["x"], inp["gamma"], mean, rstd)
    z, y2, mean2, rstd2, mask = mb.bias_dropout_residual_ln_fwd(
        inp["x"], inp["bias"], inp["residual"], inp["gamma"], inp["beta"], 0.2, 9, EPS,
        want_mask=True)
    torch.cuda.synchronize()
    mb.debug_force_staged(False)
    check_fwd(orc, inp["x"], inp["gamma"], inp["beta"], y, mean, rstd, FMT[dtype])
    check_bwd(orc, inp["dy"], inp["x"], inp["gamma"], mean, rstd, dx, dg, db, FMT[dtype])
    check_fused(orc, inp, 0.2, 9, z, y2, mean2, rstd2, mask, FMT[dtype])
    if cols == 1:
        assert torch.all(dx == 0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_unaligned_rows(orc, dtype):
    # a base address off the 16-byte grid takes the per-element path
    rows, cols = 10, 19001
    case(f"staged unaligned {dtype} {rows}x{cols}")
    inp = synth.layer_inputs(rows, cols, dtype, seed=5)
    buf = {k: torch.empty(v.numel() + 1, dtype=dtype, device="cuda") for k, v in inp.items()}
    for k, v in inp.items():
        buf[k][1:].copy_(v.reshape(-1))
    t = {k: buf[k][1:].view(inp[k].shape) for k in inp}
    y, mean, rstd = mb.ln_fwd(t["x"], t["gamma"], t["beta"], EPS)
    dx, dg, db = mb.ln_bwd(t["dy"], t["x"], t["gamma"], mean, rstd)
    torch.cuda.synchronize()
    check_fwd(orc, t["x"], t["gamma"], t["beta"], y, mean, rstd, FMT[dtype])
    check_bwd(orc, t["dy"], t["x"], t["gamma"], mean, rstd, dx, dg, db, FMT[dtype])


def test_offset_heavy_wide_rows_fp32(orc):
    # rows ~ N(1e4, 1): the shift by the row's first value keeps rstd exact
    rows, cols = 16, 40000
    case(f"staged offset rows fp32 {rows}x{cols}")
    inp, y, mean, rstd, _ = fwd_bwd(rows, cols, torch.float32, seed=9, x_mean=1e4, bwd=False)
    check_fwd(orc, inp["x"], inp["gamma"], inp["beta"], y, mean, rstd, FMT[torch.float32])


def test_wide_backward_deterministic_and_partials_paths_agree():
    rows, cols, dtype = 700, 24000, torch.bfloat16
    case(f"staged backward determinism {rows}x{cols}")
    inp = dev(synth.layer_inputs(rows, cols, dtype, seed=11))
    _, mean, rstd = mb.ln_fwd(inp["x"], inp["gamma"], inp["beta"], EPS)
    ref = mb.ln_bwd(inp["dy"], inp["x"], inp["gamma"], mean, rstd)
    for _ in range(5):
        got = mb.ln_bwd(inp["dy"], inp["x"], inp["gamma"], mean, rstd)
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
    # stage 1 alone (partials only) gives the fused path's dgamma/dbeta bits
    ws = mb.workspace(rows, cols, inp["x"].device)
    dg, db = mb.ln_bwd_dgamma_dbeta(ws, rows, cols, dtype, partials_ready=False, dy=inp["dy"],
                                    x=inp["x"], mean=mean, rstd=rstd)
    torch.cuda.synchronize()
    assert torch.equal(dg, ref[1]) and torch.equal(db, ref[2])


@pytest.mark.parametrize("dtype", DTYPES, ids=IDS)
def test_widest_rows_large_batch_sampled(orc, dtype):
    # the widest rows at a batch that fills every workgroup several times,
    # checked on sampled rows (the column sums over all rows)
    rows, cols = 2048, MAX_BWD[dtype]
    case(f"staged widest {dtype} {rows}x{cols}")
    inp, y, mean, rstd, (dx, dg, db) = fwd_bwd(rows, cols, dtype, seed=13)
    sel = np.concatenate([np.random.default_rng(1).choice(rows, 12, replace=False),
                          [0, rows - 1]])
    t = torch.as_tensor(sel, device="cuda")
    check_fwd(orc, inp["x"][t], inp["gamma"], inp["beta"], y[t], mean[t], rstd[t], FMT[dtype])
    check_bwd(orc, inp["dy"][t], inp["x"][t], inp["gamma"], mean[t], rstd[t], dx[t], None,
              None, FMT[dtype])
    # dbeta is the plain column sum of dy: its oracle needs no statistics
    dy64 = f64(inp["dy"])
    assert_reports(cmp.check_colsum("wide.dbeta", f64(db), dy64.sum(axis=0),
                                    np.abs(dy64).sum(axis=0), rows, FMT[dtype]))


@pytest.mark.parametrize("cols", [40001, 65536])
def test_fused_forward_wide_in_place(orc, cols):
    # fp32 rows past the stage: the slots beyond it are read again in later
    # passes, also when z overwrites the residual (residual_out == residual)
    rows, dtype = 6, torch.float32
    case(f"staged fused forward in place fp32 {rows}x{cols}")
    inp = dev(synth.layer_inputs(rows, cols, dtype, seed=cols + 4))
    z, y, mean, rstd, mask = mb.bias_dropout_residual_ln_fwd(
        inp["x"], inp["bias"], inp["residual"], inp["gamma"], inp["beta"], 0.1, 17, EPS,
        want_mask=True)
    res = inp["residual"].clone()
    z2, y2, mean2, rstd2, _ = mb.bias_dropout_residual_ln_fwd(
        inp["x"], inp["bias"], res, inp["gamma"], inp["beta"], 0.1, 17, EPS, residual_out=res)
    torch.cuda.synchronize()
    assert z2.data_ptr() == res.data_ptr()
    for a, b in ((z, z2), (y, y2), (mean, mean2), (rstd, rstd2)):
        assert torch.equal(a, b)
    check_fused(orc, inp, 0.1, 17, z, y, mean, rstd, mask, FMT[dtype])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_wide_config_shape_on_the_staged_path(orc, dtype):
    # the wide-rows workload (4096 x 16384) forced onto the LDS-staged kernels
    # (the register layouts take it by default), checked on sampled rows; the
    # column sums over all rows through dbeta
    rows, cols = 4096, 16384
    case(f"forced staged path {dtype} {rows}x{cols}")
    mb.debug_force_staged(True)
    inp, y, mean, rstd, (dx, dg, db) = fwd_bwd(rows, cols, dtype, seed=21)
    mb.debug_force_staged(False)
    sel = np.concatenate([np.random.default_rng(2).choice(rows, 10, replace=False),
                          [0, rows - 1]])
    t = torch.as_tensor(sel, device="cuda")
    check_fwd(orc, inp["x"][t], inp["gamma"], inp["beta"], y[t], mean[t], rstd[t], FMT[dtype])
    check_bwd(orc, inp["dy"][t], inp["x"][t], inp["gamma"], mean[t], rstd[t], dx[t], None,
              None, FMT[dtype])
    dy64 = f64(inp["dy"])
    assert_reports(cmp.check_colsum("wide.cfg.dbeta", f64(db), dy64.sum(axis=0),
                                    np.abs(dy64).sum(axis=0), rows, FMT[dtype]))
