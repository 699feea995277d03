"""GPU parity at tensor sizes beyond 2^31 elements (64-bit row offsets in
every kernel): sampled rows -- the first, some in the middle, both sides of
row 2^21 and the last -- checked against the float64 oracle with the same
helpers as the other parity tests.  Inputs are drawn on the GPU from a
seeded torch generator (the host-side generator would need tens of GB of
host memory at these sizes); parameters come from the shared generator."""
import numpy as np
import pytest
import torch

import memory_bound_row_amd as mb
from memory_bound_row_amd import synth
from oracle import compare as cmp
from gpu_helpers import (EPS, FMT, assert_reports, case, check_bwd, check_fwd,
                         check_rmsnorm_fwd, check_softmax_bwd, check_softmax_fwd, check_xent,
                         f64)

pytestmark = pytest.mark.gpu

COLS = 1024


def big(rows, cols, dtype, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn((rows, cols), generator=g, device="cuda", dtype=torch.float32).to(dtype)


def sample(rows):
    idx = [0, 1, 2, rows // 2, rows // 2 + 1, (1 << 21) - 1, 1 << 21, rows - 2, rows - 1]
    return torch.as_tensor(idx, device="cuda")


def params(names, dtype, seed):
    return {k: v.to("cuda") for k, v in synth.layer_inputs(1, COLS, dtype, seed=seed,
                                                            names=names).items()}


def test_layernorm_beyond_2g_elements(orc):
    rows = (1 << 21) + 3          # 2^31 + 3072 elements
    case(f"LayerNorm fwd + bwd {rows}x{COLS} bf16")
    dt = torch.bfloat16
    x, dy = big(rows, COLS, dt, 1), big(rows, COLS, dt, 2)
    p = params(("gamma", "beta"), dt, 3)
    y, mean, rstd = mb.ln_fwd(x, p["gamma"], p["beta"], EPS)
    dx, dg, db = mb.ln_bwd(dy, x, p["gamma"], mean, rstd)
    torch.cuda.synchronize()
    i = sample(rows)
    check_fwd(orc, x[i], p["gamma"], p["beta"], y[i], mean[i], rstd[i], FMT[dt], name="big.ln")
    check_bwd(orc, dy[i], x[i], p["gamma"], mean[i], rstd[i], dx[i], None, None, FMT[dt],
              name="big.ln_bwd")
    assert torch.isfinite(dg).all() and torch.isfinite(db).all()


def test_fused_forward_beyond_2g_elements(orc):
    rows = (1 << 21) + 3
    case(f"fused forward {rows}x{COLS} bf16 p=0.1")
    dt = torch.bfloat16
    x, res = big(rows, COLS, dt, 4), big(rows, COLS, dt, 5)
    p = params(("bias", "gamma", "beta"), dt, 6)
    seed = 77
    z, y, mean, rstd, _ = mb.bias_dropout_residual_ln_fwd(x, p["bias"], res, p["gamma"],
                                                          p["beta"], 0.1, seed, EPS)
    torch.cuda.synchronize()
    i = sample(rows)
    # the oracle's mask at the sampled rows
    keep = np.stack([orc.dropout_keep_rows(seed, 0.1, int(r), 1, COLS)[0] for r in i.cpu()])
    z_ref = orc.bias_dropout_residual(f64(x[i]), f64(p["bias"]), f64(res[i]), keep, 0.1)
    assert_reports(cmp.check_elementwise("big.fused.z", f64(z[i]), z_ref, FMT[dt]))
    check_fwd(orc, z[i], p["gamma"], p["beta"], y[i], mean[i], rstd[i], FMT[dt],
              name="big.fused.ln")


def test_softmax_beyond_2g_elements(orc):
    rows = (1 << 21) + 5
    case(f"softmax fwd + bwd {rows}x{COLS} fp16")
    dt = torch.float16
    x, dy = big(rows, COLS, dt, 7), big(rows, COLS, dt, 8)
    y, _ = mb.attn_softmax_fwd(x, 0.5)
    dx = mb.attn_softmax_bwd(dy, y, 0.5)
    torch.cuda.synchronize()
    i = sample(rows)
    check_softmax_fwd(orc, x[i], y[i], None, FMT[dt], scale=0.5, name="big.sm")
    check_softmax_bwd(orc, dy[i], y[i], dx[i], FMT[dt], scale=0.5, name="big.sm_bwd")


def test_rmsnorm_and_xent_beyond_2g_elements(orc):
    rows = (1 << 21) + 7
    case(f"add+RMSNorm fwd, cross-entropy {rows}x{COLS} bf16")
    dt = torch.bfloat16
    x, res = big(rows, COLS, dt, 9), big(rows, COLS, dt, 10)
    gamma = params(("gamma",), dt, 11)["gamma"]
    z, y, rstd = mb.add_rmsnorm_fwd(x, gamma, 1e-6, residual=res)
    torch.cuda.synchronize()
    i = sample(rows)
    check_rmsnorm_fwd(orc, x[i], res[i], gamma, z[i], y[i], rstd[i], FMT[dt], 1e-6,
                      name="big.rms")
    del z, y, res
    lab = torch.randint(0, COLS, (rows,), device="cuda",
                        generator=torch.Generator(device="cuda").manual_seed(12))
    loss, dx = mb.cross_entropy_fwd_bwd(x, lab, label_smoothing=0.1, grad_scale=1.0)
    torch.cuda.synchronize()
    check_xent(orc, x[i], lab[i], COLS, 0.1, 1.0, loss[i], dx[i], FMT[dt], name="big.xent")


def test_staged_layernorm_beyond_2g_elements(orc):
    # rows past the register layouts, staged in LDS: 2^31 + 32768 elements
    rows, cols = (1 << 16) + 1, 32768
    case(f"LDS-staged LayerNorm fwd + bwd {rows}x{cols} bf16")
    dt = torch.bfloat16
    x, dy = big(rows, cols, dt, 13), big(rows, cols, dt, 14)
    p = {k: v.to("cuda") for k, v in synth.layer_inputs(1, cols, dt, seed=15,
                                                         names=("gamma", "beta")).items()}
    y, mean, rstd = mb.ln_fwd(x, p["gamma"], p["beta"], EPS)
    dx, dg, db = mb.ln_bwd(dy, x, p["gamma"], mean, rstd)
    torch.cuda.synchronize()
    i = torch.as_tensor([0, 1, rows // 2, (1 << 16) - 1, 1 << 16], device="cuda")
    check_fwd(orc, x[i], p["gamma"], p["beta"], y[i], mean[i], rstd[i], FMT[dt],
              name="big.staged")
    check_bwd(orc, dy[i], x[i], p["gamma"], mean[i], rstd[i], dx[i], None, None, FMT[dt],
              name="big.staged_bwd")
    assert torch.isfinite(dg).all() and torch.isfinite(db).all()


def test_two_pass_beyond_2g_elements(orc):
    # the widest rows (2^24 columns) on the two-pass path: 2^31 + 2^24 elements
    rows, cols = 129, 1 << 24
    case(f"two-pass softmax fwd + bwd, cross-entropy {rows}x{cols}")
    dt = torch.float16
    x, dy = big(rows, cols, dt, 16), big(rows, cols, dt, 17)
    y, _ = mb.attn_softmax_fwd(x, 0.5)
    dx = mb.attn_softmax_bwd(dy, y, 0.5)
    torch.cuda.synchronize()
    i = torch.as_tensor([0, 64, rows - 1], device="cuda")
    check_softmax_fwd(orc, x[i], y[i], None, FMT[dt], scale=0.5, name="big.stream.sm")
    check_softmax_bwd(orc, dy[i], y[i], dx[i], FMT[dt], scale=0.5, name="big.stream.sm_bwd")
    del y, dy, dx
    lab = torch.randint(0, cols, (rows,), device="cuda",
                        generator=torch.Generator(device="cuda").manual_seed(18))
    loss, dl = mb.cross_entropy_fwd_bwd(x, lab, label_smoothing=0.1, grad_scale=1.0)
    torch.cuda.synchronize()
    check_xent(orc, x[i], lab[i], cols, 0.1, 1.0, loss[i], dl[i], FMT[dt],
               name="big.stream.xent")
