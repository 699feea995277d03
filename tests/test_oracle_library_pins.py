"""Pins of the float64 oracle against library routines (CPU only).

The LayerNorm, RMSNorm and softmax definitions the oracle writes out are
also PyTorch's: ``torch.nn.functional.layer_norm`` (biased variance, eps
inside the root), ``torch.nn.functional.rms_norm`` (eps inside the root) and
``torch.softmax``.  Run in float64 on the CPU with autograd, they give the
forward values and every gradient of the backward -- dx, dgamma, dbeta --
by an implementation that shares nothing with the oracle's C code.  The
oracle's backward entry points take saved statistics: the oracle's own mean
and rstd, first checked equal to the library's, and for the softmax the
library's y.  eps is a
float32 argument of the library (and so of the oracle), so the library
routines get its float32 value: at one or two columns dx is proportional to
eps, and 1e-5 in float64 differs from it by 2.5e-8 relative.
"""
import numpy as np
import pytest
import torch

import oracle as orc

F = torch.nn.functional
RTOL, ATOL = 1e-11, 1e-12


def close(name, got, ref):
    ref = ref.detach().numpy() if torch.is_tensor(ref) else ref
    assert np.allclose(got, ref, rtol=RTOL, atol=ATOL), \
        f"{name}: max |diff| {np.max(np.abs(got - ref)):.3e}"


def data(rows, cols, seed, mean=0.0):
    g = np.random.default_rng(seed)
    x = g.normal(mean, 1.0, (rows, cols))
    gamma = g.uniform(0.5, 1.5, cols)
    beta = g.normal(0.0, 0.1, cols)
    dy = g.normal(0.0, 1.0, (rows, cols))
    return x, gamma, beta, dy


@pytest.mark.parametrize("rows,cols,mean", [(7, 1, 0.0), (5, 2, 0.0), (9, 33, 0.0),
                                            (4, 768, 0.0), (3, 1000, 3.0)])
def test_layernorm_against_torch(rows, cols, mean):
    x, gamma, beta, dy = data(rows, cols, 11 + cols, mean)
    eps = float(np.float32(1e-5))
    xt = torch.tensor(x, requires_grad=True)
    gt = torch.tensor(gamma, requires_grad=True)
    bt = torch.tensor(beta, requires_grad=True)
    yt = F.layer_norm(xt, (cols,), gt, bt, eps)
    yt.backward(torch.tensor(dy))
    y, mu, rs = orc.ln_fwd(x, gamma, beta, eps)
    close("y", y, yt)
    close("mean", mu, torch.tensor(x).mean(dim=1))
    var = torch.tensor(x).var(dim=1, unbiased=False)
    close("rstd", rs, 1.0 / torch.sqrt(var + eps))
    # the backward from the oracle's saved statistics (checked equal above)
    for form in ("hw4", "slides"):
        close(f"dx[{form}]", orc.ln_bwd_dx(dy, x, gamma, mu, rs, form=form), xt.grad)
    dg, db, _, _ = orc.ln_bwd_params(dy, x, mu, rs)
    close("dgamma", dg, gt.grad)
    close("dbeta", db, bt.grad)


@pytest.mark.parametrize("rows,cols", [(6, 1), (5, 3), (8, 64), (3, 4096)])
def test_rmsnorm_against_torch(rows, cols):
    x, gamma, _, dy = data(rows, cols, 21 + cols)
    eps = float(np.float32(1e-6))
    xt = torch.tensor(x, requires_grad=True)
    gt = torch.tensor(gamma, requires_grad=True)
    yt = F.rms_norm(xt, (cols,), gt, eps)
    yt.backward(torch.tensor(dy))
    y, rs = orc.rmsnorm_fwd(x, gamma, eps)
    close("y", y, yt)
    dx, dg, _ = orc.rmsnorm_bwd(dy, x, gamma, rs)
    close("dx", dx, xt.grad)
    close("dgamma", dg, gt.grad)


@pytest.mark.parametrize("rows,cols,scale,masked", [(4, 1, 1.0, False), (6, 17, 0.125, False),
                                                    (8, 256, 0.5, True), (2, 4096, 1.0, True)])
def test_softmax_against_torch(rows, cols, scale, masked):
    g = np.random.default_rng(31 + cols)
    x = g.normal(0.0, 3.0, (rows, cols))
    dy = g.normal(0.0, 1.0, (rows, cols))
    mask = None
    if masked:
        mask = np.where(g.random((1, cols)) < 0.25, -np.inf, g.normal(0.0, 1.0, (1, cols)))
        mask[0, 0] = 0.0                      # at least one key in play
    xt = torch.tensor(x, requires_grad=True)
    t = scale * xt
    if masked:
        t = t + torch.tensor(mask)
    yt = torch.softmax(t, dim=1)
    yt.backward(torch.tensor(dy))
    y = orc.attn_softmax_fwd(x, scale=scale, mask=mask, rows_per_mask=rows, causal=False)
    close("y", y, yt)
    dx = orc.attn_softmax_bwd(dy, yt.detach().numpy(), scale=scale)
    close("dx", dx, xt.grad)
