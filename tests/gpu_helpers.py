"""Shared steps of the GPU parity tests: run the HIP library through its
binding, run the float64 oracle on the same stored values, compare under the
tolerance rule of oracle/compare.py."""
import sys

import numpy as np
import torch

import memory_bound_row_amd as mb
from memory_bound_row_amd import synth
from oracle import compare as cmp

FMT = {torch.float32: cmp.F32, torch.float16: cmp.F16, torch.bfloat16: cmp.BF16}
EPS = 1e-5


def case(msg: str) -> None:
    """Name the case on stderr before its GPU work starts."""
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def dev(d: dict) -> dict:
    return {k: v.to("cuda") for k, v in d.items()}


def f64(t) -> np.ndarray:
    return synth.as_f64(t)


def assert_reports(*reports):
    bad = [r for r in reports if not r.ok]
    msg = "\n".join(str(r) + (f" first failures: {r.details}" if r.details else "")
                    for r in reports)
    assert not bad, msg
    return reports


def assert_no_wide(reports):
    """No output needed a clause wider than the headline max-abs bound."""
    wide = [str(r) for r in reports if r.n_wide]
    assert not wide, "wider tolerance clause used:\n" + "\n".join(wide)


def check_fwd(orc, x, gamma, beta, y, mean, rstd, fmt, eps=EPS, name="fwd", strict=False):
    """`strict`: also require that no element needed a wider clause than the
    headline max-abs bound (the fp32 configurations meet it outright)."""
    y_ref, mu_ref, rs_ref = orc.ln_fwd(f64(x).reshape(-1, x.shape[-1]), f64(gamma),
                                       f64(beta), eps)
    reps = [cmp.check_elementwise(f"{name}.y", f64(y).reshape(y_ref.shape), y_ref, fmt)]
    if mean is not None:
        reps.append(cmp.check_stats(f"{name}.mean", f64(mean), mu_ref))
        reps.append(cmp.check_stats(f"{name}.rstd", f64(rstd), rs_ref))
    assert_reports(*reps)
    if strict:
        assert_no_wide(reps)
    return reps


def check_bwd(orc, dy, x, gamma, mean, rstd, dx, dgamma, dbeta, fmt, name="bwd",
              strict=False):
    """Reference dx, dgamma, dbeta from the stored inputs and the stored fp32
    mean/rstd the GPU read.  `strict`: dx needs no wider clause, and the
    column sums also meet the statistical bound of cmp.check_colsum_stat."""
    rows, cols = x.shape[0], x.shape[-1]
    dy64, x64 = f64(dy).reshape(rows, cols), f64(x).reshape(rows, cols)
    mu64, rs64 = f64(mean), f64(rstd)
    reps = []
    if dx is not None:
        dx_ref = orc.ln_bwd_dx(dy64, x64, f64(gamma), mu64, rs64)
        scale = orc.ln_bwd_dx_scale(dy64, x64, f64(gamma), mu64, rs64)
        reps.append(cmp.check_elementwise(f"{name}.dx", f64(dx).reshape(rows, cols),
                                          dx_ref, fmt, term_scale=scale, row_len=cols))
    if dgamma is not None:
        dg, db, sg, sb = orc.ln_bwd_params(dy64, x64, mu64, rs64)
        reps.append(cmp.check_colsum(f"{name}.dgamma", f64(dgamma), dg, sg, rows, fmt))
        reps.append(cmp.check_colsum(f"{name}.dbeta", f64(dbeta), db, sb, rows, fmt))
    assert_reports(*reps)
    if strict:
        if dx is not None:
            assert_no_wide(reps[:1])
        if dgamma is not None:
            xh = (x64 - mu64[:, None]) * rs64[:, None]
            assert_reports(
                cmp.check_colsum_stat(f"{name}.dgamma.stat", f64(dgamma), dg,
                                      np.sum((dy64 * xh) ** 2, axis=0), rows),
                cmp.check_colsum_stat(f"{name}.dbeta.stat", f64(dbeta), db,
                                      np.sum(dy64 ** 2, axis=0), rows))
    return reps


def check_fused(orc, inp, p, seed, z, y, mean, rstd, mask, fmt, eps=EPS, name="fused"):
    rows, cols = inp["x"].shape
    keep = orc.dropout_keep(seed, p, rows, cols)
    reps = []
    if mask is not None:
        m = mask.cpu().numpy()
        n_diff = int(np.count_nonzero(m != keep))
        assert n_diff == 0, f"{name}: {n_diff} mask bits differ from the oracle"
    z_ref = orc.bias_dropout_residual(f64(inp["x"]), f64(inp["bias"]), f64(inp["residual"]),
                                      keep, p)
    reps.append(cmp.check_elementwise(f"{name}.z", f64(z), z_ref, fmt))
    # the LayerNorm runs on z as stored
    reps += list(check_fwd(orc, z, inp["gamma"], inp["beta"], y, mean, rstd, fmt, eps,
                           name=f"{name}.ln"))
    return assert_reports(*reps)


def check_dropout_bwd(orc, dy, dz_extra, z, gamma, mean, rstd, p, seed, dres, dx, dgamma,
                      dbeta, dbias, fmt, name="drop_bwd"):
    """Reference of the prologue backward from the stored inputs: dz = the
    LayerNorm's dx + dz_extra, dresidual = dz, dx = keep * dz / (1 - p),
    dbias = column sums of dx; dgamma, dbeta as for the LayerNorm backward.
    The GPU forms dz in float32 (the dx clause of the tolerance rule, plus one
    rounding of the dz_extra add) and scales it by 1/(1 - p) before rounding;
    dbias sums those float32 values."""
    import math
    rows, cols = z.shape[0], z.shape[-1]
    dy64, z64 = f64(dy).reshape(rows, cols), f64(z).reshape(rows, cols)
    mu64, rs64, g64 = f64(mean), f64(rstd), f64(gamma)
    ez64 = np.zeros_like(dy64) if dz_extra is None else f64(dz_extra).reshape(rows, cols)
    dz = orc.ln_bwd_dx(dy64, z64, g64, mu64, rs64) + ez64
    scale = orc.ln_bwd_dx_scale(dy64, z64, g64, mu64, rs64) + np.abs(ez64)
    keep = orc.dropout_keep(seed, p, rows, cols)
    dx_ref, dbias_ref, sbias = orc.dropout_residual_bwd(dz, keep, p)
    s = 1.0 / (1.0 - np.float64(np.float32(p)))
    dx_scale = scale * s * keep
    k = 4 + math.ceil(math.log2(max(cols, 2)))
    bias_err = np.sum(k * 2.0 ** -24 * dx_scale, axis=0)
    dg, db, sg, sb = orc.ln_bwd_params(dy64, z64, mu64, rs64)
    reps = [
        cmp.check_elementwise(f"{name}.dresidual", f64(dres).reshape(rows, cols), dz, fmt,
                              term_scale=scale, row_len=cols),
        cmp.check_elementwise(f"{name}.dx", f64(dx).reshape(rows, cols), dx_ref, fmt,
                              term_scale=dx_scale, row_len=cols),
        cmp.check_colsum(f"{name}.dgamma", f64(dgamma), dg, sg, rows, fmt),
        cmp.check_colsum(f"{name}.dbeta", f64(dbeta), db, sb, rows, fmt),
        cmp.check_colsum(f"{name}.dbias", f64(dbias), dbias_ref, sbias, rows, fmt,
                         term_err=bias_err),
    ]
    # dropped positions carry exactly no gradient
    dropped = f64(dx).reshape(rows, cols)[keep == 0]
    assert np.all(dropped == 0.0), f"{name}: nonzero dx at dropped positions"
    return assert_reports(*reps)


def softmax_refs(orc, x, mask, rows_per_mask, causal, scale):
    """Oracle y of the stored scores and the size of the float32 terms behind
    each y_j (|t_j| + |max t| + 1 in units of y_j: the exponent's rounding and
    the exp, sum and divide), for the arithmetic clause."""
    rows, cols = x.shape
    x64 = f64(x)
    m64 = None if mask is None else f64(mask).reshape(-1, cols)
    y_ref = orc.attn_softmax_fwd(x64, scale=scale, mask=m64, rows_per_mask=rows_per_mask,
                                 causal=causal)
    t = np.float64(np.float32(scale)) * x64
    if m64 is not None:
        t = t + np.repeat(m64, rows_per_mask, axis=0)[:rows]
    finite = np.where(np.isfinite(t), t, 0.0)
    mx = np.max(np.where(y_ref > 0, finite, -np.inf), axis=1, keepdims=True)
    mx = np.where(np.isfinite(mx), mx, 0.0)
    y_scale = y_ref * (1.0 + np.abs(finite) + np.abs(mx))
    return y_ref, y_scale


def check_softmax_fwd(orc, x, y, y_dropped, fmt, scale=1.0, mask=None, rows_per_mask=1,
                      causal=False, p=0.0, seed=0, name="softmax"):
    rows, cols = x.shape
    y_ref, y_scale = softmax_refs(orc, x, mask, rows_per_mask, causal, scale)
    reps = [cmp.check_scaled(f"{name}.y", f64(y), y_ref, fmt, term_scale=y_scale,
                             row_len=cols)]
    if y_dropped is not None:
        keep = orc.dropout_keep(seed, p, rows, cols)
        s = 1.0 / (1.0 - np.float64(np.float32(p)))
        reps.append(cmp.check_scaled(f"{name}.y_dropped", f64(y_dropped),
                                     np.where(keep == 1, y_ref * s, 0.0), fmt,
                                     term_scale=y_scale * s * keep, row_len=cols))
        yd = f64(y_dropped)
        assert np.all(yd[keep == 0] == 0.0), f"{name}: dropped positions not zero"
    return assert_reports(*reps)


def check_softmax_bwd(orc, dy, y, dx, fmt, scale=1.0, p=0.0, seed=0, name="softmax_bwd",
                      row_ids=None):
    """Reference dx from the stored dy and the GPU's stored y.  row_ids: the
    rows' indices in the tensor the kernel ran on, when these are sampled
    rows (the dropout mask depends on the row index)."""
    rows, cols = y.shape
    dy64, y64 = f64(dy), f64(y)
    keep = None
    if p > 0:
        keep = (orc.dropout_keep(seed, p, rows, cols) if row_ids is None else
                np.concatenate([orc.dropout_keep_rows(seed, p, int(r), 1, cols)
                                for r in row_ids]))
    dx_ref = orc.attn_softmax_bwd(dy64, y64, keep=keep, p=p, scale=scale)
    s = 1.0 / (1.0 - np.float64(np.float32(p)))
    g = dy64 * s if keep is None else np.where(keep == 1, dy64 * s, 0.0)
    term = abs(scale) * y64 * (np.abs(g) + np.sum(np.abs(g * y64), axis=1, keepdims=True))
    return assert_reports(cmp.check_scaled(f"{name}.dx", f64(dx), dx_ref, fmt,
                                           term_scale=term, row_len=cols))


def check_rmsnorm_fwd(orc, x, residual, gamma, z, y, rstd, fmt, eps, name="rms"):
    """Reference z = x + residual (rounded once to T; the GPU adds in float32
    and rounds, which for two T values stays within the rounding clause) and
    the RMSNorm of z as stored.  y carries the float32 error of rstd (a sum of
    m squares), so the arithmetic clause takes |y| as the size of its terms."""
    rows, cols = x.shape[0], x.shape[-1]
    reps = []
    if residual is not None:
        zero = np.zeros(cols)
        keep = np.ones((rows, cols), dtype=np.uint8)
        z_ref = orc.bias_dropout_residual(f64(x), zero, f64(residual), keep, 0.0)
        reps.append(cmp.check_elementwise(f"{name}.z", f64(z), z_ref, fmt))
    y_ref, rs_ref = orc.rmsnorm_fwd(f64(z).reshape(rows, cols), f64(gamma), eps)
    reps.append(cmp.check_elementwise(f"{name}.y", f64(y).reshape(rows, cols), y_ref, fmt,
                                      term_scale=np.abs(y_ref), row_len=cols))
    if rstd is not None:
        reps.append(cmp.check_stats(f"{name}.rstd", f64(rstd), rs_ref))
    return assert_reports(*reps)


def check_rmsnorm_bwd(orc, dy, dz_extra, z, gamma, rstd, dz, dgamma, fmt, name="rms_bwd"):
    """Reference dz = RMSNorm dx (from the stored dy, z and fp32 rstd the GPU
    read) + dz_extra, and dgamma.  The size of dx's float32 terms is
    rstd * (|g| + |xhat| * sum|g * xhat| / m), g = gamma * dy, plus |dz_extra|."""
    rows, cols = z.shape[0], z.shape[-1]
    dy64, z64 = f64(dy).reshape(rows, cols), f64(z).reshape(rows, cols)
    rs64, g64 = f64(rstd), f64(gamma)
    ez64 = np.zeros_like(dy64) if dz_extra is None else f64(dz_extra).reshape(rows, cols)
    dx_ref, dg_ref, sg = orc.rmsnorm_bwd(dy64, z64, g64, rs64)
    g = g64 * dy64
    xh = z64 * rs64[:, None]
    scale = rs64[:, None] * (np.abs(g) + np.abs(xh) * np.sum(np.abs(g * xh), axis=1,
                                                              keepdims=True) / cols)
    reps = [
        cmp.check_elementwise(f"{name}.dz", f64(dz).reshape(rows, cols), dx_ref + ez64, fmt,
                              term_scale=scale + np.abs(ez64), row_len=cols),
        cmp.check_colsum(f"{name}.dgamma", f64(dgamma), dg_ref, sg, rows, fmt),
    ]
    return assert_reports(*reps)


def check_xent(orc, logits, labels, cols, alpha, scale, loss, dx, fmt, rows_sel=None,
               name="xent"):
    """Reference loss and gradient of the stored logits (the first `cols`
    columns of each row; rows_sel restricts the check to those rows).  The
    kernel's float32 terms: the exp-sum over V values and the exp arguments
    x - m (up to max|x - m|), the sums of x; so the loss is checked against
    the arithmetic clause with S = 1 + |log Z| + |m - x_label| + a (|m| +
    sum|x| / V) + max|x - m|, and q_j against q_j (1 + |x_j - m| + max|x - m|)
    + p_j.  The gradient's padding columns must be exactly 0."""
    x_all = f64(logits)
    lab_all = labels.cpu().numpy()
    rows_idx = np.arange(x_all.shape[0]) if rows_sel is None else np.asarray(rows_sel)
    x64 = np.ascontiguousarray(x_all[rows_idx, :cols])
    lab = lab_all[rows_idx]
    loss_ref, dx_ref = orc.cross_entropy(x64, lab, alpha, scale, grad=dx is not None)
    a = float(np.float32(alpha))
    valid = (lab >= 0) & (lab < cols)
    m = x64.max(axis=1)
    spread = np.max(np.abs(x64 - m[:, None]), axis=1)
    z = np.sum(np.exp(x64 - m[:, None]), axis=1)
    xl = np.where(valid, x64[np.arange(len(lab)), np.clip(lab, 0, cols - 1)], 0.0)
    s_loss = (1.0 + np.abs(np.log(z)) + np.abs(m - xl)
              + a * (np.abs(m) + np.sum(np.abs(x64), axis=1) / cols) + spread)
    s_loss = np.where(valid, s_loss, 0.0)
    got_loss = f64(loss)[rows_idx]
    reps = [cmp.check_elementwise(f"{name}.loss", got_loss, loss_ref, cmp.F32,
                                  term_scale=s_loss, row_len=cols)]
    if dx is not None:
        q = np.exp(x64 - m[:, None]) / z[:, None]
        p = np.full_like(q, a / cols)
        p[np.arange(len(lab))[valid], lab[valid]] += 1.0 - a
        term = abs(float(np.float32(scale))) * (
            q * (1.0 + np.abs(x64 - m[:, None]) + spread[:, None]) + p)
        term = np.where(valid[:, None], term, 0.0)
        d_all = f64(dx)
        reps.append(cmp.check_scaled(f"{name}.dx", d_all[rows_idx, :cols], dx_ref, fmt,
                                     term_scale=term, row_len=cols))
        if d_all.shape[1] > cols:
            pad = d_all[rows_idx, cols:]
            assert np.all(pad == 0.0), f"{name}: nonzero gradient in padding columns"
    return assert_reports(*reps)


def run_fwd_bwd(rows, cols, dtype, seed=0, x_mean=0.0, x_std=1.0):
    inp = dev(synth.layer_inputs(rows, cols, dtype, seed=seed, x_mean=x_mean, x_std=x_std,
                                 names=("x", "gamma", "beta", "dy")))
    y, mean, rstd = mb.ln_fwd(inp["x"], inp["gamma"], inp["beta"], EPS)
    dx, dg, db = mb.ln_bwd(inp["dy"], inp["x"], inp["gamma"], mean, rstd)
    torch.cuda.synchronize()
    return inp, y, mean, rstd, dx, dg, db
