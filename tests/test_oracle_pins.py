"""Pins of the float64 oracle against what the pages and mathematics fix.

CPU only.  Each test checks the oracle against something other than itself:
values printed on the pages (tests/golden), closed forms, identities, finite
differences, an independent algorithm, or a library routine for a special
case.  The Philox4x32-10 function itself is pinned in tests/test_philox_pin.py
against an independent implementation of the published generator; its
layout and statistics are pinned here.
"""
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(rng, rows, m, mean=0.0, std=1.0):
    return rng.normal(mean, std, size=(rows, m))


# --------------------------------------------------------------------------
# Storage rounding: "GPU Performance from First Principles" §7.1 and ex. 6
# --------------------------------------------------------------------------

def _golden_rounding():
    out = []
    with open(os.path.join(GOLDEN, "storage_rounding.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            digits = int(parts[3]) if len(parts) > 3 else None
            out.append((parts[0], float(parts[1]), float(parts[2]), digits))
    return out


@pytest.mark.parametrize("fmt,value,stored,digits", _golden_rounding())
def test_rounding_golden(orc, fmt, value, stored, digits):
    got = orc.round_scalar(value, fmt)
    if digits is None:
        assert got == stored
    else:
        assert float(f"{got:.{digits}g}") == stored


def test_rounding_bf16_exact_integers(orc):
    # BF16 holds every integer up to 2^8 = 256, FP16 up to 2^11 = 2048 (ex. 6)
    ints = np.arange(0, 257, dtype=np.float64)
    assert np.array_equal(orc.round_to(ints, "bf16"), ints)
    ints16 = np.arange(0, 2049, dtype=np.float64)
    assert np.array_equal(orc.round_to(ints16, "f16"), ints16)
    assert orc.round_scalar(2049.0, "f16") == 2048.0      # tie to even
    assert orc.round_scalar(2051.0, "f16") == 2052.0      # tie to even (up)


def test_rounding_ties_and_overflow(orc):
    one = 1.0
    assert orc.round_scalar(one + 2.0 ** -8, "bf16") == one            # tie -> even
    assert orc.round_scalar(one + 3 * 2.0 ** -8, "bf16") == one + 2.0 ** -6
    assert orc.round_scalar(one + 2.0 ** -24, "f32") == one
    assert orc.round_scalar(16777217.0, "f32") == 16777216.0
    assert orc.round_scalar(65519.0, "f16") == 65504.0
    assert math.isinf(orc.round_scalar(65520.0, "f16"))                 # tie at max
    assert math.isnan(orc.round_scalar(float("nan"), "bf16"))
    assert orc.round_scalar(-0.1, "bf16") == -orc.round_scalar(0.1, "bf16")


def test_rounding_matches_library_conversions(orc):
    # Special cases that reduce to library routines: numpy's float64->float16
    # and float64->float32 casts, and torch's float32->bfloat16 cast (all
    # round to nearest even).
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 1e4, 20000),
                        rng.uniform(-6.5e4, 6.5e4, 5000), rng.normal(0, 1e-6, 5000)])
    assert np.array_equal(orc.round_to(v, "f16"), v.astype(np.float16).astype(np.float64))
    assert np.array_equal(orc.round_to(v, "f32"), v.astype(np.float32).astype(np.float64))
    v32 = v.astype(np.float32).astype(np.float64)    # exact fp32 values
    ref = torch.from_numpy(v32.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(orc.round_to(v32, "bf16"), ref)


# --------------------------------------------------------------------------
# Forward: "Accelerating Transformer on GPU (II)" §2.1, "(I)" §4.2
# --------------------------------------------------------------------------

def _golden_kv(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.startswith("#") or "=" not in line:
                continue
            k, v = line.split("=")
            d[k.strip()] = [float(t) for t in v.split()]
    return d


def test_forward_worked_example_1000_1001(orc):
    g = _golden_kv("variance_1000_1001.txt")
    x = np.array([g["x"]])
    eps = 1e-5
    y, mean, rstd = orc.ln_fwd(x, np.ones(2), np.zeros(2), eps)
    assert mean[0] == g["mean"][0]
    var = 1.0 / rstd[0] ** 2 - float(np.float32(eps))
    assert abs(var - g["var"][0]) < 1e-12
    # the printed intermediates of the E[x^2] - E[x]^2 route
    assert g["mean"][0] ** 2 == g["mean_squared"][0]
    assert np.mean(x ** 2) == g["mean_of_squares"][0]
    expect = 0.5 / math.sqrt(0.25 + float(np.float32(eps)))
    assert np.allclose(y[0], [-expect, expect], rtol=0, atol=1e-15)


def test_forward_closed_form_small_row(orc):
    # x = (1, 2, 3, 4): mean 2.5, population variance 1.25
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    gamma = np.array([2.0, 1.0, 0.5, -1.0])
    beta = np.array([0.0, 0.25, -0.5, 1.0])
    eps = 0.0
    y, mean, rstd = orc.ln_fwd(x, gamma, beta, eps)
    assert mean[0] == 2.5
    assert abs(rstd[0] - 1 / math.sqrt(1.25)) < 1e-15
    xhat = (x[0] - 2.5) / math.sqrt(1.25)
    assert np.allclose(y[0], gamma * xhat + beta, rtol=0, atol=1e-15)


@pytest.mark.parametrize("m", [1, 7, 64, 768, 1280])
def test_forward_normalised_rows(orc, m):
    # gamma = 1, beta = 0: each row has mean 0 and variance var/(var + eps)
    rng = np.random.default_rng(m)
    x = _rows(rng, 16, m, mean=rng.uniform(-3, 3), std=2.0)
    eps = float(np.float32(1e-5))
    y, mean, rstd = orc.ln_fwd(x, np.ones(m), np.zeros(m), 1e-5)
    var = np.var(x, axis=1)
    assert np.allclose(np.mean(y, axis=1), 0.0, atol=1e-13)
    assert np.allclose(np.var(y, axis=1), var / (var + eps), rtol=1e-12, atol=1e-15)
    assert np.allclose(mean, np.mean(x, axis=1), rtol=1e-14, atol=1e-14)


def test_forward_constant_row(orc):
    m = 33
    x = np.full((2, m), 3.25)
    beta = np.linspace(-1, 1, m)
    y, mean, rstd = orc.ln_fwd(x, np.linspace(0.5, 1.5, m), beta, 1e-5)
    assert np.array_equal(y, np.broadcast_to(beta, (2, m)))
    assert np.allclose(rstd, 1 / math.sqrt(float(np.float32(1e-5))), rtol=1e-15)


def test_welford_matches_two_pass_on_offset_rows(orc):
    # Two independent algorithms (two-pass; Welford + Chan merge, "(I)" §4.2)
    rng = np.random.default_rng(7)
    x = _rows(rng, 64, 768, mean=1e4, std=1.0)
    _, mean, rstd = orc.ln_fwd(x, np.ones(768), np.zeros(768), 0.0)
    wmean, wvar = orc.row_stats_welford(x)
    assert np.allclose(wmean, mean, rtol=1e-12, atol=0)
    assert np.allclose(wvar, 1.0 / rstd ** 2, rtol=1e-11, atol=0)


def test_fp32_naive_variance_fails_at_large_mean(orc):
    # "(I)" §4.2: with mean 10000 the fp32 E[x^2]-E[x]^2 variance collapses
    # (<= 0 or wildly wrong), while the fp32 per-lane Welford/Chan merge
    # keeps the leading digits (its running means still round at 1e4, so it
    # loses about four of fp32's seven digits here).
    rng = np.random.default_rng(11)
    x = np.float64(np.float32(_rows(rng, 32, 768, mean=1e4, std=1.0)))
    true_var = np.var(x, axis=1)
    naive = orc.var_naive_f32(x)
    chan = orc.var_chan_f32(x, lanes=64)
    rel_naive = np.abs(naive - true_var) / true_var
    rel_chan = np.abs(chan - true_var) / true_var
    assert np.all((naive <= 0) | (rel_naive > 0.5))
    assert np.max(rel_chan) < 1e-3
    # at mean 0 the naive form is fine (the hazard is the offset)
    x0 = np.float64(np.float32(_rows(rng, 32, 768)))
    rel0 = np.abs(orc.var_naive_f32(x0) - np.var(x0, axis=1)) / np.var(x0, axis=1)
    assert np.max(rel0) < 1e-5


def test_fp32_chan_handles_ragged_lanes(orc):
    rng = np.random.default_rng(3)
    for m in (1, 5, 63, 65, 1000):
        x = np.float64(np.float32(_rows(rng, 4, m, mean=50.0, std=3.0)))
        got = orc.var_chan_f32(x, lanes=64)
        ref = np.var(x, axis=1)
        assert np.allclose(got, ref, rtol=1e-4, atol=1e-6), m


# --------------------------------------------------------------------------
# Backward: "Accelerating Transformer on GPU (II)" §2.1, exercise 2
# --------------------------------------------------------------------------

def _fwd_loss(orc, x, gamma, beta, dy, eps):
    y, _, _ = orc.ln_fwd(x, gamma, beta, eps)
    return float(np.sum(dy * y))


@pytest.mark.parametrize("m", [1, 2, 3, 5, 8])
def test_backward_finite_differences(orc, m):
    rng = np.random.default_rng(100 + m)
    rows = 3
    x = _rows(rng, rows, m, std=1.5)
    gamma = rng.uniform(0.5, 1.5, m)
    beta = rng.normal(0, 0.1, m)
    dy = _rows(rng, rows, m)
    eps = 1e-5
    _, mean, rstd = orc.ln_fwd(x, gamma, beta, eps)
    dx = orc.ln_bwd_dx(dy, x, gamma, mean, rstd, form="hw4")
    fd = np.zeros_like(x)
    for r in range(rows):
        for j in range(m):
            h = 1e-6 * max(1.0, abs(x[r, j]))
            xp, xm = x.copy(), x.copy()
            xp[r, j] += h
            xm[r, j] -= h
            fd[r, j] = (_fwd_loss(orc, xp, gamma, beta, dy, eps)
                        - _fwd_loss(orc, xm, gamma, beta, dy, eps)) / (2 * h)
    scale = max(1.0, np.max(np.abs(dx)))
    assert np.max(np.abs(fd - dx)) <= 1e-7 * scale
    if m == 1:
        assert np.all(dx == 0.0)
    # parameter gradients: L is linear in gamma and beta
    dg, db, _, _ = orc.ln_bwd_params(dy, x, mean, rstd)
    for j in range(m):
        for which, grad in (("g", dg), ("b", db)):
            gp, gm = gamma.copy(), gamma.copy()
            bp, bm = beta.copy(), beta.copy()
            if which == "g":
                gp[j] += 0.5
                gm[j] -= 0.5
            else:
                bp[j] += 0.5
                bm[j] -= 0.5
            fdp = (_fwd_loss(orc, x, gp, bp, dy, eps)
                   - _fwd_loss(orc, x, gm, bm, dy, eps)) / 1.0
            assert abs(fdp - grad[j]) <= 1e-12 * max(1.0, abs(grad[j])), (which, j)


# --------------------------------------------------------------------------
# Backward of the bias + dropout + residual prologue: the chain rule through
# the composed forward ("Accelerating Transformer on GPU (I)" §2.3 order),
# pinned by central finite differences of a scalar loss that uses both y and
# z (z also feeds the residual stream)
# --------------------------------------------------------------------------

def _fused_loss(orc, x, bias, res, keep, p, gamma, beta, dy, dzx, eps):
    z = orc.bias_dropout_residual(x, bias, res, keep, p)
    y, _, _ = orc.ln_fwd(z, gamma, beta, eps)
    return float(np.sum(dy * y) + np.sum(dzx * z))


@pytest.mark.parametrize("m", [1, 2, 3, 5, 8])
def test_dropout_residual_backward_finite_differences(orc, m):
    rng = np.random.default_rng(300 + m)
    rows, p, eps = 3, 0.3, 1e-5
    x, res, dy, dzx = (_rows(rng, rows, m) for _ in range(4))
    bias = rng.normal(0.0, 0.5, m)
    gamma = rng.uniform(0.5, 1.5, m)
    beta = rng.normal(0.0, 0.1, m)
    keep = (rng.uniform(size=(rows, m)) >= p).astype(np.uint8)
    keep[0, 0], keep[-1, -1] = 0, 1            # both cases present
    z = orc.bias_dropout_residual(x, bias, res, keep, p)
    _, mean, rstd = orc.ln_fwd(z, gamma, beta, eps)
    dz = orc.ln_bwd_dx(dy, z, gamma, mean, rstd) + dzx
    dx, dbias, sbias = orc.dropout_residual_bwd(dz, keep, p)

    def loss(xx=x, rr=res, bb=bias):
        return _fused_loss(orc, xx, bb, rr, keep, p, gamma, beta, dy, dzx, eps)

    scale = max(1.0, np.max(np.abs(dx)), np.max(np.abs(dz)))
    for r in range(rows):
        for j in range(m):
            for name, arr, grad in (("x", x, dx), ("residual", res, dz)):
                h = 1e-6 * max(1.0, abs(arr[r, j]))
                ap, am = arr.copy(), arr.copy()
                ap[r, j] += h
                am[r, j] -= h
                kw_p = {"xx": ap} if name == "x" else {"rr": ap}
                kw_m = {"xx": am} if name == "x" else {"rr": am}
                fd = (loss(**kw_p) - loss(**kw_m)) / (2 * h)
                assert abs(fd - grad[r, j]) <= 1e-7 * scale, (name, r, j, fd, grad[r, j])
    for j in range(m):
        h = 1e-6 * max(1.0, abs(bias[j]))
        bp, bm = bias.copy(), bias.copy()
        bp[j] += h
        bm[j] -= h
        fd = (loss(bb=bp) - loss(bb=bm)) / (2 * h)
        assert abs(fd - dbias[j]) <= 1e-7 * max(1.0, np.max(np.abs(dbias))), (j, fd, dbias[j])
    # dropped positions get exactly no gradient; the absolute sums bound the sums
    assert np.all(dx[keep == 0] == 0.0)
    assert np.all(sbias >= np.abs(dbias))


@pytest.mark.parametrize("m", [64, 768, 1280])
def test_backward_two_forms_agree(orc, m):
    # The x-hat ("HW4") form and the slides' alpha/beta form: algebraically
    # equal, numerically within float64 rounding on N(0,1) rows.
    rng = np.random.default_rng(m)
    x = _rows(rng, 32, m)
    gamma = rng.uniform(0.5, 1.5, m)
    dy = _rows(rng, 32, m)
    _, mean, rstd = orc.ln_fwd(x, gamma, np.zeros(m), 1e-5)
    a = orc.ln_bwd_dx(dy, x, gamma, mean, rstd, form="hw4")
    b = orc.ln_bwd_dx(dy, x, gamma, mean, rstd, form="slides")
    assert np.max(np.abs(a - b)) / np.max(np.abs(a)) <= 1e-14


def test_backward_slides_form_cancellation_on_offset_rows(orc):
    # "(II)" §2.3: on rows ~ N(mean, 1) the slides form loses accuracy that
    # the x-hat form keeps (its two large terms cancel).  Values sit on a
    # 2^-20 grid so that shifting them by 2^20 is exact: the x-hat form then
    # sees exactly the same centred values, the slides form does not.
    rng = np.random.default_rng(5)
    m = 256
    grid = 2.0 ** 20
    x0 = np.round(_rows(rng, 64, m) * grid) / grid
    gamma = rng.uniform(0.5, 1.5, m)
    dy = _rows(rng, 64, m)
    _, mean0, rstd0 = orc.ln_fwd(x0, gamma, np.zeros(m), 1e-5)
    mean0 = np.round(mean0 * grid) / grid
    ref = orc.ln_bwd_dx(dy, x0, gamma, mean0, rstd0, form="hw4")
    shift = 2.0 ** 20
    x, mean = x0 + shift, mean0 + shift
    assert np.array_equal(x - shift, x0) and np.array_equal(mean - shift, mean0)
    e_hw4 = np.max(np.abs(orc.ln_bwd_dx(dy, x, gamma, mean, rstd0, "hw4") - ref))
    e_sl = np.max(np.abs(orc.ln_bwd_dx(dy, x, gamma, mean, rstd0, "slides") - ref))
    assert e_hw4 == 0.0
    assert e_sl > 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("m", [2, 17, 768])
def test_backward_identities(orc, m):
    # sum_j dx_j = 0 (exercise 2); sum_j dx_j xhat_j = r eps/(var+eps) sum g xhat
    rng = np.random.default_rng(2 * m)
    x = _rows(rng, 8, m, mean=0.5, std=0.3)
    gamma = rng.uniform(0.5, 1.5, m)
    dy = _rows(rng, 8, m)
    eps = 1e-2                         # large eps makes the second identity visible
    _, mean, rstd = orc.ln_fwd(x, gamma, np.zeros(m), eps)
    dx = orc.ln_bwd_dx(dy, x, gamma, mean, rstd)
    assert np.all(np.abs(dx.sum(axis=1)) <= 1e-13 * np.abs(dx).sum(axis=1))
    xhat = (x - mean[:, None]) * rstd[:, None]
    g = gamma * dy
    var = np.var(x, axis=1)
    lhs = (dx * xhat).sum(axis=1)
    eps64 = float(np.float32(eps))
    rhs = rstd * eps64 / (var + eps64) * (g * xhat).sum(axis=1)
    assert np.allclose(lhs, rhs, rtol=1e-9, atol=1e-12)


def test_backward_constant_row(orc):
    m = 16
    x = np.full((1, m), -2.0)
    gamma = np.linspace(0.5, 1.5, m)
    dy = np.linspace(-1, 1, m)[None, :] ** 3 + 0.3
    _, mean, rstd = orc.ln_fwd(x, gamma, np.zeros(m), 1e-5)
    dx = orc.ln_bwd_dx(dy, x, gamma, mean, rstd)
    g = gamma * dy[0]
    assert np.allclose(dx[0], rstd[0] * (g - g.mean()), rtol=1e-14, atol=1e-14)


def test_params_abs_sums_bound_sums(orc):
    rng = np.random.default_rng(9)
    x, dy = _rows(rng, 50, 20), _rows(rng, 50, 20)
    _, mean, rstd = orc.ln_fwd(x, np.ones(20), np.zeros(20), 1e-5)
    dg, db, sg, sb = orc.ln_bwd_params(dy, x, mean, rstd)
    assert np.all(np.abs(dg) <= sg) and np.all(np.abs(db) <= sb)
    assert np.allclose(sb, np.abs(dy).sum(axis=0), rtol=1e-14)


# --------------------------------------------------------------------------
# Dropout mask (Philox4x32-10) and the fused prologue ("(I)" §2.3)
# --------------------------------------------------------------------------

def test_dropout_threshold(orc):
    assert orc.dropout_threshold(0.0) == 0
    assert orc.dropout_threshold(0.1) == 6554
    assert orc.dropout_threshold(0.5) == 32768
    assert orc.dropout_threshold(np.nextafter(np.float32(1), np.float32(0))) == 65536


def test_dropout_mask_layout(orc):
    # mask is a pure function of (seed, row, col): prefixes agree, and an
    # element equals its 16-bit half of the Philox output for its counter
    seed, p = 0x0123456789ABCDEF, 0.25
    big = orc.dropout_keep(seed, p, 20, 40)
    assert np.array_equal(orc.dropout_keep(seed, p, 7, 13), big[:7, :13])
    thr = orc.dropout_threshold(p)
    for r, c in ((0, 0), (3, 9), (19, 39), (11, 16)):
        w = orc.philox4x32_10([c >> 3, r, 0, 0], [seed & 0xFFFFFFFF, seed >> 32])
        k = c & 7
        u = (int(w[k >> 1]) >> (16 * (k & 1))) & 0xFFFF
        assert big[r, c] == (1 if u >= thr else 0)


@pytest.mark.parametrize("seed", [0, 1, 2 ** 63 + 5])
def test_dropout_keep_rate(orc, seed):
    rows, cols, p = 512, 1280, 0.1
    keep = orc.dropout_keep(seed, p, rows, cols)
    n = keep.size
    q = 1.0 - orc.dropout_threshold(p) / 65536.0
    sd = math.sqrt(n * q * (1 - q))
    assert abs(int(keep.sum()) - n * q) <= 6 * sd
    # per-column and per-row rates show no structure beyond binomial noise
    col_rate = keep.mean(axis=0)
    assert np.max(np.abs(col_rate - q)) <= 6 * math.sqrt(q * (1 - q) / rows)


def test_dropout_two_seeds_independent(orc):
    rows, cols, p = 256, 1024, 0.3
    a = orc.dropout_keep(1, p, rows, cols)
    b = orc.dropout_keep(2, p, rows, cols)
    agree = np.mean(a == b)
    expect = p * p + (1 - p) * (1 - p)
    assert abs(agree - expect) < 6 * math.sqrt(expect * (1 - expect) / a.size)
    assert np.all(orc.dropout_keep(5, 0.0, 8, 64) == 1)


def test_fused_prologue_definition(orc):
    rng = np.random.default_rng(4)
    rows, m, p = 6, 24, 0.4
    x, res = _rows(rng, rows, m), _rows(rng, rows, m)
    bias = rng.normal(0, 0.02, m)
    keep = orc.dropout_keep(77, p, rows, m)
    z = orc.bias_dropout_residual(x, bias, res, keep, p)
    q = 1.0 - float(np.float32(p))
    for r in range(rows):
        for j in range(m):
            want = res[r, j] + ((x[r, j] + bias[j]) / q if keep[r, j] else 0.0)
            assert z[r, j] == want
    # p = 0 keeps everything: z = residual + x + bias
    z0 = orc.bias_dropout_residual(x, bias, res, np.ones_like(keep), 0.0)
    assert np.array_equal(z0, res + (x + bias))


@pytest.mark.parametrize("p", [0.1, 0.3, 0.5, 0.9])
def test_fused_prologue_keeps_the_expectation(orc, p):
    """Dropout followed by the residual add ("(I)" §2.3) must leave the
    expected value of z unchanged: averaged over dropout seeds, z - residual
    equals x + bias.  The oracle's prologue, driven by its own keep masks, is
    fitted with one scale s in z - residual = s * (x + bias) over 2^20
    (element, seed) pairs; s must be 1 within the binomial band plus the
    quantisation of p to a 16-bit threshold (|thr/65536 - p| <= 2^-17).  A
    scale of (1 - p), or none, moves s by at least 0.1 at every p here (the
    band is below 3e-3).  Dropped positions hold exactly the residual: the
    bias is dropped with x, and the residual is never dropped."""
    rng = np.random.default_rng(31)
    rows, m, seeds = 64, 256, 64
    x, res = _rows(rng, rows, m), _rows(rng, rows, m)
    bias = rng.normal(0, 0.5, m)
    t = x + bias
    num = den = 0.0
    for s in range(seeds):
        keep = orc.dropout_keep(1000 + s, p, rows, m)
        z = orc.bias_dropout_residual(x, bias, res, keep, p)
        assert np.array_equal(z[keep == 0], res[keep == 0])
        d = z - res
        num += float(np.sum(d * t))
        den += float(np.sum(t * t))
    s_fit = num / den
    n = rows * m * seeds
    q = 1.0 - orc.dropout_threshold(p) / 65536.0
    pf = float(np.float32(p))
    # Var of sum(keep t^2)/sum(t^2) for Bernoulli(q) keeps: q(1-q) sum t^4 / (sum t^2)^2
    t4 = float(np.sum(t ** 4)) * seeds
    sd = math.sqrt(q * (1 - q) * t4) / den / (1 - pf)
    assert abs(s_fit - 1.0) <= 6 * sd + 2.0 ** -17 / (1 - pf) + 1e-12, (s_fit, sd)
    # the band excludes the other readings: kept values scaled by (1 - p), or
    # not scaled at all, would give s = q (1 - p) or s = q
    for wrong in (q * (1 - pf), q):
        assert abs(wrong - 1.0) > 6 * sd + 2.0 ** -17 / (1 - pf) + 0.05


def test_dx_term_scale_bounds_dx(orc):
    # |dx_j| = r |g_j - (A + xhat_j B)/m| <= r (|g_j| + (sum|g| + |xhat_j| sum|g xhat|)/m)
    rng = np.random.default_rng(12)
    x, dy = _rows(rng, 20, 50, mean=2.0), _rows(rng, 20, 50)
    gamma = rng.uniform(0.5, 1.5, 50)
    _, mean, rstd = orc.ln_fwd(x, gamma, np.zeros(50), 1e-5)
    dx = orc.ln_bwd_dx(dy, x, gamma, mean, rstd)
    scale = orc.ln_bwd_dx_scale(dy, x, gamma, mean, rstd)
    assert np.all(np.abs(dx) <= scale * (1 + 1e-12))
    assert np.all(scale <= 10 * rstd[:, None] * (np.abs(gamma * dy) + 10))


# --------------------------------------------------------------------------
# Attention softmax: "Accelerating Transformer on GPU (I)" §4.1 (forward:
# scale, mask, max, exp, sum, divide) and "(II)" §3 (backward, fused with
# the dropout backward)
# --------------------------------------------------------------------------

def test_softmax_backward_worked_example(orc):
    g = _golden_kv("softmax_backward_example.txt")
    y, dy = np.array([g["y"]]), np.array([g["dy"]])
    dx = orc.attn_softmax_bwd(dy, y)
    assert np.allclose(dx[0], g["dx"], rtol=0, atol=1e-15)
    assert abs(float(np.sum(dy * y)) - g["s"][0]) < 1e-15
    assert abs(float(np.sum(dx))) < 1e-15          # the page's check: the sum is 0


def test_softmax_forward_matches_library(orc):
    from scipy.special import softmax
    rng = np.random.default_rng(21)
    for m in (1, 2, 7, 64, 1000):
        x = _rows(rng, 5, m, std=3.0)
        for scale in (1.0, 0.125):
            y = orc.attn_softmax_fwd(x, scale=scale)
            ref = softmax(scale * x, axis=1)
            assert np.allclose(y, ref, rtol=1e-13, atol=1e-300), (m, scale)
            assert np.allclose(np.sum(y, axis=1), 1.0, rtol=0, atol=1e-13)


def test_softmax_forward_shift_invariance_and_large_scores(orc):
    rng = np.random.default_rng(22)
    x = _rows(rng, 4, 33)
    y = orc.attn_softmax_fwd(x)
    # softmax ignores a constant added to the row; huge scores do not overflow
    # because the row maximum is subtracted first
    assert np.allclose(orc.attn_softmax_fwd(x + 1000.0), y, rtol=1e-12, atol=1e-15)
    big = orc.attn_softmax_fwd(np.array([[1000.0, 999.0, -1000.0]]))
    e = np.exp(-1.0)
    assert np.allclose(big[0], [1 / (1 + e), e / (1 + e), 0.0], rtol=1e-14, atol=1e-300)


def test_softmax_forward_masks(orc):
    from scipy.special import softmax
    rng = np.random.default_rng(23)
    m = 16
    x = _rows(rng, 2 * m, m)                       # two square blocks
    y = orc.attn_softmax_fwd(x, causal=True)
    for r in range(2 * m):
        q = r % m
        assert np.all(y[r, q + 1:] == 0.0)
        assert np.allclose(y[r, :q + 1], softmax(x[r, :q + 1]), rtol=1e-13, atol=1e-300)
    # an additive mask row per 8 rows; -inf removes a key, a finite value shifts it
    mask = np.zeros((4, m))
    mask[1, 3] = -np.inf
    mask[2, :] = 5.0
    y = orc.attn_softmax_fwd(x, mask=mask, rows_per_mask=8)
    assert np.all(y[8:16, 3] == 0.0)
    assert np.allclose(y[16:24], softmax(x[16:24], axis=1), rtol=1e-13)
    # a row with every key masked gives zeros
    mask[3, :] = -np.inf
    y = orc.attn_softmax_fwd(x, mask=mask, rows_per_mask=8)
    assert np.all(y[24:32] == 0.0)


def _softmax_loss(orc, x, dy, keep, p, scale):
    y = orc.attn_softmax_fwd(x, scale=scale)
    yd = np.where(keep == 1, y / (1.0 - np.float64(np.float32(p))), 0.0)
    return float(np.sum(dy * yd))


@pytest.mark.parametrize("m", [1, 2, 5, 8])
def test_softmax_backward_finite_differences(orc, m):
    rng = np.random.default_rng(400 + m)
    rows, p, scale = 3, 0.25, 0.7
    x, dy = _rows(rng, rows, m), _rows(rng, rows, m)
    keep = (rng.uniform(size=(rows, m)) >= p).astype(np.uint8)
    y = orc.attn_softmax_fwd(x, scale=scale)
    dx = orc.attn_softmax_bwd(dy, y, keep=keep, p=p, scale=scale)
    for r in range(rows):
        for j in range(m):
            h = 1e-6 * max(1.0, abs(x[r, j]))
            xp, xm = x.copy(), x.copy()
            xp[r, j] += h
            xm[r, j] -= h
            fd = (_softmax_loss(orc, xp, dy, keep, p, scale)
                  - _softmax_loss(orc, xm, dy, keep, p, scale)) / (2 * h)
            assert abs(fd - dx[r, j]) <= 1e-8 * max(1.0, np.max(np.abs(dx))), (r, j)
    # each row of dx sums to 0 (softmax ignores a constant added to its input)
    assert np.allclose(np.sum(dx, axis=1), 0.0, atol=1e-14)


# --------------------------------------------------------------------------
# RMSNorm: "GPU Performance from First Principles" §6 (fused add + RMSNorm:
# one sum of squares, no mean)
# --------------------------------------------------------------------------

def test_rmsnorm_is_layernorm_of_the_centred_row(orc):
    # LayerNorm(x) with beta = 0 is RMSNorm(x - mean(x)): pins the RMSNorm
    # oracle against the (separately pinned) LayerNorm oracle
    rng = np.random.default_rng(31)
    for m in (1, 3, 64, 1000):
        x = _rows(rng, 6, m, mean=2.0, std=1.5)
        gamma = rng.uniform(0.5, 1.5, m)
        y_ln, mean, rstd_ln = orc.ln_fwd(x, gamma, np.zeros(m), 1e-5)
        y_rms, rstd_rms = orc.rmsnorm_fwd(x - mean[:, None], gamma, 1e-5)
        assert np.allclose(y_rms, y_ln, rtol=1e-12, atol=1e-12), m
        assert np.allclose(rstd_rms, rstd_ln, rtol=1e-12), m


def test_rmsnorm_closed_form(orc):
    rng = np.random.default_rng(32)
    x = _rows(rng, 5, 300, std=4.0)
    eps = 1e-5
    y, rstd = orc.rmsnorm_fwd(x, np.ones(300), eps)
    ms = np.mean(x * x, axis=1)
    e32 = float(np.float32(eps))
    assert np.allclose(np.mean(y * y, axis=1), ms / (ms + e32), rtol=1e-13)
    assert np.allclose(rstd, 1.0 / np.sqrt(ms + e32), rtol=1e-14)


def _rms_loss(orc, x, gamma, dy, eps):
    y, _ = orc.rmsnorm_fwd(x, gamma, eps)
    return float(np.sum(dy * y))


@pytest.mark.parametrize("m", [1, 2, 3, 5, 8])
def test_rmsnorm_backward_finite_differences(orc, m):
    rng = np.random.default_rng(500 + m)
    rows, eps = 3, 1e-5
    x, dy = _rows(rng, rows, m, std=1.5), _rows(rng, rows, m)
    gamma = rng.uniform(0.5, 1.5, m)
    _, rstd = orc.rmsnorm_fwd(x, gamma, eps)
    dx, dg, sg = orc.rmsnorm_bwd(dy, x, gamma, rstd)
    scale = max(1.0, np.max(np.abs(dx)))
    for r in range(rows):
        for j in range(m):
            h = 1e-6 * max(1.0, abs(x[r, j]))
            xp, xm = x.copy(), x.copy()
            xp[r, j] += h
            xm[r, j] -= h
            fd = (_rms_loss(orc, xp, gamma, dy, eps) - _rms_loss(orc, xm, gamma, dy, eps)) / (2 * h)
            assert abs(fd - dx[r, j]) <= 1e-7 * scale, (r, j, fd, dx[r, j])
    for j in range(m):                       # the loss is linear in gamma
        gp, gm = gamma.copy(), gamma.copy()
        gp[j] += 0.5
        gm[j] -= 0.5
        fd = _rms_loss(orc, x, gp, dy, eps) - _rms_loss(orc, x, gm, dy, eps)
        assert abs(fd - dg[j]) <= 1e-12 * max(1.0, abs(dg[j])), j
    assert np.all(sg >= np.abs(dg))



# --- cross-entropy with label smoothing ([L10] §5.2; [LLMC] §6.1) ----------

def test_cross_entropy_matches_torch_label_smoothing(orc):
    # the lecture notes state that their target p = (1 - a) y + a / V is the
    # convention of torch's label_smoothing, and check the gradient q - p
    # against autograd; both are library special cases here (float64, CPU)
    import torch
    rng = np.random.default_rng(41)
    for V, alpha in ((2, 0.0), (7, 0.1), (300, 0.25), (1000, 0.0)):
        x = rng.normal(0.0, 3.0, (9, V))
        lab = rng.integers(0, V, 9)
        lab[4] = -100                              # torch's ignore_index
        scale = 0.375
        loss, dx = orc.cross_entropy(x, lab, alpha, scale)
        xt = torch.tensor(x, requires_grad=True)
        lt = torch.nn.functional.cross_entropy(xt, torch.tensor(lab), reduction="none",
                                               label_smoothing=float(np.float32(alpha)),
                                               ignore_index=-100)
        (lt * scale).sum().backward()
        np.testing.assert_allclose(loss, lt.detach().numpy(), rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-15)
        assert loss[4] == 0.0 and np.all(dx[4] == 0.0)


def test_cross_entropy_closed_form(orc):
    # loss = log Z + m - [(1 - a) x_label + (a / V) sum x]  ([L10] §5.2)
    rng = np.random.default_rng(42)
    V, alpha = 513, 0.1
    x = rng.normal(0.0, 2.0, (6, V))
    lab = rng.integers(0, V, 6)
    loss, _ = orc.cross_entropy(x, lab, alpha, 1.0, grad=False)
    a = float(np.float32(alpha))
    for r in range(6):
        m = x[r].max()
        logz = np.log(np.sum(np.exp(x[r] - m)))
        ref = logz + m - ((1 - a) * x[r, lab[r]] + a / V * x[r].sum())
        assert abs(loss[r] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_cross_entropy_special_rows(orc):
    # uniform logits: q = 1/V, so loss = log V for any smoothing; the gradient
    # sums to 0 over a row (sum q = sum p = 1) and is negative at the label
    rng = np.random.default_rng(43)
    for V in (1, 2, 50, 4096):
        loss, dx = orc.cross_entropy(np.full((2, V), 3.5), [0, V - 1], 0.2, 1.0)
        np.testing.assert_allclose(loss, np.log(V), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(dx.sum(axis=1), 0.0, atol=1e-14)
    x = rng.normal(0.0, 1.0, (5, 333))
    lab = np.array([0, 17, 332, 100, 5])
    _, dx = orc.cross_entropy(x, lab, 0.05, 2.0)
    np.testing.assert_allclose(dx.sum(axis=1), 0.0, atol=1e-13)
    assert np.all(dx[np.arange(5), lab] < 0)
    # one-hot target: loss = -log q_label
    loss, _ = orc.cross_entropy(x, lab, 0.0, 1.0, grad=False)
    q = np.exp(x - x.max(axis=1, keepdims=True))
    q /= q.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(loss, -np.log(q[np.arange(5), lab]), rtol=1e-13)
    # a label outside the vocabulary has no target: NaN
    loss, dx = orc.cross_entropy(x[:1], [333], 0.0, 1.0)
    assert np.isnan(loss[0]) and np.all(np.isnan(dx))


def test_cross_entropy_finite_differences(orc):
    rng = np.random.default_rng(44)
    V, alpha, h = 11, 0.3, 1e-6
    x = rng.normal(0.0, 2.0, (1, V))
    lab = [4]
    _, dx = orc.cross_entropy(x, lab, alpha, 1.0)
    for j in range(V):
        xp, xm = x.copy(), x.copy()
        xp[0, j] += h
        xm[0, j] -= h
        fd = (orc.cross_entropy(xp, lab, alpha, 1.0, grad=False)[0][0]
              - orc.cross_entropy(xm, lab, alpha, 1.0, grad=False)[0][0]) / (2 * h)
        assert abs(fd - dx[0, j]) < 1e-8, (j, fd, dx[0, j])


def test_dropout_keep_rows_is_the_same_mask(orc):
    # the row-range form of the mask equals the corresponding rows of the
    # whole-tensor form (including rows past 2^32, where the row's high word
    # enters the counter)
    full = orc.dropout_keep(123, 0.3, 40, 77)
    assert np.array_equal(orc.dropout_keep_rows(123, 0.3, 7, 20, 77), full[7:27])
    hi = orc.dropout_keep_rows(5, 0.5, (1 << 32) + 3, 2, 64)
    lo = orc.dropout_keep_rows(5, 0.5, 3, 2, 64)
    assert not np.array_equal(hi, lo)
