"""Tolerance rule for judging GPU outputs against the float64 oracle.

Test infrastructure only.  The headline bound is max-abs 1e-5 for fp32
storage and 2e-2 for fp16/bf16 storage.  Two outputs cannot meet a bare
max-abs bound at every magnitude, and take a wider clause derived from the
arithmetic; every use of the wider clause is counted in the report:

* elementwise outputs stored in T (y, z, dx): the value must be stored in T,
  so half a storage step of T is unavoidable.  Pass iff
  |o - r| <= max(atol_T, 0.5 * ulp_T(r) * (1 + 2^-8)); the (1 + 2^-8) covers
  the fp32 error of the value before it is rounded.  Half a step exceeds atol
  only for bf16 |r| >= 8, fp16 |r| >= 32 and fp32 |r| >= 256.
* float32 arithmetic (any storage): an output formed from terms of size
  up to `scale` through at most k roundings, with k = 4 + ceil(log2 m) for a
  row of m values (products, a reduction tree of depth log2 m, the final
  update), may be off by k * 2^-24 * scale.  This only matters where the
  terms are much larger than the result or than atol (dx of a near-constant
  row, where rstd = 1/sqrt(eps) is about 316); elsewhere atol dominates.
* column sums (dgamma, dbeta, float32): pass iff |o - r| <= atol_T or
  |o - r| <= 0.5 * ulp_f32(r) + ceil(log2 rows) * 2^-24 * S_j, with
  S_j = sum_r |term_rj|: the rounding of a float32 result plus the error
  bound of a balanced summation tree over `rows` terms ("GPU Performance
  from First Principles", §7.4: a tree sum rounds each term log2(n) times).
* mean / rstd (float32): pass iff |o - r| <= 1e-5 * max(1, |r|).
* probability-sized outputs (softmax y, its dropped copy and dx; the
  cross-entropy gradient): these are far below 1 (about 1/L for a row of L
  keys), so an absolute floor of 2e-2 or 1e-5 would pass an all-zero output.
  They take no absolute floor: pass iff
  |o - r| <= 0.5 * ulp_T(r) * (1 + 2^-8) + k * 2^-24 * scale + 2^-126, the
  storage rounding, the float32 arithmetic clause above with the size of the
  terms behind each value, and float32's smallest normal (below it the
  arithmetic itself is denormal).  An exact 0 of the reference (a masked or
  dropped position) must be an exact 0.  `n_wide` counts the elements that
  needed more than the storage rounding.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F32, F16, BF16 = 0, 1, 2
ATOL = {F32: 1e-5, F16: 2e-2, BF16: 2e-2}
_BITS = {F32: (24, -126), F16: (11, -14), BF16: (8, -126)}


def ulp(r, fmt) -> np.ndarray:
    """Spacing of the storage format at each |r| (subnormal spacing below)."""
    p, emin = _BITS[fmt]
    a = np.abs(np.asarray(r, dtype=np.float64))
    _, k = np.frexp(a)
    e = np.maximum(k.astype(np.int64) - 1, emin)
    e = np.where(a == 0, emin, e)
    return np.ldexp(1.0, (e - (p - 1)).astype(np.int64))


@dataclass
class Report:
    name: str
    ok: bool
    max_abs: float
    worst_index: tuple
    n: int
    n_wide: int = 0          # elements that needed the wider clause
    n_fail: int = 0
    details: list = field(default_factory=list)

    def __str__(self):
        return (f"{self.name}: ok={self.ok} max_abs={self.max_abs:.3e} "
                f"n={self.n} wide={self.n_wide} fail={self.n_fail} "
                f"worst={self.worst_index}")


def _finish(name, out, ref, err, tol, atol):
    both_nan = np.isnan(out) & np.isnan(ref)
    err = np.where(both_nan, 0.0, err)
    bad = ~(err <= tol)
    n_wide = int(np.count_nonzero((err > atol) & ~bad))
    if err.size:
        idx = np.unravel_index(int(np.nanargmax(np.where(np.isnan(err), np.inf, err))),
                               err.shape)
        mx = float(err[idx])
    else:
        idx, mx = (), 0.0
    details = []
    if bad.any():
        for i in np.argwhere(bad)[:8]:
            t = tuple(int(v) for v in i)
            details.append((t, float(out[t]), float(ref[t]), float(tol[t])))
    return Report(name, not bad.any(), mx, tuple(int(v) for v in idx), int(err.size),
                  n_wide, int(np.count_nonzero(bad)), details)


def check_elementwise(name, out, ref, fmt, term_scale=None, row_len: int = 1) -> Report:
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    atol = ATOL[fmt]
    tol = np.maximum(atol, 0.5 * ulp(ref, fmt) * (1.0 + 2.0 ** -8))
    if term_scale is not None:
        k = 4 + math.ceil(math.log2(max(row_len, 2)))
        arith = 0.5 * ulp(ref, fmt) + k * 2.0 ** -24 * np.asarray(term_scale, np.float64)
        tol = np.maximum(tol, arith)
    err = np.abs(out - ref)
    return _finish(name, out, ref, err, tol, atol)


def check_scaled(name, out, ref, fmt, term_scale, row_len: int) -> Report:
    """Value-scaled rule of probability-sized outputs (no absolute floor)."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    k = 4 + math.ceil(math.log2(max(row_len, 2)))
    store = 0.5 * ulp(ref, fmt) * (1.0 + 2.0 ** -8)
    store = np.where(ref == 0, 0.0, store)
    arith = k * 2.0 ** -24 * np.asarray(term_scale, np.float64)
    tol = store + arith + np.where(ref == 0, 0.0, 2.0 ** -126)
    err = np.abs(out - ref)
    rep = _finish(name, out, ref, err, tol, 0.0)
    rep.n_wide = int(np.count_nonzero((err > store) & (err <= tol)))
    return rep


def check_colsum(name, out, ref, abs_sum, rows: int, fmt, term_err=None) -> Report:
    """Column sums: |o - r| <= atol, or <= half an fp32 step + the rounding of
    a depth-ceil(log2 rows) summation of |terms| (abs_sum).  `term_err`, when
    given, is the per-column sum of the error bounds of the summed terms
    themselves (terms that the GPU forms in float32 before summing them)."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    s = np.asarray(abs_sum, dtype=np.float64)
    atol = ATOL[fmt]
    depth = math.ceil(math.log2(max(rows, 2)))
    tol = np.maximum(atol, 0.5 * ulp(ref, F32) + depth * 2.0 ** -24 * s)
    if term_err is not None:
        tol = tol + np.asarray(term_err, dtype=np.float64)
    err = np.abs(out - ref)
    return _finish(name, out, ref, err, tol, atol)


def check_colsum_stat(name, out, ref, sq_sum, rows: int) -> Report:
    """Column sums against the random-rounding model of float32 summation
    (the rule of thumb that rounding errors of a long sum grow like the square
    root of the number of roundings, not linearly): each addition rounds its
    partial sum s_k with an error of at most 2^-24 |s_k|, so the error is
    about 2^-24/sqrt(3) * sqrt(sum_k s_k^2).  For terms of random sign summed
    in any order whose partial sums carry no more than D = 4 ceil(log2 rows)
    times the terms' own energy (sum_k s_k^2 <= D * sum_i t_i^2; a balanced
    tree has D = log2 rows, runs of a few dozen sequential adds per level stay
    well inside), the bound is six standard deviations:
    |o - r| <= 0.5 ulp_f32(r) + 6 * 2^-24/sqrt(3) * sqrt(D * sum_i t_i^2).
    It is far tighter than the worst-case tree clause of check_colsum, so a
    change that loses accuracy (a worse order, a term rounded twice, a lost
    row) fails it.  `sq_sum` is sum_r t_rj^2 per column."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    depth = 4 * math.ceil(math.log2(max(rows, 2)))
    sd = 2.0 ** -24 / math.sqrt(3.0) * np.sqrt(depth * np.asarray(sq_sum, np.float64))
    tol = 0.5 * ulp(ref, F32) + 6.0 * sd
    err = np.abs(out - ref)
    return _finish(name, out, ref, err, tol, 0.0)


def check_stats(name, out, ref) -> Report:
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    tol = 1e-5 * np.maximum(1.0, np.abs(ref))
    err = np.abs(out - ref)
    return _finish(name, out, ref, err, tol, 1e-5)
