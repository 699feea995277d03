"""ctypes marshalling for the float64 C oracle (test infrastructure only).

Every function takes and returns numpy arrays.  Inputs are converted to
float64 exactly (every fp32/fp16/bf16 value is a double); no arithmetic of the
method happens here, it all happens in ``ln_oracle.c`` (see its header for the
passage each function follows).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ln_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_ln.so")

F32, F16, BF16 = 0, 1, 2
_FMT_NAMES = {"f32": F32, "float32": F32, "f16": F16, "float16": F16,
              "bf16": BF16, "bfloat16": BF16}

_lib = None


def build(force: bool = True) -> str:
    """Compile ln_oracle.c into liboracle_ln.so with gcc; returns the path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
               "-fPIC", "-shared", _SRC, "-lm", "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    i64 = ctypes.c_int64
    lib.orc_round.restype = ctypes.c_double
    lib.orc_round.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.orc_round_array.argtypes = [dp, dp, i64, ctypes.c_int]
    lib.orc_ln_fwd.argtypes = [dp, dp, dp, i64, i64, ctypes.c_double, dp, dp, dp]
    lib.orc_row_stats_welford.argtypes = [dp, i64, i64, dp, dp]
    lib.orc_var_naive_f32.argtypes = [dp, i64, i64, dp]
    lib.orc_var_chan_f32.argtypes = [dp, i64, i64, ctypes.c_int, dp]
    lib.orc_philox4x32_10.argtypes = [u32p, u32p, u32p]
    lib.orc_dropout_threshold.restype = ctypes.c_uint32
    lib.orc_dropout_threshold.argtypes = [ctypes.c_float]
    lib.orc_dropout_keep.argtypes = [ctypes.c_uint64, ctypes.c_float, i64, i64, u8p]
    lib.orc_dropout_keep_rows.argtypes = [ctypes.c_uint64, ctypes.c_float, i64, i64, i64, u8p]
    lib.orc_bias_dropout_residual.argtypes = [dp, dp, dp, u8p, ctypes.c_float,
                                              i64, i64, dp]
    for name in ("orc_ln_bwd_dx_hw4", "orc_ln_bwd_dx_slides", "orc_ln_bwd_dx_scale"):
        getattr(lib, name).argtypes = [dp, dp, dp, dp, dp, i64, i64, dp]
    lib.orc_ln_bwd_params.argtypes = [dp, dp, dp, dp, i64, i64, dp, dp, dp, dp]
    lib.orc_dropout_residual_bwd.argtypes = [dp, u8p, ctypes.c_float, i64, i64, dp, dp, dp]
    lib.orc_rmsnorm_fwd.argtypes = [dp, dp, i64, i64, ctypes.c_double, dp, dp]
    lib.orc_rmsnorm_bwd.argtypes = [dp, dp, dp, dp, i64, i64, dp, dp, dp]
    lib.orc_cross_entropy.argtypes = [dp, ctypes.POINTER(ctypes.c_int64), i64, i64,
                                      ctypes.c_double, ctypes.c_double, dp, dp]
    lib.orc_attn_softmax_fwd.argtypes = [dp, dp, i64, i64, i64, ctypes.c_double, ctypes.c_int,
                                         dp]
    lib.orc_attn_softmax_bwd.argtypes = [dp, dp, u8p, ctypes.c_float, i64, i64, ctypes.c_double,
                                         dp]
    _lib = lib
    return lib


def _d(a) -> np.ndarray:
    """Exact float64 copy of an array (C-contiguous)."""
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray, ctype=ctypes.c_double):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _fmt(fmt) -> int:
    if isinstance(fmt, int):
        return fmt
    return _FMT_NAMES[str(fmt).replace("torch.", "")]


def _shape2(x: np.ndarray):
    if x.ndim != 2:
        raise ValueError("expected a [rows, cols] array")
    return x.shape[0], x.shape[1]


def round_to(a, fmt) -> np.ndarray:
    """Round each value to the storage format (RNE); result as float64."""
    a = _d(a)
    out = np.empty_like(a)
    _load().orc_round_array(_ptr(a), _ptr(out), a.size, _fmt(fmt))
    return out


def round_scalar(v: float, fmt) -> float:
    return float(_load().orc_round(float(v), _fmt(fmt)))


def ln_fwd(x, gamma, beta, eps: float):
    """Two-pass LayerNorm forward in float64 -> (y, mean, rstd)."""
    x = _d(x)
    rows, m = _shape2(x)
    g, b = _d(gamma), _d(beta)
    y = np.empty_like(x)
    mean = np.empty(rows)
    rstd = np.empty(rows)
    _load().orc_ln_fwd(_ptr(x), _ptr(g), _ptr(b), rows, m,
                       float(np.float32(eps)), _ptr(y), _ptr(mean), _ptr(rstd))
    return y, mean, rstd


def row_stats_welford(x):
    x = _d(x)
    rows, m = _shape2(x)
    mean = np.empty(rows)
    var = np.empty(rows)
    _load().orc_row_stats_welford(_ptr(x), rows, m, _ptr(mean), _ptr(var))
    return mean, var


def var_naive_f32(x):
    x = _d(x)
    rows, m = _shape2(x)
    var = np.empty(rows)
    _load().orc_var_naive_f32(_ptr(x), rows, m, _ptr(var))
    return var


def var_chan_f32(x, lanes: int = 64):
    x = _d(x)
    rows, m = _shape2(x)
    var = np.empty(rows)
    _load().orc_var_chan_f32(_ptr(x), rows, m, int(lanes), _ptr(var))
    return var


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.empty(4, dtype=np.uint32)
    _load().orc_philox4x32_10(_ptr(c, ctypes.c_uint32), _ptr(k, ctypes.c_uint32),
                              _ptr(out, ctypes.c_uint32))
    return out


def dropout_threshold(p: float) -> int:
    return int(_load().orc_dropout_threshold(ctypes.c_float(p)))


def dropout_keep(seed: int, p: float, rows: int, cols: int) -> np.ndarray:
    keep = np.empty((rows, cols), dtype=np.uint8)
    _load().orc_dropout_keep(ctypes.c_uint64(seed), ctypes.c_float(p), rows, cols,
                             _ptr(keep, ctypes.c_uint8))
    return keep


def dropout_keep_rows(seed: int, p: float, row0: int, rows: int, cols: int) -> np.ndarray:
    """The keep mask of rows [row0, row0 + rows) of a tensor."""
    keep = np.empty((rows, cols), dtype=np.uint8)
    _load().orc_dropout_keep_rows(ctypes.c_uint64(seed), ctypes.c_float(p), row0, rows, cols,
                                  _ptr(keep, ctypes.c_uint8))
    return keep


def bias_dropout_residual(x, bias, residual, keep, p: float) -> np.ndarray:
    """Exact (unrounded) z = residual + dropout(x + bias) in float64."""
    x = _d(x)
    rows, m = _shape2(x)
    b, r = _d(bias), _d(residual)
    k = np.ascontiguousarray(np.asarray(keep, dtype=np.uint8))
    z = np.empty_like(x)
    _load().orc_bias_dropout_residual(_ptr(x), _ptr(b), _ptr(r),
                                      _ptr(k, ctypes.c_uint8), ctypes.c_float(p),
                                      rows, m, _ptr(z))
    return z


def ln_bwd_dx(dy, x, gamma, mean, rstd, form: str = "hw4") -> np.ndarray:
    """dx of LayerNorm, 'hw4' (x-hat sums) or 'slides' (alpha/beta) form."""
    dy, x = _d(dy), _d(x)
    rows, m = _shape2(x)
    g, mu, rs = _d(gamma), _d(mean), _d(rstd)
    dx = np.empty_like(x)
    fn = {"hw4": _load().orc_ln_bwd_dx_hw4,
          "slides": _load().orc_ln_bwd_dx_slides}[form]
    fn(_ptr(dy), _ptr(x), _ptr(g), _ptr(mu), _ptr(rs), rows, m, _ptr(dx))
    return dx


def ln_bwd_dx_scale(dy, x, gamma, mean, rstd) -> np.ndarray:
    """Per-element magnitude of the terms of dx (for the float32 error bound)."""
    dy, x = _d(dy), _d(x)
    rows, m = _shape2(x)
    g, mu, rs = _d(gamma), _d(mean), _d(rstd)
    out = np.empty_like(x)
    _load().orc_ln_bwd_dx_scale(_ptr(dy), _ptr(x), _ptr(g), _ptr(mu), _ptr(rs), rows, m,
                                _ptr(out))
    return out


def ln_bwd_params(dy, x, mean, rstd):
    """-> (dgamma, dbeta, sum|dy*xhat|, sum|dy|) column sums in float64."""
    dy, x = _d(dy), _d(x)
    rows, m = _shape2(x)
    mu, rs = _d(mean), _d(rstd)
    dg, db, sg, sb = (np.empty(m) for _ in range(4))
    _load().orc_ln_bwd_params(_ptr(dy), _ptr(x), _ptr(mu), _ptr(rs), rows, m,
                              _ptr(dg), _ptr(db), _ptr(sg), _ptr(sb))
    return dg, db, sg, sb


def dropout_residual_bwd(dz, keep, p: float):
    """Backward of z = residual + keep*(x + bias)/(1 - p) given dz:
    (dx, dbias, sbias); dresidual is dz itself."""
    dz = _d(dz)
    rows, m = _shape2(dz)
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    if keep.shape != dz.shape:
        raise ValueError("keep must match dz")
    dx = np.empty_like(dz)
    db = np.empty(m)
    sb = np.empty(m)
    _load().orc_dropout_residual_bwd(_ptr(dz), _ptr(keep, ctypes.c_uint8), ctypes.c_float(p),
                                     rows, m, _ptr(dx), _ptr(db), _ptr(sb))
    return dx, db, sb



def attn_softmax_fwd(x, scale: float = 1.0, mask=None, rows_per_mask: int = 1,
                     causal: bool = False) -> np.ndarray:
    """Row softmax of scale*x + mask (mask row r // rows_per_mask), causal over
    square blocks (q = r mod cols); fully masked rows give 0."""
    x = _d(x)
    rows, m = _shape2(x)
    mk = None
    if mask is not None:
        mk = _d(mask)
        if mk.ndim != 2 or mk.shape[1] != m or mk.shape[0] * int(rows_per_mask) < rows:
            raise ValueError("mask must be [ceil(rows / rows_per_mask), cols]")
    y = np.empty_like(x)
    _load().orc_attn_softmax_fwd(_ptr(x), None if mk is None else _ptr(mk), int(rows_per_mask),
                                 rows, m, float(scale), 1 if causal else 0, _ptr(y))
    return y


def attn_softmax_bwd(dy, y, keep=None, p: float = 0.0, scale: float = 1.0) -> np.ndarray:
    """dx of the attention softmax, after the dropout backward (keep, p)."""
    dy, y = _d(dy), _d(y)
    rows, m = _shape2(y)
    kp = None
    if keep is not None:
        kp = np.ascontiguousarray(keep, dtype=np.uint8)
        if kp.shape != y.shape:
            raise ValueError("keep must match y")
    dx = np.empty_like(y)
    _load().orc_attn_softmax_bwd(_ptr(dy), _ptr(y), None if kp is None else _ptr(kp, ctypes.c_uint8),
                                 ctypes.c_float(p), rows, m, float(scale), _ptr(dx))
    return dx



def rmsnorm_fwd(x, gamma, eps: float):
    """RMSNorm: (y, rstd) with rstd = 1/sqrt(mean(x^2) + eps)."""
    x = _d(x)
    rows, m = _shape2(x)
    g = _d(gamma)
    y = np.empty_like(x)
    rs = np.empty(rows)
    _load().orc_rmsnorm_fwd(_ptr(x), _ptr(g), rows, m, float(np.float32(eps)), _ptr(y), _ptr(rs))
    return y, rs


def rmsnorm_bwd(dy, x, gamma, rstd):
    """(dx, dgamma, sgamma) of RMSNorm given the saved rstd."""
    dy, x, g, rs = _d(dy), _d(x), _d(gamma), _d(rstd)
    rows, m = _shape2(x)
    dx = np.empty_like(x)
    dg, sg = np.empty(m), np.empty(m)
    _load().orc_rmsnorm_bwd(_ptr(dy), _ptr(x), _ptr(g), _ptr(rs), rows, m, _ptr(dx), _ptr(dg),
                            _ptr(sg))
    return dx, dg, sg


def cross_entropy(x, labels, alpha: float = 0.0, scale: float = 1.0, grad: bool = True):
    """(loss [rows], dx [rows, V] or None) of label-smoothed cross-entropy.

    alpha and scale are taken as the float32 values the GPU library receives;
    a negative label is an ignored row (loss 0, dx 0)."""
    x = _d(x)
    rows, V = _shape2(x)
    lab = np.ascontiguousarray(np.asarray(labels, dtype=np.int64))
    if lab.shape != (rows,):
        raise ValueError("labels must be [rows]")
    loss = np.empty(rows)
    dx = np.empty_like(x) if grad else None
    _load().orc_cross_entropy(_ptr(x), lab.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                              rows, V, float(np.float32(alpha)), float(np.float32(scale)),
                              _ptr(loss), None if dx is None else _ptr(dx))
    return loss, dx


__all__ = ["F32", "F16", "BF16", "build", "round_to", "round_scalar", "ln_fwd",
           "row_stats_welford", "var_naive_f32", "var_chan_f32", "philox4x32_10",
           "dropout_threshold", "dropout_keep", "dropout_keep_rows", "bias_dropout_residual",
           "ln_bwd_dx", "ln_bwd_dx_scale", "ln_bwd_params", "dropout_residual_bwd",
           "attn_softmax_fwd", "attn_softmax_bwd", "rmsnorm_fwd", "rmsnorm_bwd",
           "cross_entropy"]
