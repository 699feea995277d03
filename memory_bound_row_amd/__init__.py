"""Fused LayerNorm forward/backward for AMD MI355X (gfx950).

A thin binding over the C ABI of ``libmbrow_ln.so`` (declared in
``include/mbrow_ln.h``): it checks tensor placement and layout, allocates
outputs with torch when the caller passes none, and hands raw device pointers
and the current HIP stream to the library.  Every step of the computation
runs in the library's HIP kernels; there is no fallback.  Calling any op
without the built library raises ``RuntimeError``.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmbrow_ln.so")

LN_F32, LN_F16, LN_BF16 = 0, 1, 2
_DTYPES = {torch.float32: LN_F32, torch.float16: LN_F16, torch.bfloat16: LN_BF16}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built: run `python -m memory_bound_row_amd.build` "
            "(the HIP library is required; there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    L.ln_status_string.restype = ctypes.c_char_p
    L.ln_status_string.argtypes = [i32]
    L.ln_fwd.restype = i32
    L.ln_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, vp]
    L.bias_dropout_residual_ln_fwd.restype = i32
    L.bias_dropout_residual_ln_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                               i64, i64, f32, f32, ctypes.c_uint64, i32, vp]
    L.ln_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.ln_bwd_workspace_bytes.argtypes = [i64, i64]
    L.ln_bwd_dx.restype = i32
    L.ln_bwd_dx.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i64, i64, i32, vp]
    L.ln_bwd_dgamma_dbeta.restype = i32
    L.ln_bwd_dgamma_dbeta.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i32,
                                      i64, i64, i32, vp]
    L.ln_bwd_noalloc.restype = i32
    L.ln_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, vp]
    L.bias_dropout_residual_ln_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.bias_dropout_residual_ln_bwd_workspace_bytes.argtypes = [i64, i64]
    L.bias_dropout_residual_ln_bwd.restype = i32
    L.bias_dropout_residual_ln_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                               ctypes.c_size_t, i64, i64, f32, ctypes.c_uint64,
                                               i32, vp]
    L.bias_dropout_residual_ln_bwd_dx.restype = i32
    L.bias_dropout_residual_ln_bwd_dx.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                  ctypes.c_size_t, i64, i64, f32,
                                                  ctypes.c_uint64, i32, vp]
    L.bias_dropout_residual_ln_bwd_fold.restype = i32
    L.bias_dropout_residual_ln_bwd_fold.argtypes = [vp, ctypes.c_size_t, vp, vp, vp, i64, i64,
                                                    vp]
    L.attn_softmax_fwd.restype = i32
    L.attn_softmax_fwd.argtypes = [vp, vp, i64, vp, vp, i64, i64, f32, i32, f32,
                                   ctypes.c_uint64, i32, vp]
    L.attn_softmax_bwd.restype = i32
    L.attn_softmax_bwd.argtypes = [vp, vp, vp, i64, i64, f32, i32, f32, ctypes.c_uint64, i32, vp]
    L.add_rmsnorm_fwd.restype = i32
    L.add_rmsnorm_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, vp]
    L.add_rmsnorm_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.add_rmsnorm_bwd_workspace_bytes.argtypes = [i64, i64]
    L.add_rmsnorm_bwd.restype = i32
    L.add_rmsnorm_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i64, i64,
                                  i32, vp]
    L.cross_entropy_fwd_bwd.restype = i32
    L.cross_entropy_fwd_bwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, f32, f32, i32, vp]
    L.hbm_copy.restype = i32
    L.hbm_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
    L.hbm_stream.restype = i32
    L.hbm_stream.argtypes = [ctypes.POINTER(vp), i32, ctypes.POINTER(vp), i32, ctypes.c_size_t,
                             vp]
    L.ln_debug_force_path.restype = i32
    L.ln_debug_force_path.argtypes = [i32, i32, i32]
    L.ln_debug_force_grid.restype = i32
    L.ln_debug_force_grid.argtypes = [i32]
    L.ln_debug_force_two_pass.restype = i32
    L.ln_debug_force_two_pass.argtypes = [i32]
    L.ln_debug_force_staged.restype = i32
    L.ln_debug_force_staged.argtypes = [i32]
    _lib = L
    return L


def status_string(code: int) -> str:
    return lib().ln_status_string(int(code)).decode()


def _check(code: int) -> None:
    if code != 0:
        raise RuntimeError(status_string(code))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32, float16 or bfloat16")
    return _DTYPES[t.dtype]


def _mat(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() < 1:
        raise ValueError(f"{name} must have a last (row) dimension")
    cols = t.shape[-1]
    rows = t.numel() // cols if cols else 0
    return rows, cols


def _vec(t: torch.Tensor, cols: int, dtype, name: str):
    if not t.is_cuda or not t.is_contiguous() or t.numel() != cols or t.dtype != dtype:
        raise ValueError(f"{name} must be a contiguous GPU tensor of {cols} {dtype} values")


def _out(t, shape, dtype, device, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if (not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != tuple(shape)
            or t.dtype != dtype):
        raise ValueError(f"{name} must be a contiguous GPU tensor {tuple(shape)} {dtype}")
    return t


def ln_fwd(x, gamma, beta, eps: float = 1e-5, *, y=None, mean=None, rstd=None,
           stats: bool = True):
    """LayerNorm over the last dimension -> (y, mean, rstd) (stats None if not kept)."""
    rows, cols = _mat(x, "x")
    _vec(gamma, cols, x.dtype, "gamma")
    _vec(beta, cols, x.dtype, "beta")
    y = _out(y, x.shape, x.dtype, x.device, "y")
    if stats:
        mean = _out(mean, (rows,), torch.float32, x.device, "mean")
        rstd = _out(rstd, (rows,), torch.float32, x.device, "rstd")
    if rows == 0:
        return y, mean, rstd
    _check(lib().ln_fwd(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), _ptr(mean), _ptr(rstd),
                        rows, cols, float(eps), _dt(x), _stream(x)))
    return y, mean, rstd


def bias_dropout_residual_ln_fwd(x, bias, residual, gamma, beta, p: float, seed: int,
                                 eps: float = 1e-5, *, residual_out=None, y=None, mean=None,
                                 rstd=None, mask_out=None, stats: bool = True,
                                 want_mask: bool = False):
    """z = residual + dropout(x + bias); y = LayerNorm(z) -> (z, y, mean, rstd, mask)."""
    rows, cols = _mat(x, "x")
    if residual.shape != x.shape or residual.dtype != x.dtype:
        raise ValueError("residual must match x")
    _mat(residual, "residual")
    for t, n in ((bias, "bias"), (gamma, "gamma"), (beta, "beta")):
        _vec(t, cols, x.dtype, n)
    residual_out = _out(residual_out, x.shape, x.dtype, x.device, "residual_out")
    y = _out(y, x.shape, x.dtype, x.device, "y")
    if stats:
        mean = _out(mean, (rows,), torch.float32, x.device, "mean")
        rstd = _out(rstd, (rows,), torch.float32, x.device, "rstd")
    if want_mask or mask_out is not None:
        mask_out = _out(mask_out, x.shape, torch.uint8, x.device, "mask_out")
    if rows == 0:
        return residual_out, y, mean, rstd, mask_out
    _check(lib().bias_dropout_residual_ln_fwd(
        _ptr(x), _ptr(bias), _ptr(residual), _ptr(gamma), _ptr(beta), _ptr(residual_out),
        _ptr(y), _ptr(mean), _ptr(rstd), _ptr(mask_out), rows, cols, float(eps), float(p),
        int(seed) & 0xFFFFFFFFFFFFFFFF, _dt(x), _stream(x)))
    return residual_out, y, mean, rstd, mask_out


def ln_bwd_workspace_bytes(rows: int, cols: int) -> int:
    return int(lib().ln_bwd_workspace_bytes(int(rows), int(cols)))


def workspace(rows: int, cols: int, device) -> torch.Tensor:
    """A float32 workspace of the size the backward needs."""
    n = ln_bwd_workspace_bytes(rows, cols) // 4
    return torch.empty(max(n, 1), dtype=torch.float32, device=device)


def ln_bwd_dx(dy, x, gamma, mean, rstd, *, dx=None, workspace=None):
    """dx of LayerNorm; with `workspace` also writes the dgamma/dbeta partials."""
    rows, cols = _mat(x, "x")
    if dy.shape != x.shape or dy.dtype != x.dtype:
        raise ValueError("dy must match x")
    _mat(dy, "dy")
    _vec(gamma, cols, x.dtype, "gamma")
    for t, n in ((mean, "mean"), (rstd, "rstd")):
        _vec(t, rows, torch.float32, n)
    dx = _out(dx, x.shape, x.dtype, x.device, "dx")
    ws_bytes = 0
    if workspace is not None:
        if workspace.dtype != torch.float32 or not workspace.is_cuda:
            raise ValueError("workspace must be a float32 GPU tensor")
        ws_bytes = workspace.numel() * 4
    if rows == 0:
        return dx
    _check(lib().ln_bwd_dx(_ptr(dy), _ptr(x), _ptr(gamma), _ptr(mean), _ptr(rstd), _ptr(dx),
                           _ptr(workspace), ws_bytes, rows, cols, _dt(x), _stream(x)))
    return dx


def ln_bwd_dgamma_dbeta(workspace, rows: int, cols: int, dtype, *, partials_ready: bool,
                        dy=None, x=None, mean=None, rstd=None, dgamma=None, dbeta=None):
    """dgamma, dbeta (float32): fold the partials, after stage 1 unless ready."""
    device = workspace.device
    dgamma = _out(dgamma, (cols,), torch.float32, device, "dgamma")
    dbeta = _out(dbeta, (cols,), torch.float32, device, "dbeta")
    if not partials_ready:
        r, c = _mat(x, "x")
        if (r, c) != (rows, cols) or dy.shape != x.shape:
            raise ValueError("dy/x must be [rows, cols]")
    if workspace.dtype != torch.float32:
        raise ValueError("workspace must be float32")
    if rows == 0:
        return dgamma.zero_(), dbeta.zero_()
    _check(lib().ln_bwd_dgamma_dbeta(
        _ptr(dy), _ptr(x), _ptr(mean), _ptr(rstd), _ptr(dgamma), _ptr(dbeta), _ptr(workspace),
        workspace.numel() * 4, 1 if partials_ready else 0, int(rows), int(cols),
        _DTYPES[dtype], _stream(workspace)))
    return dgamma, dbeta


def ln_bwd(dy, x, gamma, mean, rstd, *, dx=None, workspace_buf=None, dgamma=None, dbeta=None):
    """Whole LayerNorm backward: dx with fused partials, then the fold."""
    rows, cols = _mat(x, "x")
    ws = workspace_buf if workspace_buf is not None else workspace(rows, cols, x.device)
    dx = ln_bwd_dx(dy, x, gamma, mean, rstd, dx=dx, workspace=ws)
    dgamma, dbeta = ln_bwd_dgamma_dbeta(ws, rows, cols, x.dtype, partials_ready=True,
                                        dgamma=dgamma, dbeta=dbeta)
    return dx, dgamma, dbeta


NOALLOC_SCRATCH_BYTES = 16 << 20   # LN_NOALLOC_SCRATCH_BYTES


def ln_bwd_noalloc(dy, x, gamma, mean, rstd, *, dx, dgamma, dbeta):
    """Whole LayerNorm backward with the library's static scratch for the
    column partials: the C call allocates nothing, and neither does this
    wrapper (every output is the caller's)."""
    rows, cols = _mat(x, "x")
    if dy.shape != x.shape or dy.dtype != x.dtype:
        raise ValueError("dy must match x")
    _mat(dy, "dy")
    _vec(gamma, cols, x.dtype, "gamma")
    for t, n in ((mean, "mean"), (rstd, "rstd")):
        _vec(t, rows, torch.float32, n)
    dx = _out(dx, x.shape, x.dtype, x.device, "dx")
    dgamma = _out(dgamma, (cols,), torch.float32, x.device, "dgamma")
    dbeta = _out(dbeta, (cols,), torch.float32, x.device, "dbeta")
    _check(lib().ln_bwd_noalloc(_ptr(dy), _ptr(x), _ptr(gamma), _ptr(mean), _ptr(rstd),
                                _ptr(dx), _ptr(dgamma), _ptr(dbeta), rows, cols, _dt(x),
                                _stream(x)))
    return dx, dgamma, dbeta


def bias_dropout_residual_ln_bwd_workspace_bytes(rows: int, cols: int) -> int:
    return int(lib().bias_dropout_residual_ln_bwd_workspace_bytes(int(rows), int(cols)))


def dropout_workspace(rows: int, cols: int, device) -> torch.Tensor:
    """A float32 workspace of the size bias_dropout_residual_ln_bwd needs."""
    n = bias_dropout_residual_ln_bwd_workspace_bytes(rows, cols) // 4
    return torch.empty(max(n, 1), dtype=torch.float32, device=device)


def bias_dropout_residual_ln_bwd(dy, z, gamma, mean, rstd, p: float, seed: int, *,
                                 dz_extra=None, dresidual=None, dx=None, dgamma=None,
                                 dbeta=None, dbias=None, workspace=None):
    """Backward of bias_dropout_residual_ln_fwd -> (dresidual, dx, dgamma, dbeta, dbias).

    dz = LayerNorm dx (from dy) + dz_extra; dresidual = dz; dx = mask * dz / (1 - p)
    with the forward's mask regenerated from (seed, p); dbias = column sums of dx."""
    rows, cols = _mat(z, "z")
    for t, n in ((dy, "dy"), (dz_extra, "dz_extra")):
        if t is not None and (t.shape != z.shape or t.dtype != z.dtype):
            raise ValueError(f"{n} must match z")
        if t is not None:
            _mat(t, n)
    _vec(gamma, cols, z.dtype, "gamma")
    for t, n in ((mean, "mean"), (rstd, "rstd")):
        _vec(t, rows, torch.float32, n)
    dresidual = _out(dresidual, z.shape, z.dtype, z.device, "dresidual")
    dx = _out(dx, z.shape, z.dtype, z.device, "dx")
    dgamma = _out(dgamma, (cols,), torch.float32, z.device, "dgamma")
    dbeta = _out(dbeta, (cols,), torch.float32, z.device, "dbeta")
    dbias = _out(dbias, (cols,), torch.float32, z.device, "dbias")
    if workspace is None:
        workspace = dropout_workspace(rows, cols, z.device)
    if workspace.dtype != torch.float32 or not workspace.is_cuda:
        raise ValueError("workspace must be a float32 GPU tensor")
    if rows == 0:
        return dresidual, dx, dgamma.zero_(), dbeta.zero_(), dbias.zero_()
    _check(lib().bias_dropout_residual_ln_bwd(
        _ptr(dy), _ptr(dz_extra), _ptr(z), _ptr(gamma), _ptr(mean), _ptr(rstd),
        _ptr(dresidual), _ptr(dx), _ptr(dgamma), _ptr(dbeta), _ptr(dbias), _ptr(workspace),
        workspace.numel() * 4, rows, cols, float(p), int(seed) & 0xFFFFFFFFFFFFFFFF, _dt(z),
        _stream(z)))
    return dresidual, dx, dgamma, dbeta, dbias


def bias_dropout_residual_ln_bwd_dx(dy, z, gamma, mean, rstd, p: float, seed: int, *,
                                    workspace, dz_extra=None, dresidual=None, dx=None):
    """Stage 1 of bias_dropout_residual_ln_bwd -> (dresidual, dx); the column
    partials go to `workspace` (finish with bias_dropout_residual_ln_bwd_fold)."""
    rows, cols = _mat(z, "z")
    for t, n in ((dy, "dy"), (dz_extra, "dz_extra")):
        if t is not None and (t.shape != z.shape or t.dtype != z.dtype):
            raise ValueError(f"{n} must match z")
        if t is not None:
            _mat(t, n)
    _vec(gamma, cols, z.dtype, "gamma")
    for t, n in ((mean, "mean"), (rstd, "rstd")):
        _vec(t, rows, torch.float32, n)
    dresidual = _out(dresidual, z.shape, z.dtype, z.device, "dresidual")
    dx = _out(dx, z.shape, z.dtype, z.device, "dx")
    if workspace.dtype != torch.float32 or not workspace.is_cuda:
        raise ValueError("workspace must be a float32 GPU tensor")
    if rows == 0:
        return dresidual, dx
    _check(lib().bias_dropout_residual_ln_bwd_dx(
        _ptr(dy), _ptr(dz_extra), _ptr(z), _ptr(gamma), _ptr(mean), _ptr(rstd),
        _ptr(dresidual), _ptr(dx), _ptr(workspace), workspace.numel() * 4, rows, cols,
        float(p), int(seed) & 0xFFFFFFFFFFFFFFFF, _dt(z), _stream(z)))
    return dresidual, dx


def bias_dropout_residual_ln_bwd_fold(workspace, rows: int, cols: int, *, dgamma=None,
                                      dbeta=None, dbias=None):
    """Stage 2 of bias_dropout_residual_ln_bwd -> (dgamma, dbeta, dbias) float32."""
    device = workspace.device
    dgamma = _out(dgamma, (cols,), torch.float32, device, "dgamma")
    dbeta = _out(dbeta, (cols,), torch.float32, device, "dbeta")
    dbias = _out(dbias, (cols,), torch.float32, device, "dbias")
    if workspace.dtype != torch.float32 or not workspace.is_cuda:
        raise ValueError("workspace must be a float32 GPU tensor")
    if rows == 0:
        return dgamma.zero_(), dbeta.zero_(), dbias.zero_()
    _check(lib().bias_dropout_residual_ln_bwd_fold(
        _ptr(workspace), workspace.numel() * 4, _ptr(dgamma), _ptr(dbeta), _ptr(dbias),
        int(rows), int(cols), _stream(workspace)))
    return dgamma, dbeta, dbias


def attn_softmax_fwd(x, scale: float = 1.0, *, mask=None, rows_per_mask: int = 1,
                     causal: bool = False, p: float = 0.0, seed: int = 0, y=None,
                     y_dropped=None, want_dropped: bool = False):
    """Row softmax of scale*x + mask (+ causal mask) -> (y, y_dropped or None)."""
    rows, cols = _mat(x, "x")
    if mask is not None:
        mrows = (rows + rows_per_mask - 1) // max(rows_per_mask, 1)
        if (not mask.is_cuda or not mask.is_contiguous() or mask.dtype != x.dtype
                or mask.numel() != mrows * cols):
            raise ValueError(f"mask must be a contiguous GPU tensor [{mrows}, {cols}] {x.dtype}")
    y = _out(y, x.shape, x.dtype, x.device, "y")
    if want_dropped or y_dropped is not None:
        y_dropped = _out(y_dropped, x.shape, x.dtype, x.device, "y_dropped")
    if rows == 0:
        return y, y_dropped
    _check(lib().attn_softmax_fwd(_ptr(x), _ptr(mask), int(rows_per_mask), _ptr(y),
                                  _ptr(y_dropped), rows, cols, float(scale),
                                  1 if causal else 0, float(p),
                                  int(seed) & 0xFFFFFFFFFFFFFFFF, _dt(x), _stream(x)))
    return y, y_dropped


def attn_softmax_bwd(dy, y, scale: float = 1.0, *, causal: bool = False, p: float = 0.0,
                     seed: int = 0, dx=None):
    """dx of the attention softmax after the dropout backward (mask from seed, p)."""
    rows, cols = _mat(y, "y")
    if dy.shape != y.shape or dy.dtype != y.dtype:
        raise ValueError("dy must match y")
    _mat(dy, "dy")
    dx = _out(dx, y.shape, y.dtype, y.device, "dx")
    if rows == 0:
        return dx
    _check(lib().attn_softmax_bwd(_ptr(dy), _ptr(y), _ptr(dx), rows, cols, float(scale),
                                  1 if causal else 0, float(p),
                                  int(seed) & 0xFFFFFFFFFFFFFFFF, _dt(y), _stream(y)))
    return dx


def add_rmsnorm_fwd(x, gamma, eps: float = 1e-6, *, residual=None, residual_out=None,
                    y=None, rstd=None, stats: bool = True):
    """z = x + residual (x alone without one); y = RMSNorm(z) -> (z, y, rstd).

    Without a residual z is x itself (nothing is written); rstd is None when
    `stats` is false."""
    rows, cols = _mat(x, "x")
    if residual is not None:
        if residual.shape != x.shape or residual.dtype != x.dtype:
            raise ValueError("residual must match x")
        _mat(residual, "residual")
        residual_out = _out(residual_out, x.shape, x.dtype, x.device, "residual_out")
    elif residual_out is not None:
        raise ValueError("residual_out needs a residual")
    _vec(gamma, cols, x.dtype, "gamma")
    y = _out(y, x.shape, x.dtype, x.device, "y")
    if stats:
        rstd = _out(rstd, (rows,), torch.float32, x.device, "rstd")
    z = residual_out if residual is not None else x
    if rows == 0:
        return z, y, rstd
    _check(lib().add_rmsnorm_fwd(_ptr(x), _ptr(residual), _ptr(gamma), _ptr(residual_out),
                                 _ptr(y), _ptr(rstd), rows, cols, float(eps), _dt(x),
                                 _stream(x)))
    return z, y, rstd


def add_rmsnorm_bwd_workspace_bytes(rows: int, cols: int) -> int:
    return int(lib().add_rmsnorm_bwd_workspace_bytes(int(rows), int(cols)))


def rmsnorm_workspace(rows: int, cols: int, device) -> torch.Tensor:
    """A float32 workspace of the size add_rmsnorm_bwd needs."""
    n = add_rmsnorm_bwd_workspace_bytes(rows, cols) // 4
    return torch.empty(max(n, 1), dtype=torch.float32, device=device)


def add_rmsnorm_bwd(dy, z, gamma, rstd, *, dz_extra=None, dz=None, dgamma=None,
                    workspace=None):
    """Backward of add_rmsnorm_fwd -> (dz, dgamma).

    dz = RMSNorm dx (from dy) + dz_extra is the gradient of both x and the
    residual; dgamma (float32) = column sums of dy * z * rstd."""
    rows, cols = _mat(z, "z")
    for t, n in ((dy, "dy"), (dz_extra, "dz_extra")):
        if t is not None and (t.shape != z.shape or t.dtype != z.dtype):
            raise ValueError(f"{n} must match z")
        if t is not None:
            _mat(t, n)
    _vec(gamma, cols, z.dtype, "gamma")
    _vec(rstd, rows, torch.float32, "rstd")
    dz = _out(dz, z.shape, z.dtype, z.device, "dz")
    dgamma = _out(dgamma, (cols,), torch.float32, z.device, "dgamma")
    if workspace is None:
        workspace = rmsnorm_workspace(rows, cols, z.device)
    if workspace.dtype != torch.float32 or not workspace.is_cuda:
        raise ValueError("workspace must be a float32 GPU tensor")
    if rows == 0:
        return dz, dgamma.zero_()
    _check(lib().add_rmsnorm_bwd(_ptr(dy), _ptr(dz_extra), _ptr(z), _ptr(gamma), _ptr(rstd),
                                 _ptr(dz), _ptr(dgamma), _ptr(workspace), workspace.numel() * 4,
                                 rows, cols, _dt(z), _stream(z)))
    return dz, dgamma


def cross_entropy_fwd_bwd(logits, labels, *, cols: int = None, label_smoothing: float = 0.0,
                          grad_scale: float = 1.0, grad: bool = True, loss=None,
                          dlogits=None):
    """Label-smoothed cross-entropy of each row -> (loss float32 [rows], dlogits or None).

    logits is [..., ld]; the first `cols` columns (all by default) are the
    classes, the rest padding.  labels are int64 (negative: ignored row).
    dlogits = grad_scale * (softmax - target); pass dlogits=logits to
    overwrite the logits with it."""
    rows, ld = _mat(logits, "logits")
    cols = ld if cols is None else int(cols)
    if (not labels.is_cuda or not labels.is_contiguous() or labels.dtype != torch.int64
            or labels.numel() != rows):
        raise ValueError(f"labels must be a contiguous GPU int64 tensor of {rows} values")
    loss = _out(loss, (rows,), torch.float32, logits.device, "loss")
    if grad or dlogits is not None:
        dlogits = _out(dlogits, logits.shape, logits.dtype, logits.device, "dlogits")
    if rows == 0:
        return loss, dlogits
    _check(lib().cross_entropy_fwd_bwd(_ptr(logits), _ptr(labels), _ptr(loss), _ptr(dlogits),
                                       rows, cols, ld, float(label_smoothing),
                                       float(grad_scale), _dt(logits), _stream(logits)))
    return loss, dlogits


def hbm_copy(src, dst) -> None:
    """Copy src into dst (same byte size, device tensors, 16-byte aligned and
    sized, not overlapping) with the library's plain 16-byte copy kernel: the
    attainable-bandwidth reference for measurements."""
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("hbm_copy needs contiguous GPU tensors")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("hbm_copy: src and dst differ in size")
    _check(lib().hbm_copy(_ptr(src), _ptr(dst), nbytes, _stream(src)))


def hbm_stream(srcs, dsts) -> None:
    """Measurement reference: read every tensor of `srcs` (1-3) and write every
    tensor of `dsts` (0-2), all contiguous GPU tensors of one byte size."""
    ts = list(srcs) + list(dsts)
    if not ts or any(not t.is_cuda or not t.is_contiguous() for t in ts):
        raise ValueError("hbm_stream takes contiguous GPU tensors")
    nbytes = srcs[0].numel() * srcs[0].element_size()
    if any(t.numel() * t.element_size() != nbytes for t in ts):
        raise ValueError("hbm_stream tensors must have one byte size")
    s = (ctypes.c_void_p * max(1, len(srcs)))(*[t.data_ptr() for t in srcs])
    d = (ctypes.c_void_p * max(1, len(dsts)))(*[t.data_ptr() for t in dsts])
    _check(lib().hbm_stream(s, len(srcs), d, len(dsts), nbytes, _stream(srcs[0])))


def debug_force_path(lanes_per_row: int = 0, slots_per_lane: int = 0,
                     scalar: bool = False) -> None:
    """Test-only: force the row layout of later calls (0 restores the default)."""
    _check(lib().ln_debug_force_path(int(lanes_per_row), int(slots_per_lane),
                                     1 if scalar else 0))


def debug_force_staged(on: bool = False) -> None:
    """Test hook: route every LayerNorm call through the LDS-staged path."""
    _check(lib().ln_debug_force_staged(1 if on else 0))


def debug_force_two_pass(on: bool = False) -> None:
    """Test-only: softmax and cross-entropy calls take the two-pass path at
    every width (False restores the width-based choice)."""
    _check(lib().ln_debug_force_two_pass(1 if on else 0))


def debug_force_grid(workgroups_per_cu: int = 0) -> None:
    """Test-only: persistent-grid size of the forward (0 default, -1 one per block)."""
    _check(lib().ln_debug_force_grid(int(workgroups_per_cu)))
