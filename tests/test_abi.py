"""The C ABI on the CPU: the library loads, exports every symbol the public
headers declare, and rejects every invalid argument on the host (before any
HIP call, so these run without a GPU)."""
import ctypes
import glob
import os
import re

import pytest

import memory_bound_row_amd as mb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

LN_OK, LN_ERR_NULL, LN_ERR_SHAPE, LN_ERR_DTYPE, LN_ERR_PARAM = 0, 1, 2, 3, 4
LN_ERR_WORKSPACE, LN_ERR_UNSUPPORTED, LN_ERR_HIP, LN_ERR_SCRATCH = 5, 6, 7, 8
F32, F16, BF16 = 0, 1, 2

# fake but non-NULL device addresses: validation never dereferences them
A, B, C, D, E, F, G, H, I, J, K, M = (0x10000000 * k for k in range(1, 13))
STREAM_MAX = 1 << 24   # LN_MAX_COLS_STREAM


@pytest.fixture(scope="module")
def L():
    return mb.lib()


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(?:ln_status_t|size_t|const char\s*\*)\s*(\w+)\s*\(", text):
            names.add(m.group(1))
    return sorted(names)


def test_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert {"ln_fwd", "bias_dropout_residual_ln_fwd", "ln_bwd_dx", "ln_bwd_dgamma_dbeta",
            "ln_bwd_workspace_bytes", "ln_status_string", "bias_dropout_residual_ln_bwd",
            "bias_dropout_residual_ln_bwd_workspace_bytes", "attn_softmax_fwd",
            "attn_softmax_bwd", "add_rmsnorm_fwd", "add_rmsnorm_bwd",
            "add_rmsnorm_bwd_workspace_bytes", "cross_entropy_fwd_bwd"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in range(9):
        s = mb.status_string(code)
        assert s and s != "unknown ln_status_t"
    assert mb.status_string(99) == "unknown ln_status_t"


def test_workspace_bytes(L):
    assert L.ln_bwd_workspace_bytes(0, 10) == 0
    assert L.ln_bwd_workspace_bytes(10, 0) == 0
    assert L.ln_bwd_workspace_bytes(-1, 10) == 0
    # P = min(rows, 256) partitions of [2, cols] float32
    assert L.ln_bwd_workspace_bytes(8192, 1280) == 256 * 2 * 1280 * 4
    assert L.ln_bwd_workspace_bytes(64, 768) == 64 * 2 * 768 * 4
    assert L.ln_bwd_workspace_bytes(1, 7) == 1 * 2 * 7 * 4


def fwd(L, x=A, g=B, b=C, y=D, mean=None, rstd=None, rows=4, cols=8, eps=1e-5, dt=BF16):
    return L.ln_fwd(x, g, b, y, mean, rstd, rows, cols, eps, dt, None)


def test_ln_fwd_validation(L):
    assert fwd(L, x=None) == LN_ERR_NULL
    assert fwd(L, g=None) == LN_ERR_NULL
    assert fwd(L, b=None) == LN_ERR_NULL
    assert fwd(L, y=None) == LN_ERR_NULL
    assert fwd(L, rows=-1) == LN_ERR_SHAPE
    assert fwd(L, cols=0) == LN_ERR_SHAPE
    assert fwd(L, cols=-3) == LN_ERR_SHAPE
    assert fwd(L, dt=3) == LN_ERR_DTYPE
    assert fwd(L, dt=-1) == LN_ERR_DTYPE
    assert fwd(L, eps=-1e-6) == LN_ERR_PARAM
    assert fwd(L, eps=float("nan")) == LN_ERR_PARAM
    assert fwd(L, eps=float("inf")) == LN_ERR_PARAM
    assert fwd(L, cols=65537, dt=F32) == LN_ERR_UNSUPPORTED     # LN_MAX_COLS
    assert fwd(L, cols=65537, dt=BF16) == LN_ERR_UNSUPPORTED
    assert fwd(L, cols=65536, dt=F16, rows=0) == LN_OK
    assert fwd(L, cols=16385, dt=F32, rows=0) == LN_OK           # the LDS-staged path
    assert fwd(L, rows=2 ** 31) == LN_ERR_UNSUPPORTED
    assert fwd(L, rows=0) == LN_OK            # no-op, nothing enqueued
    # y may be x exactly, but not a partial overlap of it
    assert fwd(L, rows=0, y=A) == LN_OK
    assert fwd(L, y=A + 2) == LN_ERR_UNSUPPORTED
    # outputs must not overlap parameters or each other
    assert fwd(L, y=B) == LN_ERR_UNSUPPORTED
    assert fwd(L, mean=E, rstd=E) == LN_ERR_UNSUPPORTED
    assert fwd(L, mean=D + 8) == LN_ERR_UNSUPPORTED


def fused(L, x=A, bias=B, res=C, g=D, b=E, z=F, y=G, mean=None, rstd=None, mask=None,
          rows=4, cols=8, eps=1e-5, p=0.1, seed=0, dt=BF16):
    return L.bias_dropout_residual_ln_fwd(x, bias, res, g, b, z, y, mean, rstd, mask,
                                          rows, cols, eps, p, seed, dt, None)


def test_fused_fwd_validation(L):
    for k in ("x", "bias", "res", "g", "b", "z", "y"):
        assert fused(L, **{k: None}) == LN_ERR_NULL, k
    assert fused(L, rows=-5) == LN_ERR_SHAPE
    assert fused(L, cols=0) == LN_ERR_SHAPE
    assert fused(L, dt=7) == LN_ERR_DTYPE
    assert fused(L, p=-0.1) == LN_ERR_PARAM
    assert fused(L, p=1.0) == LN_ERR_PARAM
    assert fused(L, p=float("nan")) == LN_ERR_PARAM
    assert fused(L, eps=-1.0) == LN_ERR_PARAM
    assert fused(L, rows=0) == LN_OK
    assert fused(L, rows=0, z=C, y=A) == LN_OK                 # in place
    assert fused(L, z=G) == LN_ERR_UNSUPPORTED                  # z and y alias
    assert fused(L, z=B) == LN_ERR_UNSUPPORTED                  # z over bias
    assert fused(L, mask=A) == LN_ERR_UNSUPPORTED               # mask over x


def bwd_dx(L, dy=A, x=B, g=C, mean=D, rstd=E, dx=F, ws=None, wsb=0, rows=4, cols=8, dt=BF16):
    return L.ln_bwd_dx(dy, x, g, mean, rstd, dx, ws, wsb, rows, cols, dt, None)


def test_bwd_dx_validation(L):
    for k in ("dy", "x", "g", "mean", "rstd", "dx"):
        assert bwd_dx(L, **{k: None}) == LN_ERR_NULL, k
    assert bwd_dx(L, rows=-1) == LN_ERR_SHAPE
    assert bwd_dx(L, cols=0) == LN_ERR_SHAPE
    assert bwd_dx(L, dt=5) == LN_ERR_DTYPE
    need = L.ln_bwd_workspace_bytes(4, 8)
    assert bwd_dx(L, ws=G, wsb=need - 1) == LN_ERR_WORKSPACE
    assert bwd_dx(L, rows=0) == LN_OK
    assert bwd_dx(L, rows=0, dx=A) == LN_OK                     # dx == dy in place
    assert bwd_dx(L, dx=A + 4) == LN_ERR_UNSUPPORTED
    assert bwd_dx(L, ws=A, wsb=need) == LN_ERR_UNSUPPORTED      # workspace over dy
    # widest rows: LN_MAX_COLS_BWD_F32 / LN_MAX_COLS_BWD_16 (staged in LDS)
    assert bwd_dx(L, cols=19969, dt=F32) == LN_ERR_UNSUPPORTED
    assert bwd_dx(L, cols=32769, dt=BF16) == LN_ERR_UNSUPPORTED
    assert bwd_dx(L, cols=32769, dt=F16) == LN_ERR_UNSUPPORTED
    assert bwd_dx(L, cols=19968, dt=F32, rows=0) == LN_OK
    assert bwd_dx(L, cols=32768, dt=BF16, rows=0) == LN_OK


def dgdb(L, dy=A, x=B, mean=C, rstd=D, dg=E, db=F, ws=G, wsb=None, ready=0, rows=4, cols=8,
         dt=BF16):
    if wsb is None:
        wsb = L.ln_bwd_workspace_bytes(rows, cols)
    return L.ln_bwd_dgamma_dbeta(dy, x, mean, rstd, dg, db, ws, wsb, ready, rows, cols, dt,
                                 None)


def test_dgamma_dbeta_validation(L):
    for k in ("dg", "db", "ws"):
        assert dgdb(L, **{k: None}) == LN_ERR_NULL, k
    for k in ("dy", "x", "mean", "rstd"):
        assert dgdb(L, **{k: None}) == LN_ERR_NULL, k
        assert dgdb(L, rows=0, ready=1, **{k: None}) == LN_OK, k
    assert dgdb(L, wsb=L.ln_bwd_workspace_bytes(4, 8) - 4) == LN_ERR_WORKSPACE
    assert dgdb(L, rows=-2) == LN_ERR_SHAPE
    assert dgdb(L, dt=9) == LN_ERR_DTYPE
    assert dgdb(L, dg=F) == LN_ERR_UNSUPPORTED                  # dgamma over dbeta


def test_debug_force_path_validation(L):
    assert L.ln_debug_force_path(48, 1, 0) == LN_ERR_UNSUPPORTED
    assert L.ln_debug_force_path(64, 9, 0) == LN_ERR_UNSUPPORTED
    assert L.ln_debug_force_path(128, 3, 0) == LN_ERR_UNSUPPORTED
    assert L.ln_debug_force_path(128, 2, 0) == LN_OK          # prologue-backward layout
    assert L.ln_debug_force_path(0, 0, 0) == LN_OK
    assert L.ln_debug_force_path(1024, 9, 0) == LN_ERR_UNSUPPORTED
    assert L.ln_debug_force_path(1024, 16, 0) == LN_OK
    assert L.ln_debug_force_path(1024, 13, 0) == LN_OK        # cross-entropy layout
    assert L.ln_debug_force_path(64, 3, 0) == LN_OK
    assert L.ln_debug_force_path(0, 0, 0) == LN_OK


def test_dropout_bwd_workspace_bytes(L):
    f = L.bias_dropout_residual_ln_bwd_workspace_bytes
    assert f(0, 10) == 0 and f(10, 0) == 0 and f(-1, 10) == 0
    # the same P partitions as the LayerNorm backward, three kinds of partials
    assert f(8192, 1280) == 256 * 3 * 1280 * 4
    assert f(64, 768) == 64 * 3 * 768 * 4
    assert f(5, 7) * 2 == L.ln_bwd_workspace_bytes(5, 7) * 3


def drop_bwd(L, dy=A, ez=None, z=B, g=C, mean=D, rstd=E, dres=F, dx=G, dg=H, db=I, dbias=J,
             ws=K, wsb=None, rows=4, cols=8, p=0.1, seed=0, dt=BF16):
    if wsb is None:
        wsb = L.bias_dropout_residual_ln_bwd_workspace_bytes(rows, cols)
    return L.bias_dropout_residual_ln_bwd(dy, ez, z, g, mean, rstd, dres, dx, dg, db, dbias,
                                          ws, wsb, rows, cols, p, seed, dt, None)


def test_dropout_bwd_validation(L):
    for k in ("dy", "z", "g", "mean", "rstd", "dres", "dx", "dg", "db", "dbias", "ws"):
        assert drop_bwd(L, **{k: None}) == LN_ERR_NULL, k
    assert drop_bwd(L, rows=0) == LN_OK                       # dz_extra may be NULL
    assert drop_bwd(L, rows=0, ez=M) == LN_OK
    assert drop_bwd(L, rows=-1) == LN_ERR_SHAPE
    assert drop_bwd(L, cols=0) == LN_ERR_SHAPE
    assert drop_bwd(L, dt=5) == LN_ERR_DTYPE
    for p in (-0.1, 1.0, float("nan")):
        assert drop_bwd(L, p=p) == LN_ERR_PARAM, p
    for dt in (F32, F16, BF16):
        assert drop_bwd(L, cols=8193, dt=dt) == LN_ERR_UNSUPPORTED, dt
        assert drop_bwd(L, cols=8192, rows=0, dt=dt) == LN_OK, dt
    need = L.bias_dropout_residual_ln_bwd_workspace_bytes(4, 8)
    assert drop_bwd(L, wsb=need - 4) == LN_ERR_WORKSPACE
    assert drop_bwd(L, wsb=L.ln_bwd_workspace_bytes(4, 8)) == LN_ERR_WORKSPACE
    # in place on one input each is allowed (checked on an empty call) ...
    assert drop_bwd(L, rows=0, dres=A, dx=B) == LN_OK
    # ... but the two outputs may not coincide, or partially overlap inputs
    assert drop_bwd(L, dres=G) == LN_ERR_UNSUPPORTED
    assert drop_bwd(L, dres=A + 2) == LN_ERR_UNSUPPORTED
    assert drop_bwd(L, dbias=H) == LN_ERR_UNSUPPORTED             # dbias over dgamma
    assert drop_bwd(L, ws=B) == LN_ERR_UNSUPPORTED                # workspace over z
    assert drop_bwd(L, rows=0, dx=M, ez=M) == LN_OK               # in place on dz_extra


def sm_fwd(L, x=A, mask=None, rpm=1, y=B, yd=None, rows=4, cols=8, scale=1.0, causal=0, p=0.0,
           seed=0, dt=BF16):
    return L.attn_softmax_fwd(x, mask, rpm, y, yd, rows, cols, scale, causal, p, seed, dt, None)


def sm_bwd(L, dy=A, y=B, dx=C, rows=4, cols=8, scale=1.0, causal=0, p=0.0, seed=0, dt=BF16):
    return L.attn_softmax_bwd(dy, y, dx, rows, cols, scale, causal, p, seed, dt, None)


def test_softmax_validation(L):
    assert sm_fwd(L, x=None) == LN_ERR_NULL
    assert sm_fwd(L, y=None) == LN_ERR_NULL
    assert sm_fwd(L, rows=0) == LN_OK                             # mask, y_dropped nullable
    assert sm_fwd(L, rows=-1) == LN_ERR_SHAPE
    assert sm_fwd(L, cols=0) == LN_ERR_SHAPE
    assert sm_fwd(L, dt=4) == LN_ERR_DTYPE
    assert sm_fwd(L, cols=STREAM_MAX + 1) == LN_ERR_UNSUPPORTED
    assert sm_fwd(L, cols=16385, rows=0) == LN_OK                 # long rows: two-pass path
    for kw in ({"scale": float("inf")}, {"scale": float("nan")}, {"causal": 2},
               {"p": 1.0}, {"p": -0.5}, {"mask": C, "rpm": 0}):
        assert sm_fwd(L, **kw) == LN_ERR_PARAM, kw
    assert sm_fwd(L, rows=0, y=A) == LN_OK                        # in place
    assert sm_fwd(L, yd=B) == LN_ERR_UNSUPPORTED                  # y_dropped over y
    assert sm_fwd(L, y=A + 2) == LN_ERR_UNSUPPORTED
    assert sm_fwd(L, mask=C, rpm=2, y=C) == LN_ERR_UNSUPPORTED    # y over the mask
    for k in ("dy", "y", "dx"):
        assert sm_bwd(L, **{k: None}) == LN_ERR_NULL, k
    assert sm_bwd(L, rows=0, dx=A) == LN_OK
    assert sm_bwd(L, rows=0, dx=B) == LN_OK
    assert sm_bwd(L, dx=B + 4) == LN_ERR_UNSUPPORTED
    assert sm_bwd(L, scale=float("inf")) == LN_ERR_PARAM
    assert sm_bwd(L, p=1.0) == LN_ERR_PARAM
    assert sm_bwd(L, cols=STREAM_MAX + 1) == LN_ERR_UNSUPPORTED
    assert sm_bwd(L, cols=STREAM_MAX, rows=0) == LN_OK



def rms_fwd(L, x=A, res=B, g=C, z=D, y=E, rstd=None, rows=4, cols=8, eps=1e-6, dt=BF16):
    return L.add_rmsnorm_fwd(x, res, g, z, y, rstd, rows, cols, eps, dt, None)


def rms_bwd(L, dy=A, ez=None, z=B, g=C, rstd=D, dz=E, dg=F, ws=G, wsb=None, rows=4, cols=8,
            dt=BF16):
    if wsb is None:
        wsb = L.add_rmsnorm_bwd_workspace_bytes(rows, cols)
    return L.add_rmsnorm_bwd(dy, ez, z, g, rstd, dz, dg, ws, wsb, rows, cols, dt, None)


def test_rmsnorm_workspace_bytes(L):
    f = L.add_rmsnorm_bwd_workspace_bytes
    assert f(0, 10) == 0 and f(10, 0) == 0 and f(-1, 10) == 0
    # the same P partitions as the LayerNorm backward, one kind of partial
    assert f(8192, 4096) == 256 * 4096 * 4
    assert f(5, 7) * 2 == L.ln_bwd_workspace_bytes(5, 7)


def test_rmsnorm_validation(L):
    for k in ("x", "g", "y", "z"):
        assert rms_fwd(L, **{k: None}) == LN_ERR_NULL, k      # z required with a residual
    assert rms_fwd(L, res=None, z=None, rows=0) == LN_OK        # plain RMSNorm
    assert rms_fwd(L, res=None) == LN_ERR_PARAM                 # z without a residual
    assert rms_fwd(L, rows=0, rstd=F) == LN_OK
    assert rms_fwd(L, rows=-1) == LN_ERR_SHAPE
    assert rms_fwd(L, cols=0) == LN_ERR_SHAPE
    assert rms_fwd(L, dt=3) == LN_ERR_DTYPE
    assert rms_fwd(L, cols=16385) == LN_ERR_UNSUPPORTED
    for eps in (-1e-6, float("nan"), float("inf")):
        assert rms_fwd(L, eps=eps) == LN_ERR_PARAM, eps
    assert rms_fwd(L, rows=0, z=B, y=A) == LN_OK                # in place on both inputs
    assert rms_fwd(L, y=D) == LN_ERR_UNSUPPORTED                # y over z
    assert rms_fwd(L, z=A + 2) == LN_ERR_UNSUPPORTED
    assert rms_fwd(L, rstd=C) == LN_ERR_UNSUPPORTED             # rstd over gamma
    for k in ("dy", "z", "g", "rstd", "dz", "dg", "ws"):
        assert rms_bwd(L, **{k: None}) == LN_ERR_NULL, k
    assert rms_bwd(L, rows=0) == LN_OK                          # dz_extra may be NULL
    assert rms_bwd(L, rows=0, ez=M, dz=M) == LN_OK              # in place on dz_extra
    assert rms_bwd(L, rows=0, dz=A) == LN_OK
    assert rms_bwd(L, rows=-1) == LN_ERR_SHAPE
    assert rms_bwd(L, dt=7) == LN_ERR_DTYPE
    assert rms_bwd(L, cols=16385) == LN_ERR_UNSUPPORTED
    need = L.add_rmsnorm_bwd_workspace_bytes(4, 8)
    assert rms_bwd(L, wsb=need - 4) == LN_ERR_WORKSPACE
    assert rms_bwd(L, dz=B + 2) == LN_ERR_UNSUPPORTED
    assert rms_bwd(L, dg=D) == LN_ERR_UNSUPPORTED               # dgamma over rstd
    assert rms_bwd(L, ws=F) == LN_ERR_UNSUPPORTED               # workspace over dgamma


def xent(L, x=A, lab=B, loss=C, dx=None, rows=4, cols=8, ld=8, alpha=0.0, scale=1.0, dt=BF16):
    return L.cross_entropy_fwd_bwd(x, lab, loss, dx, rows, cols, ld, alpha, scale, dt, None)


def test_cross_entropy_validation(L):
    for k in ("x", "lab", "loss"):
        assert xent(L, **{k: None}) == LN_ERR_NULL, k
    assert xent(L, rows=0) == LN_OK                             # dlogits may be NULL
    assert xent(L, rows=0, dx=A) == LN_OK                       # in place on the logits
    assert xent(L, rows=0, dx=D) == LN_OK
    assert xent(L, rows=-1) == LN_ERR_SHAPE
    assert xent(L, cols=0) == LN_ERR_SHAPE
    assert xent(L, cols=9, ld=8) == LN_ERR_SHAPE                # ld < cols
    assert xent(L, dt=3) == LN_ERR_DTYPE
    assert xent(L, cols=65536, ld=65536, rows=0, dt=F32) == LN_OK
    assert xent(L, cols=65537, ld=65537, rows=0, dt=F32) == LN_OK     # two-pass path
    assert xent(L, cols=STREAM_MAX + 1, ld=STREAM_MAX + 1, dt=F32) == LN_ERR_UNSUPPORTED
    assert xent(L, cols=100, ld=STREAM_MAX + 1, dt=F32) == LN_ERR_UNSUPPORTED
    for dt in (F16, BF16):
        assert xent(L, cols=131072, ld=131072, rows=0, dt=dt) == LN_OK
        assert xent(L, cols=163840, ld=163840, rows=0, dt=dt) == LN_OK
        assert xent(L, cols=131073, ld=131073, rows=0, dt=dt) == LN_OK
        assert xent(L, cols=STREAM_MAX + 1, ld=STREAM_MAX + 1, dt=dt) == LN_ERR_UNSUPPORTED
    for kw in ({"alpha": -0.1}, {"alpha": 1.5}, {"alpha": float("nan")},
               {"scale": float("inf")}, {"scale": float("nan")}):
        assert xent(L, **kw) == LN_ERR_PARAM, kw
    assert xent(L, rows=0, alpha=1.0) == LN_OK
    assert xent(L, dx=A + 2) == LN_ERR_UNSUPPORTED              # partial overlap of logits
    assert xent(L, dx=B) == LN_ERR_UNSUPPORTED                  # dlogits over the labels
    assert xent(L, loss=B) == LN_ERR_UNSUPPORTED                # loss over the labels
    assert xent(L, loss=A) == LN_ERR_UNSUPPORTED                # loss over the logits


def test_hbm_copy_validation(L):
    assert L.hbm_copy(A, B, 0, None) == LN_OK             # no-op, nothing launched
    assert L.hbm_copy(None, B, 16, None) == LN_ERR_NULL
    assert L.hbm_copy(A, None, 16, None) == LN_ERR_NULL
    assert L.hbm_copy(A, B, 17, None) == LN_ERR_PARAM     # not a whole number of vectors
    assert L.hbm_copy(A + 8, B, 16, None) == LN_ERR_PARAM
    assert L.hbm_copy(A, B + 4, 16, None) == LN_ERR_PARAM
    assert L.hbm_copy(A, A + 16, 64, None) == LN_ERR_PARAM   # overlapping ranges
    assert L.hbm_copy(A + 16, A, 64, None) == LN_ERR_PARAM
    assert L.hbm_copy(A, A, 16, None) == LN_ERR_PARAM


def test_prologue_backward_stage_validation(L):
    # stage 1: the combined call's checks without the [cols] outputs
    ws = 1 << 40
    args = dict(dy=A, ez=None, z=B, g=C, mean=D, rstd=E, dres=F, dx=G, ws=ws, wsb=1 << 30,
                rows=4, cols=8, p=0.1, seed=1, dt=BF16)

    def st1(**kw):
        a = dict(args, **kw)
        return L.bias_dropout_residual_ln_bwd_dx(a["dy"], a["ez"], a["z"], a["g"], a["mean"],
                                                 a["rstd"], a["dres"], a["dx"], a["ws"],
                                                 a["wsb"], a["rows"], a["cols"], a["p"],
                                                 a["seed"], a["dt"], None)
    assert st1(dy=None) == LN_ERR_NULL
    assert st1(ws=None) == LN_ERR_NULL
    assert st1(rows=-1) == LN_ERR_SHAPE
    assert st1(p=1.0) == LN_ERR_PARAM
    assert st1(wsb=4) == LN_ERR_WORKSPACE
    assert st1(cols=8193) == LN_ERR_UNSUPPORTED
    assert st1(dt=9) == LN_ERR_DTYPE
    assert st1(rows=0) == LN_OK

    def fold(ws=ws, wsb=1 << 30, dg=D, db=E, dbias=F, rows=4, cols=8):
        return L.bias_dropout_residual_ln_bwd_fold(ws, wsb, dg, db, dbias, rows, cols, None)
    assert fold(ws=None) == LN_ERR_NULL
    assert fold(dbias=None) == LN_ERR_NULL
    assert fold(rows=-1) == LN_ERR_SHAPE
    assert fold(cols=0) == LN_ERR_SHAPE
    assert fold(cols=8193) == LN_ERR_UNSUPPORTED
    assert fold(wsb=8) == LN_ERR_WORKSPACE
    assert fold(dg=ws) == LN_ERR_UNSUPPORTED            # output over the partials
    assert fold(rows=0) == LN_OK


def test_roctx_ranges_switched_on_do_not_change_results():
    # MBROW_ROCTX=1 wraps every entry point in a roctx range (no tool attached
    # here): the calls still validate and return as without it
    import subprocess
    import sys
    code = ("import ctypes, memory_bound_row_amd as mb; L = mb.lib(); "
            "print(L.ln_fwd(None, None, None, None, None, None, 4, 8, ctypes.c_float(1e-5), 0, None), "
            "L.attn_softmax_fwd(None, None, 1, None, None, 4, 8, ctypes.c_float(1.0), 0, "
            "ctypes.c_float(0.0), ctypes.c_uint64(0), 0, None))")
    env = dict(os.environ, MBROW_ROCTX="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split() == [str(LN_ERR_NULL), str(LN_ERR_NULL)]
