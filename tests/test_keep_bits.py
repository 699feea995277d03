"""The dropout keep bits that each kernel actually applies, read back and
compared bit for bit with the oracle's mask ("Accelerating Transformer on GPU
(II)" §3.3: the mask is regenerated from the stored seed, so the forward, the
backward and the oracle must draw the same bits).

The inputs are chosen so that every output element shows whether the kernel
kept it, independently of any tolerance:

* bias_dropout_residual_ln_fwd with x = 0.75, bias = 0.25, residual = 0:
  z = round_T(1/(1-p)) where kept and exactly 0 where dropped;
* bias_dropout_residual_ln_bwd with dy = 0 and dz_extra = 1: the LayerNorm's
  dx is exactly 0, so dz = 1, dresidual = 1 everywhere and
  dx = round_T(1/(1-p)) where kept, exactly 0 where dropped;
* attn_softmax_fwd with x = 0: y = 1/L and y_dropped is y/(1-p) where kept,
  exactly 0 where dropped;
* attn_softmax_bwd with dy = 1 and y = round_T(1/(2L)): with g = keep/(1-p),
  dx_j = scale * y * (g_j - sum_k g_k y) is > 0 exactly where kept (the sum
  is at most g/2) and < 0 where dropped when the row keeps anything (0 when
  it keeps nothing).

Every storage type, the full configuration shape 8192 x 1280 with the seeds 0,
1 and 2^63 + 5, and every row layout each kernel is built with, on the vector
and the per-element path (ragged widths); and the softmax rows past the
register layouts (held on chip, or read twice)."""
import numpy as np
import pytest
import torch

import memory_bound_row_amd as mb
from gpu_helpers import case

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.float16, torch.bfloat16]
SEEDS = [0, 1, 2 ** 63 + 5]

LN_LAYOUTS = {4: [(16, 1), (16, 2), (16, 4), (16, 8)] + [(32, v) for v in range(1, 9)]
              + [(64, v) for v in range(1, 9)] + [(128, 4), (256, 4), (512, 4), (1024, 4)],
              8: [(16, 1), (16, 2), (16, 4)] + [(32, v) for v in range(1, 6)]
              + [(64, v) for v in range(1, 6)] + [(128, 4), (256, 4), (512, 4)]}
DROP_LAYOUTS = {4: [(16, 1), (16, 2), (16, 4), (32, 1), (32, 2), (32, 3), (32, 4), (64, 1),
                    (64, 2), (64, 3), (64, 4), (64, 5), (64, 6), (128, 4), (256, 4), (512, 4)],
                8: [(16, 1), (16, 2), (32, 1), (32, 2), (32, 3), (64, 1), (64, 2), (64, 3),
                    (128, 2), (256, 2), (512, 2)]}
SM_LAYOUTS = {4: [(16, 1), (16, 2), (16, 4), (32, 2), (32, 4), (64, 2), (64, 4), (64, 8),
                  (128, 4), (256, 4), (512, 4), (1024, 4), (1024, 5), (1024, 6), (1024, 7),
                  (1024, 8)],
              8: [(16, 1), (16, 2), (32, 1), (32, 2), (64, 1), (64, 2), (64, 4), (128, 4),
                  (256, 4), (512, 4), (512, 6), (512, 8), (1024, 3), (1024, 4), (1024, 5),
                  (1024, 6), (1024, 7), (1024, 8)]}
SM_BWD_MAX_V16 = 6     # the 16-bit softmax backward stops at 1024 x 6


def _elems(dtype):
    return 4 if dtype == torch.float32 else 8


def _stored(v, dtype):
    return float(torch.tensor(v, dtype=torch.float32).to(dtype).float())


@pytest.fixture(autouse=True)
def _default_path():
    mb.debug_force_path(0)
    yield
    mb.debug_force_path(0)


def _assert_bits(got_keep, orc_keep, what):
    got = got_keep.cpu().numpy().astype(np.uint8)
    diff = np.argwhere(got != orc_keep)
    assert diff.size == 0, (f"{what}: {len(diff)} keep bits differ from the oracle, "
                            f"first at {diff[:5].tolist()}")


def fused_forward_bits(rows, cols, dtype, p, seed):
    x = torch.full((rows, cols), 0.75, dtype=dtype, device="cuda")
    res = torch.zeros((rows, cols), dtype=dtype, device="cuda")
    bias = torch.full((cols,), 0.25, dtype=dtype, device="cuda")
    gamma = torch.ones(cols, dtype=dtype, device="cuda")
    beta = torch.zeros(cols, dtype=dtype, device="cuda")
    z, _, _, _, _ = mb.bias_dropout_residual_ln_fwd(x, bias, res, gamma, beta, p, seed,
                                                    stats=False)
    torch.cuda.synchronize()
    kept_val = _stored(1.0 / (1.0 - np.float32(p)), dtype)
    zf = z.float()
    assert torch.all((zf == 0) | (zf == kept_val)), "z holds a value other than 0 or 1/(1-p)"
    return zf != 0


def prologue_backward_bits(rows, cols, dtype, p, seed):
    z = torch.randn((rows, cols), device="cuda").to(dtype)
    dy = torch.zeros((rows, cols), dtype=dtype, device="cuda")
    ez = torch.ones((rows, cols), dtype=dtype, device="cuda")
    gamma = torch.ones(cols, dtype=dtype, device="cuda")
    mean = torch.zeros(rows, dtype=torch.float32, device="cuda")
    rstd = torch.ones(rows, dtype=torch.float32, device="cuda")
    dres, dx, _, _, dbias = mb.bias_dropout_residual_ln_bwd(dy, z, gamma, mean, rstd, p, seed,
                                                            dz_extra=ez)
    torch.cuda.synchronize()
    assert torch.all(dres.float() == 1.0), "dresidual is not dz = 1"
    kept_val = _stored(1.0 / (1.0 - np.float32(p)), dtype)
    dxf = dx.float()
    assert torch.all((dxf == 0) | (dxf == kept_val)), "dx holds a value other than 0 or 1/(1-p)"
    keep = dxf != 0
    # dbias counts the kept rows of each column, times 1/(1-p)
    scale = float(np.float32(1.0 / (1.0 - np.float64(np.float32(p)))))
    want = keep.sum(dim=0).double() * scale
    assert torch.allclose(dbias.double(), want, rtol=2e-5, atol=0), "dbias != kept count / (1-p)"
    return keep


def softmax_forward_bits(rows, cols, dtype, p, seed, masked=False):
    # masked: one all-zero mask row for every row, so y is still 1/L
    x = torch.zeros((rows, cols), dtype=dtype, device="cuda")
    mask = torch.zeros((1, cols), dtype=dtype, device="cuda") if masked else None
    y, yd = mb.attn_softmax_fwd(x, 1.0, mask=mask, rows_per_mask=rows, p=p, seed=seed,
                                want_dropped=True)
    torch.cuda.synchronize()
    assert torch.all(y > 0)
    return yd != 0


def softmax_backward_bits(rows, cols, dtype, p, seed):
    dy = torch.ones((rows, cols), dtype=dtype, device="cuda")
    y = torch.full((rows, cols), 1.0 / (2 * cols), dtype=dtype, device="cuda")
    dx = mb.attn_softmax_bwd(dy, y, float(cols), p=p, seed=seed)
    torch.cuda.synchronize()
    keep = dx > 0
    # dropped positions: negative where the row keeps anything, else exactly 0
    row_any = keep.any(dim=1, keepdim=True)
    neg_ok = torch.where(row_any, dx < 0, dx == 0)
    assert torch.all(keep | neg_ok), "a dropped position has dx >= 0 in a row that keeps some"
    return keep


KERNELS = {"fused_fwd": fused_forward_bits, "prologue_bwd": prologue_backward_bits,
           "softmax_fwd": softmax_forward_bits, "softmax_bwd": softmax_backward_bits}


@pytest.mark.parametrize("kernel", list(KERNELS))
@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f16", "bf16"])
@pytest.mark.parametrize("seed", SEEDS)
def test_keep_bits_config_shape(orc, kernel, dtype, seed):
    rows, cols, p = 8192, 1280, 0.1
    case(f"keep bits {kernel} {dtype} {rows}x{cols} p={p} seed={seed}")
    got = KERNELS[kernel](rows, cols, dtype, p, seed)
    _assert_bits(got, orc.dropout_keep(seed, p, rows, cols), f"{kernel} {dtype} seed {seed}")


def _layout_cases(layouts, e, scalar):
    for g, v in layouts:
        cols = g * v * e - e                 # one slot short of full: idle lanes
        if scalar:
            cols -= 3                        # a partial last slot
        if cols >= 1:
            yield g, v, cols


@pytest.mark.parametrize("scalar", [False, True], ids=["vec", "scalar"])
@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f16", "bf16"])
@pytest.mark.parametrize("kernel", list(KERNELS))
def test_keep_bits_every_layout(orc, kernel, dtype, scalar):
    e = _elems(dtype)
    table = {"fused_fwd": LN_LAYOUTS, "prologue_bwd": DROP_LAYOUTS,
             "softmax_fwd": SM_LAYOUTS, "softmax_bwd": SM_LAYOUTS}[kernel]
    rows, p = 37, 0.25
    for g, v, cols in _layout_cases(table[e], e, scalar):
        if kernel == "softmax_bwd" and e == 8 and g == 1024 and v > SM_BWD_MAX_V16:
            continue
        for seed in (3, 2 ** 63 + 5):
            case(f"keep bits {kernel} forced {g}x{v} scalar={scalar} {dtype} {rows}x{cols} "
                 f"seed={seed}")
            mb.debug_force_path(g, v, scalar)
            try:
                got = KERNELS[kernel](rows, cols, dtype, p, seed)
            finally:
                mb.debug_force_path(0)
            _assert_bits(got, orc.dropout_keep(seed, p, rows, cols),
                         f"{kernel} {g}x{v} scalar={scalar} {dtype} seed {seed}")


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f16", "bf16"])
def test_keep_bits_long_rows(orc, dtype):
    # rows past the register layouts: the softmax forward and backward held on
    # chip (more rows than workgroups, so each walks several; a full row of
    # 1024 lanes x 16 slots, one slot short, and a shorter row), then the
    # two-pass forward and backward (forced) on the same widths
    e = _elems(dtype)
    full = 65536 if dtype == torch.float32 else 131072
    shorter = 40000 if dtype == torch.float32 else 70000
    p = 0.25
    for rows, cols in ((2 * 256 + 3, full), (9, full - e), (9, shorter)):
        for seed in (5, 2 ** 63 + 5):
            want = orc.dropout_keep(seed, p, rows, cols)
            for kernel in ("softmax_fwd", "softmax_fwd_masked", "softmax_bwd"):
                case(f"keep bits {kernel} on chip {dtype} {rows}x{cols} seed={seed}")
                if kernel == "softmax_fwd_masked":
                    got = softmax_forward_bits(rows, cols, dtype, p, seed, masked=True)
                else:
                    got = KERNELS[kernel](rows, cols, dtype, p, seed)
                _assert_bits(got, want, f"{kernel} on chip {dtype} {rows}x{cols} seed {seed}")
    for kernel in ("softmax_fwd", "softmax_bwd"):
        for cols in (full - e, shorter):
            rows, seed = 9, 2 ** 63 + 5
            case(f"keep bits {kernel} two-pass {dtype} {rows}x{cols} seed={seed}")
            mb.debug_force_two_pass(True)
            try:
                got = KERNELS[kernel](rows, cols, dtype, p, seed)
            finally:
                mb.debug_force_two_pass(False)
            _assert_bits(got, orc.dropout_keep(seed, p, rows, cols),
                         f"{kernel} two-pass {dtype} {rows}x{cols} seed {seed}")
