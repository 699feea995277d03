"""GPU parity of the attention softmax forward (scale, additive and causal
masks, dropout output) and of its backward fused with the dropout backward,
against the float64 oracle."""
import numpy as np
import pytest
import torch

import memory_bound_row_amd as mb
from memory_bound_row_amd import synth
from gpu_helpers import FMT, case, check_softmax_bwd, check_softmax_fwd, dev

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.float16, torch.bfloat16]
SM_LAYOUTS_F32 = [(16, 1), (16, 2), (16, 4), (32, 2), (32, 4), (64, 2), (64, 4), (64, 8),
                  (128, 4), (256, 4), (512, 4), (1024, 4), (1024, 5), (1024, 6), (1024, 7),
                  (1024, 8)]
SM_LAYOUTS_16 = [(16, 1), (16, 2), (32, 1), (32, 2), (64, 1), (64, 2), (64, 4), (128, 4),
                 (256, 4), (512, 4), (512, 6), (512, 8), (1024, 3), (1024, 4), (1024, 5),
                 (1024, 6), (1024, 7), (1024, 8)]
# the register layouts' widest rows (LN_MAX_COLS_SOFTMAX_*)
MAX_FWD = {torch.float32: 32768, torch.float16: 65536, torch.bfloat16: 65536}
MAX_BWD = {torch.float32: 32768, torch.float16: 49152, torch.bfloat16: 49152}


def scores(rows, cols, dtype, seed=0, std=3.0):
    """Attention scores ~ N(0, std) and an upstream gradient ~ N(0, 1)."""
    d = synth.layer_inputs(rows, cols, dtype, seed=seed, x_std=std, names=("x", "dy"))
    return dev(d)


def run(rows, cols, dtype, scale, causal, p, seed, mask=None, rows_per_mask=1, data_seed=0):
    d = scores(rows, cols, dtype, data_seed)
    y, yd = mb.attn_softmax_fwd(d["x"], scale, mask=mask, rows_per_mask=rows_per_mask,
                                causal=causal, p=p, seed=seed, want_dropped=p > 0)
    dx = mb.attn_softmax_bwd(d["dy"], y, scale, causal=causal, p=p, seed=seed)
    torch.cuda.synchronize()
    return d, y, yd, dx


def check(orc, d, y, yd, dx, scale, causal, p, seed, mask=None, rows_per_mask=1, name="sm"):
    fmt = FMT[y.dtype]
    check_softmax_fwd(orc, d["x"], y, yd, fmt, scale=scale, mask=mask,
                      rows_per_mask=rows_per_mask, causal=causal, p=p, seed=seed,
                      name=f"{name}.fwd")
    check_softmax_bwd(orc, d["dy"], y, dx, fmt, scale=scale, p=p, seed=seed,
                      name=f"{name}.bwd")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", [(2 * 16 * 256, 256), (8 * 16 * 512, 512)])
def test_pages_attention_shapes(orc, shape, dtype):
    """Batch 2 x 16 heads x 256 x 256 with the causal mask, and 8 x 16 x 512 x
    512 with dropout (the pages' examples), in every storage type, under the
    value-scaled rule (y is about 1/512 here)."""
    rows, cols = shape
    causal, p = (True, 0.0) if cols == 256 else (False, 0.1)
    case(f"softmax {rows}x{cols} {dtype} causal={causal} p={p}")
    scale = 1.0 / np.sqrt(64.0)
    d, y, yd, dx = run(rows, cols, dtype, scale, causal, p, 3)
    check(orc, d, y, yd, dx, scale, causal, p, 3, name=f"sm.{rows}x{cols}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("cols", [1, 7, 8, 31, 32, 33, 100, 256, 1000, 1024, 4096, 8200,
                                  16384])
def test_widths(orc, dtype, cols):
    rows = 96 if cols <= 4096 else 12
    case(f"softmax {rows}x{cols} {dtype}")
    d, y, yd, dx = run(rows, cols, dtype, 0.5, False, 0.2, 9, data_seed=cols)
    check(orc, d, y, yd, dx, 0.5, False, 0.2, 9, name=f"sm.{cols}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("cols", [8, 64, 100, 512, 1024])
def test_causal(orc, dtype, cols):
    rows = 2 * cols + 3                      # two score blocks and part of a third
    case(f"softmax causal {rows}x{cols} {dtype}")
    d, y, yd, dx = run(rows, cols, dtype, 1.0, True, 0.1, 5, data_seed=7)
    check(orc, d, y, yd, dx, 1.0, True, 0.1, 5, name=f"sm.causal.{cols}")
    q = torch.arange(rows, device="cuda") % cols
    j = torch.arange(cols, device="cuda")
    assert torch.all(y[j[None, :] > q[:, None]] == 0)
    assert torch.all(dx[j[None, :] > q[:, None]] == 0)


@pytest.mark.parametrize("dtype", DTYPES)
def test_additive_mask(orc, dtype):
    rows, cols, rpm = 128, 200, 32
    case(f"softmax additive mask {rows}x{cols} {dtype}")
    mk = torch.zeros((rows // rpm, cols), dtype=torch.float32)
    mk[0, 10:50] = -torch.inf                # padded keys of the first batch
    mk[1, :] = 2.0                           # a constant shift changes nothing
    mk[2, 190:] = -torch.inf
    mk[3, :] = -torch.inf                    # every key masked: zeros
    mask = mk.to(dtype).cuda()
    d, y, yd, dx = run(rows, cols, dtype, 0.8, False, 0.15, 2, mask=mask, rows_per_mask=rpm)
    check(orc, d, y, yd, dx, 0.8, False, 0.15, 2, mask=mask, rows_per_mask=rpm,
          name="sm.mask")
    assert torch.all(y[:32, 10:50] == 0) and torch.all(y[96:] == 0)


@pytest.mark.parametrize("dtype", DTYPES)
def test_forced_layouts(orc, dtype):
    layouts = SM_LAYOUTS_F32 if dtype == torch.float32 else SM_LAYOUTS_16
    e = 4 if dtype == torch.float32 else 8
    try:
        for g, v in layouts:
            cols = g * v * e - e
            if cols <= 0:
                continue
            case(f"softmax forced {g}x{v} cols={cols} {dtype}")
            mb.debug_force_path(g, v)
            d, y, yd, dx = run(40, cols, dtype, 1.0, cols >= 64, 0.3, 4)
            check(orc, d, y, yd, dx, 1.0, cols >= 64, 0.3, 4, name=f"sm.{g}x{v}")
    finally:
        mb.debug_force_path(0)


@pytest.mark.parametrize("dtype", DTYPES)
def test_forced_wide_layouts_without_dropped_copy(orc, dtype):
    # forwards that write no dropped copy (fp32 wide rows take an instance
    # built without the dropout rounds), causal and not, with the backward
    layouts = SM_LAYOUTS_F32 if dtype == torch.float32 else SM_LAYOUTS_16
    e = 4 if dtype == torch.float32 else 8
    try:
        for g, v in layouts:
            if g < 512:
                continue
            cols = g * v * e - 3 * e
            causal = v % 2 == 1
            case(f"softmax forced {g}x{v} cols={cols} {dtype}, no dropped copy, causal={causal}")
            mb.debug_force_path(g, v)
            d, y, yd, dx = run(24, cols, dtype, 0.7, causal, 0.0, 5)
            assert yd is None
            check(orc, d, y, yd, dx, 0.7, causal, 0.0, 5, name=f"sm.plain.{g}x{v}")
    finally:
        mb.debug_force_path(0)


WIDE = {torch.float32: [16385, 20000, 32767, 32768],
        torch.float16: [16385, 24577, 49152, 65536],
        torch.bfloat16: [16392, 40000, 49153, 65536]}


@pytest.mark.parametrize("dtype", DTYPES)
def test_wide_rows(orc, dtype):
    """Rows past 16384 columns in the lean 1024-lane register layouts (each
    pass recomputes from the packed row), with dropout; up to the widest row
    each direction holds (wider 16-bit backward rows take the two-pass path)."""
    for cols in WIDE[dtype]:
        assert cols <= MAX_FWD[dtype]
        case(f"softmax wide {6}x{cols} {dtype} (backward in registers: {cols <= MAX_BWD[dtype]})")
        d, y, yd, dx = run(6, cols, dtype, 0.5, False, 0.1, 11, data_seed=cols)
        check(orc, d, y, yd, dx, 0.5, False, 0.1, 11, name=f"sm.wide.{cols}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_wide_rows_mask_causal_and_per_element(orc, dtype):
    cols = 20000 if dtype == torch.float32 else 30000   # rows of whole 16-byte slots
    case(f"softmax wide additive mask {6}x{cols} {dtype}")
    mk = torch.zeros((3, cols), dtype=torch.float32)
    mk[0, 100:9000] = -torch.inf             # padded keys
    mk[1, :] = 1.5
    mk[2, :] = -torch.inf                    # every key masked: zeros
    mask = mk.to(dtype).cuda()
    d, y, yd, dx = run(6, cols, dtype, 0.7, False, 0.2, 12, mask=mask, rows_per_mask=2)
    check(orc, d, y, yd, dx, 0.7, False, 0.2, 12, mask=mask, rows_per_mask=2,
          name="sm.wide.mask")
    assert torch.all(y[4:] == 0)
    # causal rows 0-47 of a wide row (keys past the query are not read)
    case(f"softmax wide causal 48x{cols} {dtype}")
    d, y, yd, dx = run(48, cols, dtype, 1.0, True, 0.1, 13)
    check(orc, d, y, yd, dx, 1.0, True, 0.1, 13, name="sm.wide.causal")
    # rows that are not a whole number of 16-byte slots: per-element loads
    # and stores
    case(f"softmax wide per-element path 5x{cols + 1} {dtype}")
    d, y, yd, dx = run(5, cols + 1, dtype, 0.5, True, 0.1, 14)
    check(orc, d, y, yd, dx, 0.5, True, 0.1, 14, name="sm.wide.odd")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_per_element_path(orc, dtype):
    case(f"softmax per-element path {dtype}")
    try:
        mb.debug_force_path(0, 0, scalar=True)
        d, y, yd, dx = run(64, 333, dtype, 0.5, True, 0.1, 8)
        check(orc, d, y, yd, dx, 0.5, True, 0.1, 8, name="sm.scalar")
    finally:
        mb.debug_force_path(0)


def test_rows_sum_to_one_and_p_zero():
    case("softmax row sums, p = 0")
    d, y, yd, dx = run(1000, 777, torch.float32, 1.0, False, 0.0, 0)
    assert torch.allclose(y.double().sum(dim=1), torch.ones(1000, dtype=torch.float64,
                                                            device="cuda"), atol=1e-5)
    y2, yd2 = mb.attn_softmax_fwd(d["x"], 1.0, p=0.0, want_dropped=True)
    torch.cuda.synchronize()
    assert torch.equal(yd2, y2) and torch.equal(y2, y)
    # each row of dx sums to 0 (softmax ignores a constant added to its input)
    assert torch.allclose(dx.double().sum(dim=1), torch.zeros(1000, dtype=torch.float64,
                                                              device="cuda"), atol=1e-5)


def test_in_place():
    case("softmax in place")
    d, y, yd, dx = run(300, 512, torch.bfloat16, 0.5, True, 0.1, 6)
    x2, dy2 = d["x"].clone(), d["dy"].clone()
    y2, _ = mb.attn_softmax_fwd(x2, 0.5, causal=True, p=0.1, seed=6, y=x2)
    dx2 = mb.attn_softmax_bwd(dy2, y2, 0.5, causal=True, p=0.1, seed=6, dx=dy2)
    torch.cuda.synchronize()
    assert torch.equal(y2, y) and torch.equal(dx2, dx)


# 16-bit forwards without a mask row stay in registers past
# LN_MAX_COLS_SOFTMAX_16, up to LN_MAX_COLS_SOFTMAX_PLAIN_FWD_16 (1024 lanes x
# 10, 12, 14 or 16 slots), with or without the dropped copy; backwards are
# held on chip (dy in registers, y in registers and LDS) past
# LN_MAX_COLS_SOFTMAX_BWD_16, up to LN_MAX_COLS_SOFTMAX_PLAIN_BWD_16, with or
# without dropout.
PLAIN_FWD_MAX = 131072


@pytest.mark.parametrize("p", [0.0, 0.1])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("cols", [65544, 81920, 98312, 114688, 120008, PLAIN_FWD_MAX])
def test_plain_forward_long_rows(orc, dtype, cols, p):
    seed = 2 ** 63 + cols
    case(f"softmax plain forward 6x{cols} {dtype} p={p} (registers), backward on chip")
    d, y, yd, dx = run(6, cols, dtype, 0.5, False, p, seed, data_seed=cols)
    assert (yd is None) == (p == 0)
    check(orc, d, y, yd, dx, 0.5, False, p, seed, name=f"sm.plain.{cols}")


@pytest.mark.parametrize("p", [0.0, 0.1])
@pytest.mark.parametrize("cols", [32772, 40960, 49152, 57344, 60004, 65536])
def test_plain_long_rows_fp32(orc, cols, p):
    # fp32 rows past LN_MAX_COLS_SOFTMAX_F32: forward in registers without a
    # mask, backward on chip (up to 65536), with and without dropout
    seed = 2 ** 63 + cols
    case(f"softmax plain fp32 6x{cols} p={p}: forward in registers, backward on chip")
    d, y, yd, dx = run(6, cols, torch.float32, 0.5, False, p, seed, data_seed=cols)
    check(orc, d, y, yd, dx, 0.5, False, p, seed, name=f"sm.plain32.{cols}")


def test_plain_forward_long_rows_many_per_workgroup_and_causal(orc):
    # three or four rows per workgroup (one workgroup per compute unit), rows
    # sampled; then causal rows (keys past the query are not read)
    rows, cols = 3 * 256 + 9, 100000
    case(f"softmax plain forward {rows}x{cols} fp16, sampled rows")
    g = torch.Generator(device="cuda").manual_seed(31)
    x = (torch.randn((rows, cols), device="cuda", generator=g) * 3.0).to(torch.float16)
    y, _ = mb.attn_softmax_fwd(x, 0.25)
    torch.cuda.synchronize()
    sel = torch.as_tensor([0, 1, 255, 256, 511, 512, 767, 768, rows - 1], device="cuda")
    check_softmax_fwd(orc, x[sel], y[sel], None, FMT[torch.float16], scale=0.25,
                      name="sm.plain.rows")
    dy = (torch.randn((rows, cols), device="cuda", generator=g)).to(torch.float16)
    dx = mb.attn_softmax_bwd(dy, y, 0.25)
    torch.cuda.synchronize()
    check_softmax_bwd(orc, dy[sel], y[sel], dx[sel], FMT[torch.float16], scale=0.25,
                      name="sm.plain.rows.bwd")
    case(f"softmax plain forward and backward, causal 40x{cols} bf16")
    d = scores(40, cols, torch.bfloat16, 32)
    y, _ = mb.attn_softmax_fwd(d["x"], 0.5, causal=True)
    dx = mb.attn_softmax_bwd(d["dy"], y, 0.5, causal=True)
    torch.cuda.synchronize()
    check_softmax_fwd(orc, d["x"], y, None, FMT[torch.bfloat16], scale=0.5, causal=True,
                      name="sm.plain.causal")
    check_softmax_bwd(orc, d["dy"], y, dx, FMT[torch.bfloat16], scale=0.5,
                      name="sm.plain.causal.bwd")
    assert torch.all(dx[:, 64:] == 0)
    case(f"softmax backward on chip with dropout, causal 40x{cols} bf16")
    dx = mb.attn_softmax_bwd(d["dy"], y, 0.5, causal=True, p=0.2, seed=2 ** 63 + 11)
    torch.cuda.synchronize()
    check_softmax_bwd(orc, d["dy"], y, dx, FMT[torch.bfloat16], scale=0.5, p=0.2,
                      seed=2 ** 63 + 11, name="sm.plain.causal.bwd.drop")
    assert torch.all(dx[:, 64:] == 0)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_plain_forward_long_rows_agree_with_two_pass(orc, dtype):
    # the same rows on chip and forced onto the two-pass walk, without and
    # with the dropped copy (also written over x) and with a mask row
    cols = 110000
    case(f"softmax plain forward 8x{cols} {dtype}: registers, two-pass, mask, dropout")
    d = scores(8, cols, dtype, 33)
    y, _ = mb.attn_softmax_fwd(d["x"], 0.5)
    mb.debug_force_two_pass(True)
    try:
        y2, _ = mb.attn_softmax_fwd(d["x"], 0.5)
    finally:
        mb.debug_force_two_pass(False)
    mask = (torch.randn((1, cols), device="cuda",
                        generator=torch.Generator(device="cuda").manual_seed(34))).to(dtype)
    y3, _ = mb.attn_softmax_fwd(d["x"], 0.5, mask=mask, rows_per_mask=8)
    y4, yd4 = mb.attn_softmax_fwd(d["x"], 0.5, p=0.1, seed=35, want_dropped=True)
    mb.debug_force_two_pass(True)
    try:
        y3b, _ = mb.attn_softmax_fwd(d["x"], 0.5, mask=mask, rows_per_mask=8)
    finally:
        mb.debug_force_two_pass(False)
    x6 = d["x"].clone()
    y6, yd6 = mb.attn_softmax_fwd(x6, 0.5, p=0.1, seed=35, y_dropped=x6)
    mb.debug_force_two_pass(True)
    try:
        y5, yd5 = mb.attn_softmax_fwd(d["x"], 0.5, p=0.1, seed=35, want_dropped=True)
    finally:
        mb.debug_force_two_pass(False)
    torch.cuda.synchronize()
    fmt = FMT[dtype]
    check_softmax_fwd(orc, d["x"], y, None, fmt, scale=0.5, name="sm.plain.reg")
    check_softmax_fwd(orc, d["x"], y2, None, fmt, scale=0.5, name="sm.plain.2pass")
    check_softmax_fwd(orc, d["x"], y3, None, fmt, scale=0.5, mask=mask, rows_per_mask=8,
                      name="sm.plain.mask")
    check_softmax_fwd(orc, d["x"], y3b, None, fmt, scale=0.5, mask=mask, rows_per_mask=8,
                      name="sm.plain.mask.2pass")
    check_softmax_fwd(orc, d["x"], y4, yd4, fmt, scale=0.5, p=0.1, seed=35,
                      name="sm.plain.drop")
    check_softmax_fwd(orc, d["x"], y5, yd5, fmt, scale=0.5, p=0.1, seed=35,
                      name="sm.plain.drop.2pass")
    assert yd6.data_ptr() == x6.data_ptr()
    assert torch.equal(y6.view(torch.int16), y4.view(torch.int16))
    assert torch.equal(yd6.view(torch.int16), yd4.view(torch.int16))


def _mask_rows(nmask, cols, dtype, seed, dead=()):
    """Additive mask rows: N(0, 1), about a tenth of the keys -inf, and the
    rows in `dead` -inf everywhere (their softmax rows are all 0)."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    mask = torch.randn((nmask, cols), device="cuda", generator=g)
    mask[torch.rand((nmask, cols), device="cuda", generator=g) < 0.1] = float("-inf")
    for r in dead:
        mask[r] = float("-inf")
    return mask.to(dtype)


@pytest.mark.parametrize("p", [0.0, 0.1])
@pytest.mark.parametrize("dtype", DTYPES)
def test_masked_forward_long_rows_on_chip(orc, dtype, p):
    # a mask row past the register layouts: the scores in registers, the mask
    # row in registers and LDS; one and three rows per mask row (7 rows, so
    # the last mask row serves one), a mask row that masks every key, the
    # full width, one slot short and a shorter row
    e = 4 if dtype == torch.float32 else 8
    full = 65536 if dtype == torch.float32 else PLAIN_FWD_MAX
    shorter = 40000 if dtype == torch.float32 else 70000
    for cols in (full, full - e, shorter):
        for rpm in (1, 3):
            rows, seed = 7, 2 ** 63 + cols + rpm
            case(f"softmax masked forward on chip 7x{cols} {dtype} rows_per_mask={rpm} p={p}")
            d = scores(rows, cols, dtype, cols + rpm)
            nmask = (rows + rpm - 1) // rpm
            mask = _mask_rows(nmask, cols, dtype, cols + 7 * rpm, dead=(1,))
            y, yd = mb.attn_softmax_fwd(d["x"], 0.5, mask=mask, rows_per_mask=rpm, p=p,
                                        seed=seed, want_dropped=p > 0)
            torch.cuda.synchronize()
            check_softmax_fwd(orc, d["x"], y, yd, FMT[dtype], scale=0.5, mask=mask,
                              rows_per_mask=rpm, p=p, seed=seed, name=f"sm.mask.{cols}.{rpm}")
            dead = range(rpm, min(2 * rpm, rows))
            assert torch.all(y[list(dead)] == 0)


def test_masked_forward_long_rows_many_per_workgroup_and_causal(orc):
    # more rows than workgroups (rows sampled, each with its own mask row
    # spelled out for the oracle), then causal rows with a mask and the
    # dropped copy, and the result written over x
    rows, cols, rpm = 2 * 256 + 5, 100000, 16
    case(f"softmax masked forward on chip {rows}x{cols} bf16, rows_per_mask={rpm}, sampled")
    d = scores(rows, cols, torch.bfloat16, 41)
    mask = _mask_rows((rows + rpm - 1) // rpm, cols, torch.bfloat16, 42, dead=(3,))
    y, _ = mb.attn_softmax_fwd(d["x"], 0.25, mask=mask, rows_per_mask=rpm)
    torch.cuda.synchronize()
    ids = [0, 1, 47, 48, 255, 256, 511, rows - 1]
    sel = torch.as_tensor(ids, device="cuda")
    mrows = torch.as_tensor([r // rpm for r in ids], device="cuda")
    check_softmax_fwd(orc, d["x"][sel], y[sel], None, FMT[torch.bfloat16], scale=0.25,
                      mask=mask[mrows].contiguous(), rows_per_mask=1, name="sm.mask.rows")
    assert torch.all(y[48:64] == 0)
    case(f"softmax masked forward on chip, causal 40x{cols} fp16 with the dropped copy")
    d = scores(40, cols, torch.float16, 43)
    mask = _mask_rows(5, cols, torch.float16, 44)
    x2 = d["x"].clone()
    y, yd = mb.attn_softmax_fwd(d["x"], 0.5, mask=mask, rows_per_mask=8, causal=True, p=0.2,
                                seed=45, want_dropped=True)
    y2, _ = mb.attn_softmax_fwd(x2, 0.5, mask=mask, rows_per_mask=8, causal=True, p=0.2,
                                seed=45, y=x2)
    torch.cuda.synchronize()
    check_softmax_fwd(orc, d["x"], y, yd, FMT[torch.float16], scale=0.5, mask=mask,
                      rows_per_mask=8, causal=True, p=0.2, seed=45, name="sm.mask.causal")
    assert torch.all(y[:, 64:] == 0) and torch.all(yd[:, 64:] == 0)
    assert y2.data_ptr() == x2.data_ptr()
    assert torch.equal(y2.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("dtype", DTYPES)
def test_plain_backward_long_rows_in_place_and_two_pass(orc, dtype):
    # the backward held on chip, without and with dropout: in place over dy
    # and over y, and the same rows forced onto the two-pass walk
    rows, cols = 10, (49152 if dtype == torch.float32 else 98304)
    case(f"softmax backward on chip {rows}x{cols} {dtype}: in place, two-pass, dropout")
    d = scores(rows, cols, dtype, 36)
    y, _ = mb.attn_softmax_fwd(d["x"], 0.5)
    dx = mb.attn_softmax_bwd(d["dy"], y, 0.5)
    dy2, y3 = d["dy"].clone(), y.clone()
    dx2 = mb.attn_softmax_bwd(dy2, y, 0.5, dx=dy2)
    dx3 = mb.attn_softmax_bwd(d["dy"], y3, 0.5, dx=y3)
    dx5 = mb.attn_softmax_bwd(d["dy"], y, 0.5, p=0.1, seed=37)
    dy6, y7 = d["dy"].clone(), y.clone()
    dx6 = mb.attn_softmax_bwd(dy6, y, 0.5, p=0.1, seed=37, dx=dy6)
    dx7 = mb.attn_softmax_bwd(d["dy"], y7, 0.5, p=0.1, seed=37, dx=y7)
    mb.debug_force_two_pass(True)
    try:
        dx4 = mb.attn_softmax_bwd(d["dy"], y, 0.5)
        dx8 = mb.attn_softmax_bwd(d["dy"], y, 0.5, p=0.1, seed=37)
    finally:
        mb.debug_force_two_pass(False)
    torch.cuda.synchronize()
    fmt = FMT[dtype]
    check_softmax_bwd(orc, d["dy"], y, dx, fmt, scale=0.5, name="sm.plainbwd")
    check_softmax_bwd(orc, d["dy"], y, dx4, fmt, scale=0.5, name="sm.plainbwd.2pass")
    check_softmax_bwd(orc, d["dy"], y, dx5, fmt, scale=0.5, p=0.1, seed=37,
                      name="sm.plainbwd.drop")
    check_softmax_bwd(orc, d["dy"], y, dx8, fmt, scale=0.5, p=0.1, seed=37,
                      name="sm.plainbwd.drop.2pass")
    assert dx2.data_ptr() == dy2.data_ptr() and dx3.data_ptr() == y3.data_ptr()
    assert dx6.data_ptr() == dy6.data_ptr() and dx7.data_ptr() == y7.data_ptr()
    ibits = torch.int32 if dtype == torch.float32 else torch.int16
    assert torch.equal(dx.view(ibits), dx2.view(ibits))
    assert torch.equal(dx.view(ibits), dx3.view(ibits))
    assert torch.equal(dx5.view(ibits), dx6.view(ibits))
    assert torch.equal(dx5.view(ibits), dx7.view(ibits))
