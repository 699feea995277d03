"""GPU parity of the fused cross-entropy forward and backward
(cross_entropy_fwd_bwd: label-smoothed loss and q - p in one pass) against the
float64 oracle."""
import numpy as np
import pytest
import torch

import memory_bound_row_amd as mb
from memory_bound_row_amd import synth
from gpu_helpers import FMT, case, check_xent

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.float16, torch.bfloat16]
LAYOUTS_F32 = [(16, 1), (16, 2), (16, 4), (32, 2), (32, 4), (64, 2), (64, 4), (64, 8),
               (128, 4), (256, 4), (512, 4), (512, 8), (512, 13), (1024, 4), (1024, 6),
               (1024, 8), (1024, 10), (1024, 13), (1024, 16)]
LAYOUTS_16 = [(16, 1), (16, 2), (32, 1), (32, 2), (64, 1), (64, 2), (64, 4), (128, 4),
              (256, 4), (512, 4), (512, 7), (512, 10), (512, 13), (1024, 4), (1024, 5),
              (1024, 6), (1024, 7), (1024, 8), (1024, 10), (1024, 12), (1024, 14),
              (1024, 16), (1024, 18), (1024, 20)]
GPT2_V, GPT2_VP = 50257, 50304   # GPT-2's vocabulary and its padded row


def run(orc, rows, cols, ld, dtype, seed, alpha=0.1, scale=None, grad=True, ignore=0.0,
        name="xent", rows_sel=None, **kw):
    x = synth.logits(rows, ld, dtype, seed=seed, **kw).to("cuda")
    lab = synth.class_labels(rows, cols, seed=seed, ignore_frac=ignore).to("cuda")
    scale = 1.0 / max(rows, 1) if scale is None else scale
    loss, dx = mb.cross_entropy_fwd_bwd(x, lab, cols=cols, label_smoothing=alpha,
                                        grad_scale=scale, grad=grad)
    torch.cuda.synchronize()
    check_xent(orc, x, lab, cols, alpha, scale, loss, dx, FMT[dtype], rows_sel=rows_sel,
               name=name)
    return x, lab, loss, dx


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("scale", [None, 1.0], ids=["mean", "unit"])
def test_gpt2_vocabulary(orc, dtype, scale):
    # llm.c's fused classifier shape: V = 50257 classes in rows padded to 50304;
    # with the mean loss's 1/rows and with a unit gradient scale (the
    # gradient checked under the value-scaled rule either way)
    case(f"cross-entropy 256x{GPT2_V} (ld {GPT2_VP}) {dtype} scale={scale}")
    run(orc, 256, GPT2_V, GPT2_VP, dtype, 0, scale=scale, name="xent.gpt2")


def test_gpt2_full_batch_sampled(orc):
    # the measured workload (8 x 1024 tokens), checked on sampled rows
    case(f"cross-entropy 8192x{GPT2_V} bf16, sampled rows")
    sel = np.random.default_rng(5).choice(8192, 48, replace=False)
    sel = np.concatenate([sel, [0, 8191]])
    run(orc, 8192, GPT2_V, GPT2_VP, torch.bfloat16, 1, rows_sel=sel, name="xent.8192")


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("cols,ld", [(128256, 128256), (128255, 128255), (151936, 151936),
                                     (163840, 163840)])
def test_llama3_vocabulary(orc, dtype, cols, ld):
    # a 128K vocabulary (the lecture notes' example of logits outgrowing the
    # weights); the odd width takes the per-element path at 16 slots per lane;
    # 151936 classes (Qwen-2) and the widest 16-bit register row, 163840
    case(f"cross-entropy 40x{cols} ld {ld} {dtype}")
    run(orc, 40, cols, ld, dtype, 12, name=f"xent.{cols}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("cols,ld", [(1, 1), (2, 8), (7, 7), (8, 8), (100, 104), (1000, 1000),
                                     (1024, 1024), (4097, 4104), (32000, 32000)])
def test_small_shapes(orc, dtype, cols, ld):
    rows = 200 if cols <= 4104 else 24
    case(f"cross-entropy {rows}x{cols} ld {ld} {dtype}")
    run(orc, rows, cols, ld, dtype, 3, name=f"xent.{cols}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_forced_layouts(orc, dtype):
    layouts = LAYOUTS_F32 if dtype == torch.float32 else LAYOUTS_16
    e = 4 if dtype == torch.float32 else 8
    try:
        for g, v in layouts:
            ld = g * v * e - e                 # one slot short of full: idle lanes
            cols = ld - 3                      # a partial last slot of classes
            case(f"cross-entropy forced {g}x{v} cols={cols} ld={ld} {dtype}")
            mb.debug_force_path(g, v)
            run(orc, 37, cols, ld, dtype, 11, name=f"xent.{g}x{v}")
    finally:
        mb.debug_force_path(0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_per_element_path(orc, dtype):
    case(f"cross-entropy per-element path 100x1001 {dtype}")
    run(orc, 100, 1001, 1001, dtype, 4, name="xent.1001")   # rows not 16-byte aligned
    try:
        mb.debug_force_path(0, 0, scalar=True)
        run(orc, 64, 5000, 5008, dtype, 5, name="xent.scalar")
    finally:
        mb.debug_force_path(0)


@pytest.mark.parametrize("alpha", [0.0, 0.1, 1.0])
def test_label_smoothing(orc, alpha):
    case(f"cross-entropy label smoothing {alpha}")
    run(orc, 128, 3000, 3000, torch.bfloat16, 6, alpha=alpha, scale=1.0, name="xent.alpha")


def test_large_logits(orc):
    # the row maximum is subtracted: logits around 60 (exp would overflow fp32)
    case("cross-entropy large logits")
    run(orc, 64, 4096, 4096, torch.float32, 7, mean=60.0, std=8.0, name="xent.large")


def test_ignored_and_invalid_rows(orc):
    case("cross-entropy ignored rows")
    x, lab, loss, dx = run(orc, 300, 2048, 2048, torch.bfloat16, 8, ignore=0.2,
                           name="xent.ignore")
    ign = (lab < 0).cpu()
    assert ign.any()
    assert torch.all(loss.cpu()[ign] == 0) and torch.all(dx.cpu()[ign] == 0)
    # a label past the vocabulary has no target: NaN loss and gradient
    lab2 = lab.clone()
    lab2[3] = 2048
    loss2, dx2 = mb.cross_entropy_fwd_bwd(x, lab2)
    torch.cuda.synchronize()
    assert torch.isnan(loss2[3]) and torch.isnan(dx2[3]).all()
    keep = torch.ones(300, dtype=torch.bool)
    keep[3] = False
    assert torch.equal(loss2.cpu()[keep], mb.cross_entropy_fwd_bwd(x, lab)[0].cpu()[keep])


def test_in_place_and_loss_only():
    case("cross-entropy in place and loss only")
    x = synth.logits(512, GPT2_VP, torch.bfloat16, seed=9).to("cuda")
    lab = synth.class_labels(512, GPT2_V, seed=9).to("cuda")
    loss, dx = mb.cross_entropy_fwd_bwd(x, lab, cols=GPT2_V, label_smoothing=0.1,
                                        grad_scale=0.5)
    loss_only, none = mb.cross_entropy_fwd_bwd(x, lab, cols=GPT2_V, label_smoothing=0.1,
                                               grad=False)
    x2 = x.clone()
    loss2, dx2 = mb.cross_entropy_fwd_bwd(x2, lab, cols=GPT2_V, label_smoothing=0.1,
                                          grad_scale=0.5, dlogits=x2)
    torch.cuda.synchronize()
    assert none is None and dx2.data_ptr() == x2.data_ptr()
    assert torch.equal(loss, loss_only) and torch.equal(loss, loss2)
    assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16))


def test_gradient_rows_sum_to_zero():
    # sum_j (q_j - p_j) = 0 for every row with a target
    case("cross-entropy gradient row sums")
    x = synth.logits(256, 8192, torch.float32, seed=10).to("cuda")
    lab = synth.class_labels(256, 8192, seed=10).to("cuda")
    _, dx = mb.cross_entropy_fwd_bwd(x, lab, label_smoothing=0.1, grad_scale=1.0)
    torch.cuda.synchronize()
    assert torch.allclose(dx.cpu().double().sum(dim=1), torch.zeros(256, dtype=torch.float64),
                          atol=1e-5)


def test_empty():
    x = torch.empty((0, 100), dtype=torch.bfloat16, device="cuda")
    lab = torch.empty(0, dtype=torch.int64, device="cuda")
    loss, dx = mb.cross_entropy_fwd_bwd(x, lab)
    torch.cuda.synchronize()
    assert loss.shape == (0,) and dx.shape == (0, 100)


# Rows past the register layouts on the vector path are held by one workgroup,
# part of each lane's slots in registers and the rest in LDS: 16-bit rows
# 1024 lanes x (23 + 9) slots of 8 values, fp32 rows 512 lanes x (45 + 19)
# slots of 4.  Columns held in the register slots, and the widest row held:
REG_COLS = {torch.float32: 512 * 45 * 4, torch.float16: 1024 * 23 * 8,
            torch.bfloat16: 1024 * 23 * 8}
ONCHIP_MAX = {torch.float32: 131072, torch.float16: 262144, torch.bfloat16: 262144}


@pytest.mark.parametrize("dtype,cols,ld", [
    (torch.float32, 65537, 65540),     # the first fp32 width past the register layouts
    (torch.float32, 92160, 92160),     # the register slots exactly
    (torch.float32, 92161, 92164),     # one class in an LDS slot
    (torch.float32, 128256, 128256),   # Llama-3's vocabulary
    (torch.float32, 131071, 131072),   # the widest fp32 row held on chip
    (torch.bfloat16, 163841, 163848),  # the first 16-bit width past the register layouts
    (torch.float16, 188416, 188416),   # the register slots exactly
    (torch.bfloat16, 188417, 188424),  # one class in an LDS slot
    (torch.bfloat16, 256000, 256000),
    (torch.float16, 250001, 262144),   # padding up to the widest 16-bit row
    (torch.bfloat16, 262144, 262144),
])
def test_onchip_rows(orc, dtype, cols, ld):
    case(f"cross-entropy on chip {dtype} 24x{cols} ld {ld}")
    run(orc, 24, cols, ld, dtype, 13, ignore=0.1, name=f"xent.onchip.{cols}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_onchip_many_rows_per_workgroup(orc, dtype):
    # one workgroup per compute unit walks three or four rows: each row's LDS
    # slots and cross-wave exchange reuse the previous row's
    rows = 3 * 256 + 7
    cols = REG_COLS[dtype] + 20000   # rows of whole 16-byte slots: the vector path
    case(f"cross-entropy on chip {dtype} {rows}x{cols}, sampled rows")
    g = torch.Generator(device="cuda").manual_seed(14)
    x = (torch.randn((rows, cols), device="cuda", generator=g) * 2.0).to(dtype)
    lab = torch.randint(0, cols, (rows,), device="cuda", generator=g, dtype=torch.int64)
    loss, dx = mb.cross_entropy_fwd_bwd(x, lab, label_smoothing=0.1, grad_scale=1.0)
    torch.cuda.synchronize()
    sel = [0, 1, 255, 256, 257, 511, 512, 767, 768, rows - 1]
    check_xent(orc, x, lab, cols, 0.1, 1.0, loss, dx, FMT[dtype], rows_sel=sel,
               name="xent.onchip.rows")
    # every row's loss, against the oracle's loss alone
    loss_ref, _ = orc.cross_entropy(synth.as_f64(x), lab.cpu().numpy(), 0.1, 1.0, grad=False)
    err = np.abs(synth.as_f64(loss) - loss_ref) / np.maximum(1.0, np.abs(loss_ref))
    assert err.max() < 1e-4, err.max()


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
def test_onchip_label_and_maximum_in_lds_slots(orc, dtype):
    # rows whose maximum and label lie in the LDS slots, in the register
    # slots, and one of each
    rows, cols = 8, ONCHIP_MAX[dtype]
    case(f"cross-entropy on chip {dtype} {rows}x{cols}, label and maximum placed")
    x = synth.logits(rows, cols, dtype, seed=15)
    lab = synth.class_labels(rows, cols, seed=15)
    hi, lo = cols - 5, REG_COLS[dtype] // 3   # an LDS column and a register column
    b = REG_COLS[dtype]                        # the first column of the first LDS slot
    for r, (cmax, clab) in enumerate([(hi, hi), (lo, lo), (hi, lo), (lo, hi),
                                      (b, b), (b - 1, b - 1), (b - 1, b), (cols - 1, 0)]):
        x[r, cmax] = 12.0
        lab[r] = clab
    x, lab = x.to("cuda"), lab.to("cuda")
    loss, dx = mb.cross_entropy_fwd_bwd(x, lab, label_smoothing=0.1, grad_scale=1.0)
    torch.cuda.synchronize()
    check_xent(orc, x, lab, cols, 0.1, 1.0, loss, dx, FMT[dtype], name="xent.onchip.placed")


def test_onchip_ignored_invalid_in_place_and_loss_only(orc):
    rows, cols, ld = 40, 230001, 230008
    case(f"cross-entropy on chip bf16 {rows}x{cols}: ignored, invalid, in place, loss only")
    x, lab, loss, dx = run(orc, rows, cols, ld, torch.bfloat16, 16, ignore=0.25,
                           scale=1.0, name="xent.onchip.ignore")
    ign = (lab < 0).cpu()
    assert ign.any()
    assert torch.all(loss.cpu()[ign] == 0) and torch.all(dx.cpu()[ign] == 0)
    lab2 = lab.clone()
    lab2[3] = cols
    loss2, dx2 = mb.cross_entropy_fwd_bwd(x, lab2, cols=cols, label_smoothing=0.1,
                                          grad_scale=1.0)
    loss_only, none = mb.cross_entropy_fwd_bwd(x, lab, cols=cols, label_smoothing=0.1,
                                               grad=False)
    x3 = x.clone()
    loss3, dx3 = mb.cross_entropy_fwd_bwd(x3, lab, cols=cols, label_smoothing=0.1,
                                          grad_scale=1.0, dlogits=x3)
    torch.cuda.synchronize()
    assert torch.isnan(loss2[3]) and torch.isnan(dx2[3, :cols]).all()
    assert torch.all(dx2[3, cols:] == 0)
    keep = torch.ones(rows, dtype=torch.bool)
    keep[3] = False
    assert torch.equal(loss2.cpu()[keep], loss.cpu()[keep])
    assert none is None and torch.equal(loss, loss_only) and torch.equal(loss, loss3)
    assert dx3.data_ptr() == x3.data_ptr()
    assert torch.equal(dx.view(torch.int16), dx3.view(torch.int16))


@pytest.mark.parametrize("dtype,cols", [(torch.float32, 120000), (torch.bfloat16, 240000)])
def test_onchip_and_two_pass_paths_agree(orc, dtype, cols):
    # the same rows on the on-chip path and forced onto the two-pass walk:
    # both against the oracle, and their losses within float32 rounding
    case(f"cross-entropy {dtype} 16x{cols}: on chip and two-pass")
    x, lab, loss, dx = run(orc, 16, cols, cols, dtype, 17, scale=1.0, name="xent.onchip.ab")
    mb.debug_force_two_pass(True)
    try:
        loss2, dx2 = mb.cross_entropy_fwd_bwd(x, lab, label_smoothing=0.1, grad_scale=1.0)
        torch.cuda.synchronize()
    finally:
        mb.debug_force_two_pass(False)
    check_xent(orc, x, lab, cols, 0.1, 1.0, loss2, dx2, FMT[dtype], name="xent.twopass.ab")
    assert torch.allclose(loss, loss2, rtol=1e-5, atol=1e-5)
