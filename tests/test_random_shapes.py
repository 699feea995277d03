"""GPU parity on seeded random shapes: every entry point on widths drawn
log-uniformly over its supported range, random row counts, all storage types,
and tensors that start one element into their allocation (base addresses not
16-byte aligned, which forces the per-element paths).  Each case is checked
against the float64 oracle with the same helpers as the targeted tests."""
import numpy as np
import pytest
import torch

import memory_bound_row_amd as mb
from memory_bound_row_amd import synth
from gpu_helpers import (EPS, FMT, case, check_bwd, check_dropout_bwd, check_fused, check_fwd,
                         check_rmsnorm_bwd, check_rmsnorm_fwd, check_softmax_bwd,
                         check_softmax_fwd, check_xent)

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.float16, torch.bfloat16]
KINDS = ["layernorm", "fused", "prologue_bwd", "softmax", "rmsnorm", "xent"]
MAX_COLS = {"layernorm": 16384, "fused": 16384, "prologue_bwd": 8192, "softmax": 16384,
            "rmsnorm": 16384, "xent": 60000}
N_CASES = 72


def draw(idx):
    """Shape of case idx: (kind, dtype, rows, cols, misaligned)."""
    g = np.random.default_rng([2024, idx])
    kind = KINDS[idx % len(KINDS)]
    dtype = DTYPES[int(g.integers(0, 3))]
    cols = int(np.exp(g.uniform(0.0, np.log(MAX_COLS[kind]))))
    cols = max(1, cols)
    budget = 3_000_000 if kind == "xent" else 1_500_000
    rows = int(g.integers(1, max(2, min(400, budget // cols))))
    misaligned = bool(g.integers(0, 4) == 0)
    return kind, dtype, rows, cols, misaligned


def place(t, misaligned):
    """t on the GPU, optionally starting one element into a larger buffer."""
    if not misaligned:
        return t.to("cuda")
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
    out = buf[1:].view(t.shape)
    out.copy_(t.to("cuda"))
    return out


@pytest.mark.parametrize("idx", range(N_CASES))
def test_random_shape(orc, idx):
    kind, dtype, rows, cols, mis = draw(idx)
    case(f"random case {idx}: {kind} {rows}x{cols} {dtype} misaligned={mis}")
    fmt = FMT[dtype]
    seed = 1000 + idx
    if kind in ("layernorm", "fused", "prologue_bwd"):
        cpu = synth.layer_inputs(rows, cols, dtype, seed=seed)
        d = {k: place(v, mis) for k, v in cpu.items()}
        if kind == "layernorm":
            y, mean, rstd = mb.ln_fwd(d["x"], d["gamma"], d["beta"], EPS)
            dx, dg, db = mb.ln_bwd(d["dy"], d["x"], d["gamma"], mean, rstd)
            torch.cuda.synchronize()
            check_fwd(orc, d["x"], d["gamma"], d["beta"], y, mean, rstd, fmt, name="rnd.fwd")
            check_bwd(orc, d["dy"], d["x"], d["gamma"], mean, rstd, dx, dg, db, fmt,
                      name="rnd.bwd")
        elif kind == "fused":
            z, y, mean, rstd, mask = mb.bias_dropout_residual_ln_fwd(
                d["x"], d["bias"], d["residual"], d["gamma"], d["beta"], 0.15, seed, EPS,
                want_mask=True)
            torch.cuda.synchronize()
            check_fused(orc, d, 0.15, seed, z, y, mean, rstd, mask, fmt, name="rnd.fused")
        else:
            z, _, mean, rstd, _ = mb.bias_dropout_residual_ln_fwd(
                d["x"], d["bias"], d["residual"], d["gamma"], d["beta"], 0.15, seed, EPS)
            ez = place(synth.layer_inputs(rows, cols, dtype, seed=seed + 1,
                                          names=("dy",))["dy"], mis)
            dres, dx, dg, db, dbias = mb.bias_dropout_residual_ln_bwd(
                d["dy"], z, d["gamma"], mean, rstd, 0.15, seed, dz_extra=ez)
            torch.cuda.synchronize()
            check_dropout_bwd(orc, d["dy"], ez, z, d["gamma"], mean, rstd, 0.15, seed, dres,
                              dx, dg, db, dbias, fmt, name="rnd.drop_bwd")
    elif kind == "softmax":
        cpu = synth.layer_inputs(rows, cols, dtype, seed=seed, x_std=3.0, names=("x", "dy"))
        x, dy = place(cpu["x"], mis), place(cpu["dy"], mis)
        y, yd = mb.attn_softmax_fwd(x, 0.5, p=0.1, seed=seed, want_dropped=True)
        dx = mb.attn_softmax_bwd(dy, y, 0.5, p=0.1, seed=seed)
        torch.cuda.synchronize()
        check_softmax_fwd(orc, x, y, yd, fmt, scale=0.5, p=0.1, seed=seed, name="rnd.sm")
        check_softmax_bwd(orc, dy, y, dx, fmt, scale=0.5, p=0.1, seed=seed, name="rnd.sm_bwd")
    elif kind == "rmsnorm":
        cpu = synth.layer_inputs(rows, cols, dtype, seed=seed,
                                 names=("x", "residual", "gamma", "dy"))
        d = {k: place(v, mis) for k, v in cpu.items()}
        z, y, rstd = mb.add_rmsnorm_fwd(d["x"], d["gamma"], 1e-6, residual=d["residual"])
        dz, dg = mb.add_rmsnorm_bwd(d["dy"], z, d["gamma"], rstd, dz_extra=d["residual"])
        torch.cuda.synchronize()
        check_rmsnorm_fwd(orc, d["x"], d["residual"], d["gamma"], z, y, rstd, fmt, 1e-6,
                          name="rnd.rms")
        check_rmsnorm_bwd(orc, d["dy"], d["residual"], z, d["gamma"], rstd, dz, dg, fmt,
                          name="rnd.rms_bwd")
    else:
        ld = cols + int(np.random.default_rng([7, idx]).integers(0, 9))
        x = place(synth.logits(rows, ld, dtype, seed=seed), mis)
        lab = synth.class_labels(rows, cols, seed=seed, ignore_frac=0.05).to("cuda")
        loss, dx = mb.cross_entropy_fwd_bwd(x, lab, cols=cols, label_smoothing=0.1,
                                            grad_scale=0.25)
        torch.cuda.synchronize()
        check_xent(orc, x, lab, cols, 0.1, 0.25, loss, dx, fmt, name="rnd.xent")


@pytest.mark.parametrize("idx", range(10))
def test_random_long_softmax_rows(orc, idx):
    """The softmax's long-row register layouts (16385-65536 columns) on
    seeded random widths, dtypes, scales, dropout rates and masks."""
    g = np.random.default_rng([4711, idx])
    dtype = DTYPES[int(g.integers(0, 3))]
    top = 32768 if dtype == torch.float32 else 65536
    cols = int(g.integers(16385, top + 1))
    rows = int(g.integers(1, 9))
    mis = bool(g.integers(0, 3) == 0)
    p = float(g.choice([0.0, 0.1, 0.3]))
    scale = float(g.uniform(0.05, 1.0))
    case(f"random long softmax {idx}: {rows}x{cols} {dtype} misaligned={mis} p={p}")
    cpu = synth.layer_inputs(rows, cols, dtype, seed=idx, x_std=3.0, names=("x", "dy"))
    x, dy = place(cpu["x"], mis), place(cpu["dy"], mis)
    mask = None
    if idx % 3 == 0:
        mk = synth.layer_inputs(1, cols, dtype, seed=idx + 50, x_std=2.0, names=("x",))["x"]
        mask = place(mk, mis)
    y, yd = mb.attn_softmax_fwd(x, scale, mask=mask, rows_per_mask=rows, p=p, seed=idx,
                                want_dropped=p > 0)
    dx = mb.attn_softmax_bwd(dy, y, scale, p=p, seed=idx)
    torch.cuda.synchronize()
    fmt = FMT[dtype]
    check_softmax_fwd(orc, x, y, yd, fmt, scale=scale, mask=mask, rows_per_mask=rows, p=p,
                      seed=idx, name="rnd.long_sm")
    check_softmax_bwd(orc, dy, y, dx, fmt, scale=scale, p=p, seed=idx, name="rnd.long_sm_bwd")


@pytest.mark.parametrize("idx", range(12))
def test_random_staged_and_two_pass_rows(orc, idx):
    """Rows the staged LayerNorm and the two-pass softmax / cross-entropy
    take by default, on seeded random widths, dtypes and alignments: the
    LayerNorm forward + backward (fp32 forwards from 6145 columns, every
    dtype past 16384, up to the backward's limit), the fused forward up to
    65536 columns, the rows past the register layouts up to 300000 columns
    (aligned cross-entropy rows of up to 131072 fp32 / 262144 16-bit classes
    are held in registers and LDS, the rest take the two-pass walk)."""
    g = np.random.default_rng([9001, idx])
    dtype = DTYPES[int(g.integers(0, 3))]
    mis = bool(g.integers(0, 3) == 0)
    fmt = FMT[dtype]
    seed = 5000 + idx
    kind = ("layernorm", "fused", "stream")[idx % 3]
    if kind == "layernorm":
        lo = 6145 if dtype == torch.float32 else 16385
        hi = 19968 if dtype == torch.float32 else 32768
        cols = int(g.integers(lo, hi + 1))
        rows = int(g.integers(1, 40))
        case(f"random staged LayerNorm {idx}: {rows}x{cols} {dtype} misaligned={mis}")
        d = {k: place(v, mis) for k, v in synth.layer_inputs(rows, cols, dtype, seed=seed).items()}
        y, mean, rstd = mb.ln_fwd(d["x"], d["gamma"], d["beta"], EPS)
        dx, dg, db = mb.ln_bwd(d["dy"], d["x"], d["gamma"], mean, rstd)
        torch.cuda.synchronize()
        check_fwd(orc, d["x"], d["gamma"], d["beta"], y, mean, rstd, fmt, name="rnd.staged")
        check_bwd(orc, d["dy"], d["x"], d["gamma"], mean, rstd, dx, dg, db, fmt,
                  name="rnd.staged_bwd")
    elif kind == "fused":
        cols = int(g.integers(16385, 65537))
        rows = int(g.integers(1, 12))
        case(f"random staged fused forward {idx}: {rows}x{cols} {dtype} misaligned={mis}")
        d = {k: place(v, mis) for k, v in synth.layer_inputs(rows, cols, dtype, seed=seed).items()}
        z, y, mean, rstd, mask = mb.bias_dropout_residual_ln_fwd(
            d["x"], d["bias"], d["residual"], d["gamma"], d["beta"], 0.2, seed, EPS,
            want_mask=True)
        torch.cuda.synchronize()
        check_fused(orc, d, 0.2, seed, z, y, mean, rstd, mask, fmt, name="rnd.staged_fused")
    else:
        cols = int(g.integers(65537, 300001))
        rows = int(g.integers(1, 6))
        case(f"random two-pass rows {idx}: {rows}x{cols} {dtype} misaligned={mis}")
        cpu = synth.layer_inputs(rows, cols, dtype, seed=seed, x_std=3.0, names=("x", "dy"))
        x, dy = place(cpu["x"], mis), place(cpu["dy"], mis)
        y, yd = mb.attn_softmax_fwd(x, 0.5, p=0.1, seed=seed, want_dropped=True)
        dx = mb.attn_softmax_bwd(dy, y, 0.5, p=0.1, seed=seed)
        lab = synth.class_labels(rows, cols, seed=seed, ignore_frac=0.1).to("cuda")
        loss, dl = mb.cross_entropy_fwd_bwd(x, lab, label_smoothing=0.1, grad_scale=1.0)
        torch.cuda.synchronize()
        check_softmax_fwd(orc, x, y, yd, fmt, scale=0.5, p=0.1, seed=seed, name="rnd.tp_sm")
        check_softmax_bwd(orc, dy, y, dx, fmt, scale=0.5, p=0.1, seed=seed, name="rnd.tp_sm_bwd")
        check_xent(orc, x, lab, cols, 0.1, 1.0, loss, dl, fmt, name="rnd.tp_xent")


@pytest.mark.parametrize("idx", range(10))
def test_random_rows_held_on_chip(orc, idx):
    """Rows past the register layouts that one workgroup still holds on chip
    and reads once, on seeded random widths (rows of whole 16-byte slots):
    the cross-entropy in registers and LDS (up to 131072 fp32 / 262144 16-bit
    classes), the softmax forward, with or without a mask row, and its
    backward, with or without dropout (up to 65536 fp32 / 131072 16-bit
    columns), causal or not."""
    g = np.random.default_rng([9100, idx])
    rows = int(g.integers(1, 40)) if idx % 3 else int(g.integers(257, 300))
    if idx % 2 == 0:
        dtype = DTYPES[int(g.integers(0, 3))]
        e = 4 if dtype == torch.float32 else 8
        lo, hi = (65537, 131072) if e == 4 else (163841, 262144)
        cols = int(g.integers(lo // e + 1, hi // e + 1)) * e
        ld = min(cols + e * int(g.integers(0, 3)), hi)   # padded rows, still on chip
        alpha = float(g.choice([0.0, 0.1, 0.5]))
        case(f"random on-chip cross-entropy {idx}: {rows}x{cols} ld {ld} {dtype} a={alpha}")
        x = synth.logits(rows, ld, dtype, seed=9100 + idx).to("cuda")
        lab = synth.class_labels(rows, cols, seed=9100 + idx, ignore_frac=0.1).to("cuda")
        loss, dl = mb.cross_entropy_fwd_bwd(x, lab, cols=cols, label_smoothing=alpha,
                                            grad_scale=1.0)
        torch.cuda.synchronize()
        sel = None if rows < 64 else [0, 1, 255, 256, rows - 1]
        check_xent(orc, x, lab, cols, alpha, 1.0, loss, dl, FMT[dtype], rows_sel=sel,
                   name="rnd.oc_xent")
    else:
        dtype = DTYPES[int(g.integers(0, 3))]
        e = 4 if dtype == torch.float32 else 8
        lo, hi = (32768, 65536) if e == 4 else (49152, 131072)
        cols = int(g.integers(lo // e + 1, hi // e + 1)) * e
        causal = bool(g.integers(0, 2))
        p = float(g.choice([0.0, 0.1, 0.3]))
        seed = int(g.integers(0, 2 ** 63)) * 2 + 1
        rpm = int(g.integers(1, 5)) if rows < 64 and g.integers(0, 2) else 0   # 0: no mask
        case(f"random on-chip softmax {idx}: {rows}x{cols} {dtype} causal={causal} "
             f"p={p} seed={seed} rows_per_mask={rpm}")
        cpu = synth.layer_inputs(rows, cols, dtype, seed=9100 + idx, x_std=3.0,
                                 names=("x", "dy"))
        x, dy = cpu["x"].to("cuda"), cpu["dy"].to("cuda")
        mask = None
        if rpm:
            mask = cpu["dy"][:(rows + rpm - 1) // rpm].to("cuda").clone()
            mask[:, ::7] = float("-inf")
        y, yd = mb.attn_softmax_fwd(x, 0.5, mask=mask, rows_per_mask=max(rpm, 1), causal=causal,
                                    p=p, seed=seed, want_dropped=p > 0)
        dx = mb.attn_softmax_bwd(dy, y, 0.5, causal=causal, p=p, seed=seed)
        torch.cuda.synchronize()
        fmt = FMT[dtype]
        if rows < 64:
            check_softmax_fwd(orc, x, y, yd, fmt, scale=0.5, mask=mask,
                              rows_per_mask=max(rpm, 1), causal=causal, p=p, seed=seed,
                              name="rnd.oc_sm")
            check_softmax_bwd(orc, dy, y, dx, fmt, scale=0.5, p=p, seed=seed,
                              name="rnd.oc_sm_bwd")
        else:
            # sampled rows (the oracle's causal query is a row's index in the
            # tensor it is given, so causal forwards are checked whole only)
            ids = [0, 1, 255, 256, rows - 1]
            i = torch.as_tensor(ids, device="cuda")
            if not causal:
                check_softmax_fwd(orc, x[i], y[i], None, fmt, scale=0.5, name="rnd.oc_sm")
            check_softmax_bwd(orc, dy[i], y[i], dx[i], fmt, scale=0.5, p=p, seed=seed,
                              name="rnd.oc_sm_bwd", row_ids=ids)
