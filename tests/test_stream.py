"""GPU parity of the two-pass paths for rows too long for the register
layouts (the attention softmax beyond 32768 fp32 / 65536 16-bit columns, the
cross-entropy beyond 65536 fp32 / 163840 16-bit classes), against the float64
oracle.  The module forces the two-pass path, so it is also checked at
narrower widths."""
import pytest
import torch

import memory_bound_row_amd as mb
from memory_bound_row_amd import synth
from gpu_helpers import FMT, case, check_softmax_bwd, check_softmax_fwd, check_xent, dev

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.float16, torch.bfloat16]


@pytest.fixture(autouse=True)
def two_pass():
    """Every call in this module takes the two-pass path, also at widths the
    register layouts hold (rows of 16385-65536 columns would otherwise go to
    the wide register kernels)."""
    mb.debug_force_two_pass(True)
    yield
    mb.debug_force_two_pass(False)


def softmax_run(orc, rows, cols, dtype, scale=0.5, causal=False, p=0.0, seed=3, mask_rows=0,
                name="stream.sm"):
    d = dev(synth.layer_inputs(rows, cols, dtype, seed=seed, x_std=3.0, names=("x", "dy")))
    mask = None
    rpm = 1
    if mask_rows:
        rpm = rows // mask_rows
        m = synth.layer_inputs(mask_rows, cols, dtype, seed=seed + 1, x_std=2.0,
                               names=("x",))["x"]
        mask = m.to("cuda")
    y, yd = mb.attn_softmax_fwd(d["x"], scale, mask=mask, rows_per_mask=rpm, causal=causal,
                                p=p, seed=seed, want_dropped=p > 0)
    dx = mb.attn_softmax_bwd(d["dy"], y, scale, causal=causal, p=p, seed=seed)
    torch.cuda.synchronize()
    check_softmax_fwd(orc, d["x"], y, yd, FMT[dtype], scale=scale, mask=mask,
                      rows_per_mask=rpm, causal=causal, p=p, seed=seed, name=name)
    check_softmax_bwd(orc, d["dy"], y, dx, FMT[dtype], scale=scale, p=p, seed=seed,
                      name=name + "_bwd")
    return y


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("cols", [16385, 20000, 65539, 200000])
def test_softmax_long_rows(orc, dtype, cols):
    rows = 24 if cols < 100000 else 8
    case(f"stream softmax {rows}x{cols} {dtype}")
    y = softmax_run(orc, rows, cols, dtype, p=0.1, name=f"stream.sm.{cols}")
    sums = y.float().sum(dim=1).cpu()
    assert torch.allclose(sums, torch.ones_like(sums), atol=2e-2)


def test_softmax_long_rows_mask_and_causal(orc):
    case("stream softmax 48x30000 bf16 mask + causal")
    softmax_run(orc, 48, 30000, torch.bfloat16, mask_rows=3, name="stream.sm.mask")
    # causal over rows of 30000 keys: row r sees keys 0..r (most chunks are
    # past the query and are written as zeros without being read)
    softmax_run(orc, 48, 30000, torch.bfloat16, causal=True, p=0.2, name="stream.sm.causal")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_softmax_long_rows_per_element(orc, dtype):
    case(f"stream softmax per-element path {dtype}")
    softmax_run(orc, 16, 20001, dtype, p=0.1, name="stream.sm.odd")   # rows not 16-byte aligned
    try:
        mb.debug_force_path(0, 0, scalar=True)
        softmax_run(orc, 16, 20000, dtype, p=0.1, name="stream.sm.scalar")
    finally:
        mb.debug_force_path(0)


# Columns per chunk of a row (1024 lanes x 4 16-byte slots without a mask, x 2
# with one); pass A keeps the first two chunks in LDS for pass B.
CHUNK = {torch.float32: 16384, torch.float16: 32768, torch.bfloat16: 32768}


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k,d", [(1, 0), (2, -1), (2, 0), (2, 1), (3, 0), (4, 1)])
def test_staged_chunk_boundaries(orc, dtype, k, d):
    # rows of k chunks (d columns more or fewer): all staged, the last slot of
    # the stage, one slot past it
    cols = k * CHUNK[dtype] + d
    case(f"stream softmax + cross-entropy {dtype} 6x{cols} ({k} chunks {d:+d})")
    softmax_run(orc, 6, cols, dtype, p=0.1, name=f"stream.sm.k{k}{d:+d}")
    xent_run(orc, 6, cols, cols, dtype, name=f"stream.xent.k{k}{d:+d}")


def test_causal_rows_across_the_stage(orc):
    # causal fp32 rows with a mask (chunks of 8192 columns): row r reads its
    # first r + 1 columns, so the rows below end in chunk 1, 2, 3 and 4, and
    # each equals the softmax of its prefix, zeros after it
    rows = cols = 24600
    case(f"stream causal softmax fp32 {rows}x{cols} with a mask, sampled rows")
    g = torch.Generator(device="cuda").manual_seed(21)
    x = torch.randn((rows, cols), device="cuda", generator=g) * 3.0
    mask = torch.randn((1, cols), device="cuda", generator=g)
    dy = torch.randn((rows, cols), device="cuda", generator=g)
    y, _ = mb.attn_softmax_fwd(x, 0.5, mask=mask, rows_per_mask=rows, causal=True)
    dx = mb.attn_softmax_bwd(dy, y, 0.5, causal=True)
    torch.cuda.synchronize()
    for r in (0, 8191, 8192, 16383, 16384, 24575, 24576, rows - 1):
        n = r + 1
        fmt = FMT[torch.float32]
        check_softmax_fwd(orc, x[r:r + 1, :n], y[r:r + 1, :n], None, fmt, scale=0.5,
                          mask=mask[:, :n], name=f"stream.causal.r{r}")
        check_softmax_bwd(orc, dy[r:r + 1, :n], y[r:r + 1, :n], dx[r:r + 1, :n], fmt,
                          scale=0.5, name=f"stream.causal.r{r}.bwd")
        assert torch.all(y[r, n:] == 0) and torch.all(dx[r, n:] == 0)


def xent_run(orc, rows, cols, ld, dtype, seed=5, name="stream.xent"):
    x = synth.logits(rows, ld, dtype, seed=seed).to("cuda")
    lab = synth.class_labels(rows, cols, seed=seed, ignore_frac=0.1).to("cuda")
    loss, dx = mb.cross_entropy_fwd_bwd(x, lab, cols=cols, label_smoothing=0.1,
                                        grad_scale=1.0 / rows)
    torch.cuda.synchronize()
    check_xent(orc, x, lab, cols, 0.1, 1.0 / rows, loss, dx, FMT[dtype], name=name)
    return x, lab, loss, dx


@pytest.mark.parametrize("dtype,cols,ld", [
    (torch.float32, 65537, 65540), (torch.float32, 100000, 100000),
    (torch.bfloat16, 131073, 131080), (torch.bfloat16, 256000, 256000),
    (torch.float16, 262147, 262152)])
def test_xent_long_vocabularies(orc, dtype, cols, ld):
    # 256000: the vocabulary of Gemma-sized models
    case(f"stream cross-entropy 24x{cols} ld {ld} {dtype}")
    xent_run(orc, 24, cols, ld, dtype, name=f"stream.xent.{cols}")


def test_xent_long_rows_per_element_and_invalid_label(orc):
    case("stream cross-entropy per-element path, invalid label")
    x, lab, loss, dx = xent_run(orc, 12, 150001, 150001, torch.bfloat16, name="stream.xent.odd")
    lab2 = lab.clone()
    lab2[2] = 150001
    loss2, dx2 = mb.cross_entropy_fwd_bwd(x, lab2, cols=150001)
    torch.cuda.synchronize()
    assert torch.isnan(loss2[2]) and torch.isnan(dx2[2]).all()


def test_widest_rows(orc):
    # LN_MAX_COLS_STREAM columns: the widest row the library takes (the next
    # width up is rejected on the host, tests/test_abi.py)
    cols = 1 << 24
    case(f"stream softmax and cross-entropy 2x{cols} bf16")
    softmax_run(orc, 2, cols, torch.bfloat16, p=0.1, name="stream.sm.widest")
    xent_run(orc, 2, cols, cols, torch.bfloat16, name="stream.xent.widest")


def test_stream_in_a_graph():
    case("stream paths under graph capture")
    d = dev(synth.layer_inputs(8, 40000, torch.bfloat16, seed=9, x_std=3.0, names=("x", "dy")))
    y, yd, dxs = (torch.empty_like(d["x"]) for _ in range(3))
    x = synth.logits(8, 140000, torch.bfloat16, seed=9).to("cuda")
    lab = synth.class_labels(8, 140000, seed=9).to("cuda")
    loss = torch.empty(8, dtype=torch.float32, device="cuda")
    dl = torch.empty_like(x)

    def run():
        mb.attn_softmax_fwd(d["x"], 0.25, p=0.1, seed=1, y=y, y_dropped=yd)
        mb.attn_softmax_bwd(d["dy"], y, 0.25, p=0.1, seed=1, dx=dxs)
        mb.cross_entropy_fwd_bwd(x, lab, label_smoothing=0.1, grad_scale=0.125, loss=loss,
                                 dlogits=dl)

    run()
    torch.cuda.synchronize()
    outs = [y, yd, dxs, loss, dl]
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for k in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            a = o.view(torch.int16) if o.dtype == torch.bfloat16 else o
            b = r.view(torch.int16) if r.dtype == torch.bfloat16 else r
            assert torch.equal(a, b), f"replay {k} differs"
