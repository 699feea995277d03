"""Every entry point captured into a HIP graph: replays, separated by eager
work on the same buffers and synchronisations, give the eager result bit for
bit (the calls enqueue only kernels: no memsets, copies or allocations)."""
import pytest
import torch

import memory_bound_row_amd as mb
from memory_bound_row_amd import synth
from gpu_helpers import case, dev

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t


def check_replays(run, outputs, inputs_reset=None, replays=4):
    """run() enqueues the call into preallocated outputs; compare each graph
    replay with the eager result."""
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outputs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for k in range(replays):
        for o in outputs:
            o.fill_(float("nan") if o.is_floating_point() else 0)   # eager work in between
        if inputs_reset:
            inputs_reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outputs, ref):
            assert torch.equal(bits(o), bits(r)), f"replay {k} differs"


def test_layernorm_step_in_a_graph():
    case("graph: fused forward, backward with partials, fold")
    R, C = 1000, 1280
    d = dev(synth.layer_inputs(R, C, torch.bfloat16, seed=3))
    z, y = torch.empty_like(d["x"]), torch.empty_like(d["x"])
    mean = torch.empty(R, dtype=torch.float32, device="cuda")
    rstd = torch.empty_like(mean)
    dx = torch.empty_like(d["x"])
    ws = mb.workspace(R, C, "cuda")
    dg = torch.empty(C, dtype=torch.float32, device="cuda")
    db = torch.empty_like(dg)

    def run():
        mb.bias_dropout_residual_ln_fwd(d["x"], d["bias"], d["residual"], d["gamma"], d["beta"],
                                        0.1, 5, 1e-5, residual_out=z, y=y, mean=mean, rstd=rstd)
        mb.ln_bwd_dx(d["dy"], z, d["gamma"], mean, rstd, dx=dx, workspace=ws)
        mb.ln_bwd_dgamma_dbeta(ws, R, C, torch.bfloat16, partials_ready=True, dgamma=dg,
                               dbeta=db)

    check_replays(run, [z, y, mean, rstd, dx, dg, db])


def test_prologue_backward_in_a_graph():
    case("graph: prologue backward")
    R, C = 600, 1024
    d = dev(synth.layer_inputs(R, C, torch.float16, seed=4))
    z, _, mean, rstd, _ = mb.bias_dropout_residual_ln_fwd(
        d["x"], d["bias"], d["residual"], d["gamma"], d["beta"], 0.2, 9, 1e-5)
    outs = [torch.empty_like(z), torch.empty_like(z)] + \
        [torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(3)]
    ws = mb.dropout_workspace(R, C, "cuda")

    def run():
        mb.bias_dropout_residual_ln_bwd(d["dy"], z, d["gamma"], mean, rstd, 0.2, 9,
                                        dz_extra=d["residual"], dresidual=outs[0], dx=outs[1],
                                        dgamma=outs[2], dbeta=outs[3], dbias=outs[4],
                                        workspace=ws)

    check_replays(run, outs)


def test_softmax_in_a_graph():
    case("graph: attention softmax forward and backward")
    d = dev(synth.layer_inputs(4 * 256, 256, torch.bfloat16, seed=5, x_std=3.0,
                               names=("x", "dy")))
    y, yd, dx = (torch.empty_like(d["x"]) for _ in range(3))

    def run():
        mb.attn_softmax_fwd(d["x"], 0.125, causal=True, p=0.1, seed=2, y=y, y_dropped=yd)
        mb.attn_softmax_bwd(d["dy"], y, 0.125, causal=True, p=0.1, seed=2, dx=dx)

    check_replays(run, [y, yd, dx])


def test_long_softmax_rows_in_a_graph():
    case("graph: attention softmax over 40000-key bf16 rows (lean register layouts)")
    d = dev(synth.layer_inputs(12, 40000, torch.bfloat16, seed=6, x_std=3.0,
                               names=("x", "dy")))
    mk = dev(synth.layer_inputs(3, 40000, torch.bfloat16, seed=7, names=("x",)))["x"]
    y, yd, dx = (torch.empty_like(d["x"]) for _ in range(3))

    def run():
        mb.attn_softmax_fwd(d["x"], 0.25, mask=mk, rows_per_mask=4, p=0.1, seed=3, y=y,
                            y_dropped=yd)
        mb.attn_softmax_bwd(d["dy"], y, 0.25, p=0.1, seed=3, dx=dx)

    check_replays(run, [y, yd, dx])


def test_rmsnorm_in_a_graph():
    case("graph: add + RMSNorm forward and backward")
    R, C = 512, 4096
    d = dev(synth.layer_inputs(R, C, torch.bfloat16, seed=6,
                               names=("x", "residual", "gamma", "dy")))
    z, y, dz = (torch.empty_like(d["x"]) for _ in range(3))
    rstd = torch.empty(R, dtype=torch.float32, device="cuda")
    dg = torch.empty(C, dtype=torch.float32, device="cuda")
    ws = mb.rmsnorm_workspace(R, C, "cuda")

    def run():
        mb.add_rmsnorm_fwd(d["x"], d["gamma"], 1e-6, residual=d["residual"], residual_out=z,
                           y=y, rstd=rstd)
        mb.add_rmsnorm_bwd(d["dy"], z, d["gamma"], rstd, dz_extra=d["dy"], dz=dz, dgamma=dg,
                           workspace=ws)

    check_replays(run, [z, y, rstd, dz, dg])


@pytest.mark.parametrize("R,V,LD,dtype", [
    (256, 50257, 50304, torch.bfloat16),    # rows in registers
    (520, 192000, 192000, torch.bfloat16),  # rows held in registers and LDS, 2-3 per workgroup
    (300, 100000, 100000, torch.float32),   # the same, fp32
])
def test_cross_entropy_in_a_graph(R, V, LD, dtype):
    case(f"graph: cross-entropy {R}x{V} {dtype}, gradient over the logits")
    x0 = synth.logits(R, LD, dtype, seed=7).to("cuda")
    lab = synth.class_labels(R, V, seed=7).to("cuda")
    x = x0.clone()
    loss = torch.empty(R, dtype=torch.float32, device="cuda")

    def reset():
        x.copy_(x0)

    def run():
        mb.cross_entropy_fwd_bwd(x, lab, cols=V, label_smoothing=0.1, grad_scale=1.0 / R,
                                 loss=loss, dlogits=x)

    # the call overwrites its input: restore the logits before every run
    reset()
    run()
    torch.cuda.synchronize()
    ref = [loss.clone(), x.clone()]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        reset()
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for k in range(4):
        loss.fill_(float("nan"))
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(loss, ref[0]), f"replay {k}: loss differs"
        assert torch.equal(bits(x), bits(ref[1])), f"replay {k}: gradient differs"


def test_training_step_split_stages_in_a_graph():
    # the benchmarked step: fused forward, prologue backward stage 1, fold
    case("graph: fused forward, prologue backward stages, fold")
    R, C = 1000, 1280
    d = dev(synth.layer_inputs(R, C, torch.bfloat16, seed=4))
    ez = dev(synth.layer_inputs(R, C, torch.bfloat16, seed=5, names=("dy",)))["dy"]
    z, y = torch.empty_like(d["x"]), torch.empty_like(d["x"])
    mean = torch.empty(R, dtype=torch.float32, device="cuda")
    rstd = torch.empty_like(mean)
    dres, dxin = torch.empty_like(d["x"]), torch.empty_like(d["x"])
    ws = mb.dropout_workspace(R, C, "cuda")
    pg = [torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(3)]

    def run():
        mb.bias_dropout_residual_ln_fwd(d["x"], d["bias"], d["residual"], d["gamma"], d["beta"],
                                        0.1, 5, 1e-5, residual_out=z, y=y, mean=mean, rstd=rstd)
        mb.bias_dropout_residual_ln_bwd_dx(d["dy"], z, d["gamma"], mean, rstd, 0.1, 5,
                                           workspace=ws, dz_extra=ez, dresidual=dres, dx=dxin)
        mb.bias_dropout_residual_ln_bwd_fold(ws, R, C, dgamma=pg[0], dbeta=pg[1], dbias=pg[2])

    check_replays(run, [z, y, mean, rstd, dres, dxin] + pg)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_staged_rows_in_a_graph(dtype):
    case(f"graph: LDS-staged forward, fused forward and backward {dtype}")
    R, C = 40, 20000 if dtype == torch.bfloat16 else 19000
    d = dev(synth.layer_inputs(R, C, dtype, seed=6))
    y, z, y2 = (torch.empty_like(d["x"]) for _ in range(3))
    mean = torch.empty(R, dtype=torch.float32, device="cuda")
    rstd, mean2, rstd2 = (torch.empty_like(mean) for _ in range(3))
    dx = torch.empty_like(d["x"])
    ws = mb.workspace(R, C, "cuda")
    dg = torch.empty(C, dtype=torch.float32, device="cuda")
    db = torch.empty_like(dg)

    def run():
        mb.ln_fwd(d["x"], d["gamma"], d["beta"], 1e-5, y=y, mean=mean, rstd=rstd)
        mb.bias_dropout_residual_ln_fwd(d["x"], d["bias"], d["residual"], d["gamma"], d["beta"],
                                        0.2, 8, 1e-5, residual_out=z, y=y2, mean=mean2,
                                        rstd=rstd2)
        mb.ln_bwd(d["dy"], d["x"], d["gamma"], mean, rstd, dx=dx, workspace_buf=ws, dgamma=dg,
                  dbeta=db)

    check_replays(run, [y, z, y2, mean, rstd, mean2, rstd2, dx, dg, db])


def test_noalloc_backward_in_a_graph():
    case("graph: ln_bwd_noalloc")
    R, C = 1000, 1280
    d = dev(synth.layer_inputs(R, C, torch.bfloat16, seed=7))
    _, mean, rstd = mb.ln_fwd(d["x"], d["gamma"], d["beta"], 1e-5)
    dx = torch.empty_like(d["x"])
    dg = torch.empty(C, dtype=torch.float32, device="cuda")
    db = torch.empty_like(dg)

    def run():
        mb.ln_bwd_noalloc(d["dy"], d["x"], d["gamma"], mean, rstd, dx=dx, dgamma=dg, dbeta=db)

    check_replays(run, [dx, dg, db])
