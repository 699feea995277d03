"""Stream ordering and host-thread safety: the library enqueues on the
caller's stream only (results on side streams equal those on the default
stream), and concurrent calls from several host threads, each on its own
stream, give the same bits as the same calls made one after another (the
calls release the interpreter lock, so they do run concurrently)."""
import threading

import pytest
import torch

import memory_bound_row_amd as mb
from memory_bound_row_amd import synth
from gpu_helpers import EPS, case, dev

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t


def step(d, p=0.1, seed=3):
    z, y, mean, rstd, _ = mb.bias_dropout_residual_ln_fwd(
        d["x"], d["bias"], d["residual"], d["gamma"], d["beta"], p, seed, EPS)
    dx, dg, db = mb.ln_bwd(d["dy"], z, d["gamma"], mean, rstd)
    sm, _ = mb.attn_softmax_fwd(d["x"], 0.5, causal=True)
    loss, dl = mb.cross_entropy_fwd_bwd(d["x"], d["labels"], label_smoothing=0.1)
    return [z, y, mean, rstd, dx, dg, db, sm, loss, dl]


def inputs(seed, rows=1024, cols=1024):
    d = dev(synth.layer_inputs(rows, cols, torch.bfloat16, seed=seed))
    d["labels"] = synth.class_labels(rows, cols, seed=seed).to("cuda")
    return d


def test_side_streams_match_the_default_stream():
    case("side streams vs default stream")
    d = inputs(1)
    ref = step(d)
    torch.cuda.synchronize()
    for _ in range(3):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            out = step(d)
        s.synchronize()
        for a, b in zip(out, ref):
            assert torch.equal(bits(a), bits(b))


def test_concurrent_host_threads():
    case("4 host threads x 20 steps, one stream each")
    sets = [inputs(10 + k) for k in range(4)]
    refs = []
    for d in sets:
        refs.append([t.clone() for t in step(d)])
    torch.cuda.synchronize()
    errors = []

    def worker(k):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(20):
                    out = step(sets[k])
                s.synchronize()
            for a, b in zip(out, refs[k]):
                if not torch.equal(bits(a), bits(b)):
                    errors.append(f"thread {k}: result differs")
        except Exception as e:   # report in the main thread
            errors.append(f"thread {k}: {e!r}")

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors
