#!/usr/bin/env python3
"""Benchmark of the fused LayerNorm hot path on one MI355X.

One step = one training pass of the path over one batch of synthetic rows,
at 8192 x 1280 bf16 storage with float32 arithmetic:
  bias_dropout_residual_ln_fwd (bias add, dropout p, residual add, LayerNorm;
  z and y written, mean/rstd saved)  ->  bias_dropout_residual_ln_bwd_dx (the
  LayerNorm dx from two row sums, the gradient from the residual stream added,
  the dropout/residual backward with the mask regenerated from the seed, and
  the stage-1 column partials of dgamma, dbeta, dbias)  ->
  bias_dropout_residual_ln_bwd_fold (the fixed-order fold of the partials).
The same line reports the plain LayerNorm step the hot-path scope table
defines as the metric case (ln_fwd -> ln_bwd_dx with partials -> fold) and
the fused forward followed by the plain LayerNorm backward.

The timed region replays K steps captured in one HIP graph, on inputs that
are already resident in device memory.  K steps rotate over buffer sets whose
total exceeds the 256 MB Infinity Cache several times, and each step's
backward reads a set written half a rotation earlier, so every byte comes
from HBM as it would in training (the backward of a layer runs long after
its forward).  `value` is algorithmic bytes (what the method must move) per
second over the whole step.  The `roofline` object reports the dominant
kernel alone, timed with HIP events on the stream it runs on; the CPU
baseline times the float64 oracle on the host.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
ROWS, COLS, P_DROP, EPS, SEED = 8192, 1280, 0.1, 1e-5, 0
WORKLOAD = ("training step of the fused LayerNorm, 8192x1280 bf16 storage: "
            "bias+dropout(p=0.1)+residual+LayerNorm forward, then its backward (LayerNorm "
            "dx and dgamma/dbeta, residual-stream gradient added, dropout/residual/bias "
            "backward with dbias)")


def algorithmic_bytes(rows: int, cols: int, s: int) -> dict:
    """Bytes each call of the step must move at minimum: every [rows, cols]
    tensor read or written once, gamma/beta/bias once, mean/rstd and the
    parameter gradients as float32 (the column partials are not counted)."""
    fwd = 4 * rows * cols * s + 3 * cols * s + 8 * rows        # x, res -> z, y
    bwd = 5 * rows * cols * s + cols * s + 8 * rows            # dy, dz_extra, z -> dres, dx
    fold = 12 * cols                                           # dgamma, dbeta, dbias
    return {"fused_fwd": fwd, "prologue_bwd": bwd, "fold": fold,
            "step": fwd + bwd + fold}


def ln_bwd_bytes(rows: int, cols: int, s: int) -> int:
    """The LayerNorm backward (dx, dgamma, dbeta): dy, x read, dx written."""
    return 3 * rows * cols * s + cols * s + 8 * rows + 8 * cols


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=8,
                    help="rotating buffer sets (8 x 126 MB defeats the 256 MB cache)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline (0 disables it)")
    ap.add_argument("--warm-cache", action="store_true",
                    help="one buffer set, backward on the forward's fresh z (cache-resident)")
    ap.add_argument("--configs", action="store_true",
                    help="instead of the step, measure the other workloads (decode-shaped "
                         "launch cost, 64x768 fp32, 16384x1024 bf16 backward, wide/ragged "
                         "rows) and print one JSON line each")
    ap.add_argument("--no-cpp-launch", action="store_true",
                    help="with --configs: skip the C++ launch-loop child process (for runs "
                         "under a profiler, whose preloaded library the child inherits)")
    ap.add_argument("--counter-sample", action="store_true",
                    help="launch the other operators' kernels three times each at their "
                         "workloads (prologue backward, attention softmax, add + RMSNorm, "
                         "cross-entropy, and the two-pass paths) and exit: a short program "
                         "for hardware-counter runs")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "this benchmark into profiles/traffic.json and exit")
    return ap.parse_args()


# Sources the step's kernels are compiled from (forward, backward, fold, their
# shared device code) and launched by (argument checks, layout choice, grid).
STEP_SOURCES = ("ln_api.cpp", "ln_bwd.hip", "ln_device.hpp", "ln_fold.hip", "ln_fwd.hip",
                "ln_launch.hpp")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "memory_bound_row_amd", "csrc")
    for name in STEP_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, src_hash: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(kernel)
    if not k or k.get("source_hash") != src_hash:
        return None
    return k.get("hbm_bytes_per_launch")


COPY_BYTES = 256 * 1024 * 1024   # calibration copy: 256 MiB read, 256 MiB written


def _read_counters(path: str) -> dict:
    """rocprofv3 counter_collection.csv -> {kernel name: [values per dispatch]}."""
    import csv
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name", "")
            try:
                val = float(row.get("Counter_Value", "nan"))
            except ValueError:
                continue
            out.setdefault(name, []).append(val)
    return out


BWD_MODES = {"0": "dx", "1": "dx+partials", "2": "partials", "3": "prologue", "4": "rms"}


def kernel_short_name(name: str) -> str:
    """A library kernel's demangled name -> the short name used in reports."""
    base = name.split("(")[0].replace("void ", "").replace("mbrow::", "")
    if base.startswith("ln_fwd_kernel"):
        return "ln_fwd_kernel(fused)" if base.rstrip(">").endswith("true") else "ln_fwd_kernel"
    if base.startswith("ln_bwd_kernel"):
        mode = base.rstrip(">").split(",")[-1].strip()
        return f"ln_bwd_kernel({BWD_MODES.get(mode, mode)})"
    return base.split("<")[0]


def pmc_summary(fetch_csv: str, write_csv: str) -> None:
    """HBM bytes per launch of each library kernel from FETCH_SIZE/WRITE_SIZE
    (KiB per dispatch), scaled so that the calibration copy of COPY_BYTES reads
    and writes exactly COPY_BYTES."""
    fetch, write = _read_counters(fetch_csv), _read_counters(write_csv)

    def copy_kib(d):
        # the calibration copy: the largest one-source, one-destination stream
        best = 0.0
        for name, vals in d.items():
            if "hbm_stream_kernel<1, 1>" in name:
                best = max(best, max(vals))
        return best
    fcopy, wcopy = copy_kib(fetch), copy_kib(write)
    if fcopy <= 0 or wcopy <= 0:
        raise SystemExit("no calibration copy kernel found in the counter files")
    fscale, wscale = COPY_BYTES / (fcopy * 1024), COPY_BYTES / (wcopy * 1024)
    src_hash = kernel_source_hash()
    kernels = {}
    for name in fetch:
        if "mbrow" not in name:
            continue
        f_kib = sum(fetch[name]) / len(fetch[name])
        w_kib = sum(write.get(name, [0.0])) / max(1, len(write.get(name, [0.0])))
        short = kernel_short_name(name)
        kernels[short] = {
            "kernel_name": name,
            "fetch_bytes_per_launch": round(f_kib * 1024 * fscale),
            "write_bytes_per_launch": round(w_kib * 1024 * wscale),
            "hbm_bytes_per_launch": round(f_kib * 1024 * fscale + w_kib * 1024 * wscale),
            "dispatches": len(fetch[name]),
            "source_hash": src_hash,
        }
    rec = {"copy_calibration": {"bytes": COPY_BYTES, "fetch_kib": fcopy, "write_kib": wcopy,
                                "fetch_scale": fscale, "write_scale": wscale},
           "kernels": kernels}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def capture(fn, n):
    """HIP graph of fn(0) .. fn(n-1) captured on a side stream."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)                                      # warm the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    return g


def timed(g, n):
    """Milliseconds per item of one replay of graph g holding n items
    (after one untimed replay), between HIP events."""
    import torch
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / n


def step_distribution(g, n, reps):
    """Microseconds per step over `reps` further replays of the n-step graph
    g, each between its own pair of HIP events: p10 / median / p90 of the
    per-replay averages."""
    import torch
    t = sorted(timed(g, n) * 1e3 for _ in range(reps))

    def q(f):
        return round(t[min(reps - 1, int(f * reps))], 2)
    return {"p10": q(0.1), "median": q(0.5), "p90": q(0.9), "replays": reps,
            "steps_per_replay": n}


def stream_rates(cases, S, dev, K):
    """Attainable bandwidth of each kernel's mix of reads and writes: the
    library's streaming reference (`hbm_stream`) reading `nsrc` and writing
    `ndst` tensors that together hold `nbytes`, on incompressible data,
    rotated over S buffer sets like the step, timed as a K-launch graph.
    cases: {name: (nsrc, ndst, nbytes)} -> {name: (GB/s, microseconds)}."""
    import torch
    import memory_bound_row_amd as mb_lib
    out = {}
    g = torch.Generator(device=dev).manual_seed(7)
    for name, (nsrc, ndst, nbytes) in cases.items():
        n = (nbytes // (nsrc + ndst)) // 16 * 4        # int32 elements per tensor
        sets = [[torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int32, device=dev,
                               generator=g) for _ in range(nsrc + ndst)] for _ in range(S)]
        ms = timed(capture(lambda i: mb_lib.hbm_stream(sets[i % S][:nsrc],
                                                       sets[i % S][nsrc:]), K), K)
        moved = 4 * n * (nsrc + ndst)
        out[name] = (round(moved / (ms * 1e-3) / 1e9, 1), round(ms * 1e3 * nbytes / moved, 3))
        del sets
    return out


def host_threads() -> int:
    """Threads the host leg may use: the process's CPU affinity, capped by
    OMP_NUM_THREADS when that is set."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def plain_bytes(rows: int, cols: int, s: int) -> dict:
    """Algorithmic bytes of ln_fwd and of the backward (dx, dgamma, dbeta)."""
    fwd = 2 * rows * cols * s + 2 * cols * s + 8 * rows
    bwd = 3 * rows * cols * s + cols * s + 8 * rows + 8 * cols
    return {"fwd": fwd, "bwd": bwd, "step": fwd + bwd}


def _oracle_step(orc, d, row0, rows):
    """The oracle's whole step over rows [row0, row0 + rows) of the workload:
    the fused forward, then its backward; returns the column sums (dgamma,
    dbeta, dbias) of that range."""
    import numpy as np
    sl = slice(row0, row0 + rows)
    keep = orc.dropout_keep_rows(SEED, P_DROP, row0, rows, COLS)
    z = orc.round_to(orc.bias_dropout_residual(d["x"][sl], d["bias"], d["residual"][sl], keep,
                                               P_DROP), "bf16")
    _, mu, rs = orc.ln_fwd(z, d["gamma"], d["beta"], EPS)
    mu, rs = np.float64(np.float32(mu)), np.float64(np.float32(rs))
    dz = orc.ln_bwd_dx(d["dy"][sl], z, d["gamma"], mu, rs) + d["ez"][sl]
    _, dbias, _ = orc.dropout_residual_bwd(dz, keep, P_DROP)
    dg, db, _, _ = orc.ln_bwd_params(d["dy"][sl], z, mu, rs)
    return dg, db, dbias


def cpu_baseline(inp_cpu, target_s: float):
    """The float64 oracle, as it stands, on the host: the same step on the
    same stored values, single-threaded (the reported baseline), and for
    context the same calls on row ranges split over the host's threads (the
    oracle's C routines release the interpreter lock), their column sums
    added in range order."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle as orc
    from memory_bound_row_amd import synth

    d = {k: synth.as_f64(v) for k, v in inp_cpu.items()}
    b = algorithmic_bytes(ROWS, COLS, 2)["step"]

    reps, t_total = 0, 0.0
    while reps == 0 or (t_total < target_s and reps < 50):
        t0 = time.perf_counter()
        _oracle_step(orc, d, 0, ROWS)
        t_total += time.perf_counter() - t0
        reps += 1
    out = {"value": round(b * reps / t_total / 1e9, 3), "unit": "GB/s", "cores": 1,
           "kind": "oracle",
           "sample": f"{reps} full step(s) of the workload ({ROWS}x{COLS}, float64 oracle "
                     f"on bf16-stored inputs), {t_total:.1f} s single-threaded",
           "rows_per_s": round(ROWS * reps / t_total, 1), "cpu_model": cpu_model()}

    nt = host_threads()
    if nt > 1:
        bounds = [(ROWS * i // nt, ROWS * (i + 1) // nt) for i in range(nt)]
        with ThreadPoolExecutor(nt) as pool:
            reps_p, t_par = 0, 0.0
            while reps_p == 0 or (t_par < target_s / 2 and reps_p < 50):
                t0 = time.perf_counter()
                parts = list(pool.map(lambda r: _oracle_step(orc, d, r[0], r[1] - r[0]), bounds))
                sums = list(parts[0])
                for part in parts[1:]:
                    sums = [a + b for a, b in zip(sums, part)]
                t_par += time.perf_counter() - t0
                reps_p += 1
        out["all_threads"] = {"value": round(b * reps_p / t_par / 1e9, 3), "unit": "GB/s",
                              "cores": nt,
                              "sample": f"{reps_p} full step(s), rows split over {nt} threads, "
                                        f"{t_par:.1f} s"}
    return out


def oracle_rate(prep, work, row_bytes, max_rows, target_s=0.5):
    """CPU baseline of a workload: the float64 oracle's rate on a sample of
    its rows.  prep(n) builds the oracle's inputs for the first n rows
    (untimed); work(args) runs the oracle's computation of the workload on
    them (timed, single thread).  n doubles until one run takes target_s or
    reaches max_rows."""
    n = 1
    while True:
        args = prep(n)
        t0 = time.perf_counter()
        work(args)
        dt = time.perf_counter() - t0
        if dt >= target_s or n >= max_rows:
            return {"value": round(n * row_bytes / dt / 1e9, 3), "unit": "GB/s",
                    "cores": 1, "kind": "oracle",
                    "sample": f"the first {n} rows, {dt:.2f} s single-threaded"}
        n = min(max_rows, n * 2)


def counter_sample() -> None:
    """Three launches of each of the other operators' kernels at their
    workloads, nothing timed (for rocprofv3 --pmc): the prologue backward
    (8192 x 1280 bf16, dz_extra given), the attention softmax forward (y and
    dropped y) and backward (8 x 16 x 512 x 512 fp16, p = 0.1), add + RMSNorm
    forward and backward (2048 x 4096 bf16), the cross-entropy (8192 x 50257
    bf16, rows of 50304), the cross-entropy over 2048 x 256000 bf16 (rows held
    in registers and LDS, then forced onto the two-pass path), and the
    softmax over 2048 x 131072 fp16 (the forward in registers, without and
    with the dropped copy, and the backward without and with dropout,
    p = 0.1, held on chip; the forward with a mask row shared by 16 rows,
    held on chip; then all five forced onto the two-pass path)."""
    import torch
    import memory_bound_row_amd as mb
    from memory_bound_row_amd import synth
    dev = torch.device("cuda", 0)
    bf, hf = torch.bfloat16, torch.float16

    d = {k: v.to(dev) for k, v in synth.layer_inputs(ROWS, COLS, bf, seed=SEED).items()}
    ez = synth.layer_inputs(ROWS, COLS, bf, seed=SEED + 1, names=("dy",))["dy"].to(dev)
    z, _, mean, rstd, _ = mb.bias_dropout_residual_ln_fwd(d["x"], d["bias"], d["residual"],
                                                          d["gamma"], d["beta"], P_DROP, SEED,
                                                          EPS)
    for _ in range(3):
        mb.bias_dropout_residual_ln_bwd(d["dy"], z, d["gamma"], mean, rstd, P_DROP, SEED,
                                        dz_extra=ez)
    del d, ez, z
    d = {k: v.to(dev) for k, v in synth.layer_inputs(8 * 16 * 512, 512, hf, seed=SEED,
                                                     x_std=3.0, names=("x", "dy")).items()}
    for _ in range(3):
        y, _ = mb.attn_softmax_fwd(d["x"], 0.125, p=0.1, seed=SEED, want_dropped=True)
        mb.attn_softmax_bwd(d["dy"], y, 0.125, p=0.1, seed=SEED)
    del d, y
    d = {k: v.to(dev) for k, v in synth.layer_inputs(
        2048, 4096, bf, seed=SEED, names=("x", "residual", "gamma", "dy")).items()}
    for _ in range(3):
        z, _, rs = mb.add_rmsnorm_fwd(d["x"], d["gamma"], 1e-6, residual=d["residual"])
        mb.add_rmsnorm_bwd(d["dy"], z, d["gamma"], rs, dz_extra=d["residual"])
    del d, z
    x = synth.logits(8192, 50304, bf, seed=SEED).to(dev)
    lab = synth.class_labels(8192, 50257, seed=SEED).to(dev)
    for _ in range(3):
        mb.cross_entropy_fwd_bwd(x, lab, cols=50257, label_smoothing=0.1, grad_scale=1.0 / 8192)
    torch.cuda.synchronize()
    del x

    x = synth.logits(2048, 256000, torch.bfloat16, seed=SEED).to(dev)
    lab = synth.class_labels(2048, 256000, seed=SEED).to(dev)
    loss = torch.empty(2048, dtype=torch.float32, device=dev)
    dx = torch.empty_like(x)
    for two_pass in (False, True):
        mb.debug_force_two_pass(two_pass)
        for _ in range(3):
            mb.cross_entropy_fwd_bwd(x, lab, label_smoothing=0.1, grad_scale=1.0, loss=loss,
                                     dlogits=dx)
        torch.cuda.synchronize()
    mb.debug_force_two_pass(False)
    del x, dx
    d = synth.layer_inputs(2048, 131072, torch.float16, seed=SEED, x_std=3.0, names=("x", "dy"))
    s, dy = d["x"].to(dev), d["dy"].to(dev)
    y, ds, yd = torch.empty_like(s), torch.empty_like(s), torch.empty_like(s)
    mask = synth.layer_inputs(2048 // 16, 131072, torch.float16, seed=SEED + 1,
                              names=("dy",))["dy"].to(dev)
    for two_pass in (False, True):
        mb.debug_force_two_pass(two_pass)
        for _ in range(3):
            mb.attn_softmax_fwd(s, 0.125, y=y)
            mb.attn_softmax_bwd(dy, y, 0.125, dx=ds)
        for _ in range(3):
            mb.attn_softmax_fwd(s, 0.125, p=0.1, seed=SEED, y=y, y_dropped=yd)
            mb.attn_softmax_bwd(dy, y, 0.125, p=0.1, seed=SEED, dx=ds)
        for _ in range(3):
            mb.attn_softmax_fwd(s, 0.125, mask=mask, rows_per_mask=16, y=y)
        torch.cuda.synchronize()
    mb.debug_force_two_pass(False)
    print("counter sample: done", flush=True)


def configs_report(cpp_launch: bool = True) -> None:
    """Figures of the workloads other than the step, one JSON line each:
      * decode-shaped fp16 ln_fwd, 1 and 8 rows x 4096, 10^4 back-to-back
        calls without saved statistics: microseconds per call from a C++
        loop (the `launch_bench` tool, run first as a child process), a
        Python loop through the binding, and a HIP graph of the calls;
      * the fused backward of the whole layer (bias_dropout_residual_ln_bwd)
        at 8192x1280 bf16, alone and after the fused forward;
      * the attention softmax forward and backward at 8x16x512x512 (dropout)
        and 2x16x256x256 (causal), fp16;
      * fused residual add + RMSNorm forward and backward at 2048x4096 bf16
        (one layer of a 2048-token Llama-3-8B prefill), rotated past the
        cache, and the forward at 64x4096 (a decode step of 64 requests);
      * fused cross-entropy loss + gradient over GPT-2's vocabulary (50257
        classes in rows padded to 50304), 8x1024 tokens, bf16 and fp32, with
        the gradient in its own buffer and over the logits;
      * long softmax rows, fp16: 16x256 rows of 32768 keys in the register
        layouts and forced onto the two-pass path, and 8x256 rows of
        131072 keys (held on chip; the backward also with dropout) and
        forced onto the two-pass path, and the cross-entropy over a
        256000-class bf16 vocabulary at 2048 tokens (held on chip, then
        forced onto the two-pass path); the algorithmic bytes count one read
        and one write, though the two-pass path reads each row twice;
      * 64x768 fp32 forward + backward (launch-bound): microseconds per pass;
      * 16384x1024 bf16 backward (dx, dgamma, dbeta), rotated past the cache;
      * wide and ragged rows, fp32 and bf16: 4096x16384 and 65536x1000
        forward + backward (each pass moves more than the cache holds);
      * rows past the register layouts, staged in LDS: 4096x32768 bf16 and
        4096x19968 fp32 forward + backward, 2048x65536 forward in both.
    Rates of 16 MB or more come with the plain copy's rate at the same byte
    count; the prologue backward, the softmax with dropout, add + RMSNorm and
    the cross-entropy also with a CPU baseline (the float64 oracle on a
    sample of the rows, one thread)."""
    import subprocess
    tool = os.path.join(ROOT, "memory_bound_row_amd", "launch_bench")
    if not os.path.exists(tool):
        raise RuntimeError(f"{tool} is not built (run the package build)")
    cpp = {1: {}, 8: {}}
    for rows in ((1, 8) if cpp_launch else ()):
        r = subprocess.run([tool, str(rows), "4096", "10000", "1"], capture_output=True,
                           text=True, timeout=300)
        if r.returncode != 0:
            raise RuntimeError(f"launch_bench failed: {r.stderr.strip()}")
        cpp[rows] = json.loads(r.stdout)

    import numpy as np
    import torch
    import memory_bound_row_amd as mb
    import oracle as orc   # the CPU baselines only
    from memory_bound_row_amd import synth
    torch.cuda.init()
    dev = torch.device("cuda", 0)

    copy_cache = {}

    def copy_gbps(nbytes):
        """GB/s of the library's plain copy (`hbm_copy`) moving nbytes (half
        read, half written), rotated over enough buffer pairs to exceed the
        Infinity Cache: the attainable rate at that byte count."""
        key = int(round(nbytes / 1e6))
        if key not in copy_cache:
            n = (int(nbytes) // 2) // 16 * 4            # int32 elements per side
            pairs = max(2, -(-1_100_000_000 // (8 * n)))
            bufs = [(torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int32, device=dev),
                     torch.empty(n, dtype=torch.int32, device=dev)) for _ in range(pairs)]
            k = 20
            ms = timed(capture(lambda i: mb.hbm_copy(bufs[i % pairs][0], bufs[i % pairs][1]),
                               k), k)
            copy_cache[key] = 8 * n / (ms * 1e-3) / 1e9
            del bufs
            torch.cuda.empty_cache()
        return copy_cache[key]

    def emit(rec):
        # each rate of at least 16 MB next to the copy rate at its byte count
        for pre, bkey in (("", "bytes_per_pass"), ("fwd_", "fwd_bytes"), ("bwd_", "bwd_bytes")):
            rate, nb = rec.get(pre + "GBps"), rec.get(bkey)
            if rate is not None and nb and nb >= 16_000_000:
                c = copy_gbps(nb)
                rec[pre + "copy_GBps"] = round(c, 1)
                rec[pre + "pct_of_copy"] = round(100.0 * rate / c, 1)
        print(json.dumps(rec), flush=True)

    # decode-shaped launch cost
    n = 10000
    for rows in (1, 8):
        inp = {k: v.to(dev) for k, v in
               synth.layer_inputs(rows, 4096, torch.float16, x_mean=3.0, x_std=2.0,
                                  names=("x", "gamma", "beta")).items()}
        y = torch.empty_like(inp["x"])

        def call(i, inp=inp, y=y):
            mb.ln_fwd(inp["x"], inp["gamma"], inp["beta"], EPS, y=y, stats=False)

        for i in range(200):
            call(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            call(i)
        torch.cuda.synchronize()
        py_us = (time.perf_counter() - t0) / n * 1e6
        g_us = timed(capture(call, n), n) * 1e3
        b = plain_bytes(rows, 4096, 2)["fwd"] - 8 * rows
        emit({"workload": f"decode-shaped fp16 LayerNorm forward, {rows}x4096, no saved stats",
              "calls": n, "bytes_per_call": b,
              "cpp_loop_us": cpp[rows].get("cpp_loop_us"), "cpp_graph_us": cpp[rows].get("graph_us"),
              "python_loop_us": round(py_us, 3), "torch_graph_us": round(g_us, 3)})

    def fwd_bwd(rows, cols, dtype, sets, iters, label, fwd=True, bwd=True):
        s = torch.tensor([], dtype=dtype).element_size()
        inp = synth.layer_inputs(rows, cols, dtype, names=("x", "gamma", "beta", "dy"))
        gamma, beta = inp["gamma"].to(dev), inp["beta"].to(dev)
        st = []
        for _ in range(sets):
            a = {"x": inp["x"].to(dev), "dy": inp["dy"].to(dev)}
            a["y"] = torch.empty_like(a["x"])
            a["dx"] = torch.empty_like(a["x"])
            a["mean"] = torch.empty(rows, dtype=torch.float32, device=dev)
            a["rstd"] = torch.empty(rows, dtype=torch.float32, device=dev)
            st.append(a)
        del inp
        ws = mb.workspace(rows, cols, dev)
        dg = torch.empty(cols, dtype=torch.float32, device=dev)
        db = torch.empty(cols, dtype=torch.float32, device=dev)

        def f(i):
            a = st[i % sets]
            mb.ln_fwd(a["x"], gamma, beta, EPS, y=a["y"], mean=a["mean"], rstd=a["rstd"])

        def bw(i):
            a = st[(i + sets // 2) % sets]
            mb.ln_bwd_dx(a["dy"], a["x"], gamma, a["mean"], a["rstd"], dx=a["dx"],
                         workspace=ws)
            mb.ln_bwd_dgamma_dbeta(ws, rows, cols, dtype, partials_ready=True, dgamma=dg,
                                   dbeta=db)

        def both(i):
            if fwd:
                f(i)
            if bwd:
                bw(i)

        for i in range(sets):
            f(i)
        torch.cuda.synchronize()
        pb = plain_bytes(rows, cols, s)
        ms = timed(capture(both, iters), iters)
        rec = {"workload": label, "rows": rows, "cols": cols, "storage": str(dtype)[6:],
               "buffer_sets": sets, "iters": iters}
        nb = (pb["step"] if fwd else pb["bwd"]) if bwd else pb["fwd"]
        rec["bytes_per_pass"] = nb
        rec["us_per_pass"] = round(ms * 1e3, 3)
        rec["GBps"] = round(nb / (ms * 1e-3) / 1e9, 1)
        rec["pct_of_hbm_peak"] = round(100.0 * nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)
        if fwd and bwd:
            msf = timed(capture(f, iters), iters)
            rec["fwd_bytes"] = pb["fwd"]
            rec["fwd_us"] = round(msf * 1e3, 3)
            rec["fwd_GBps"] = round(pb["fwd"] / (msf * 1e-3) / 1e9, 1)
        if bwd:
            msb = timed(capture(bw, iters), iters)
            rec["bwd_bytes"] = pb["bwd"]
            rec["bwd_fold_us"] = round(msb * 1e3, 3)
            rec["bwd_GBps"] = round(pb["bwd"] / (msb * 1e-3) / 1e9, 1)
        emit(rec)
        del st, ws
        torch.cuda.empty_cache()

    # the backward of the whole fused layer: LayerNorm dx + the prologue's
    # backward (dresidual, dx with the regenerated mask, dgamma/dbeta/dbias),
    # alone and after the fused forward (a training layer), rotated past the
    # cache
    R, C, S = ROWS, COLS, 8
    dt16 = torch.bfloat16
    inp = synth.layer_inputs(R, C, dt16, seed=SEED)
    ez_cpu = synth.layer_inputs(R, C, dt16, seed=SEED + 1, names=("dy",))["dy"]
    sh = {k: inp[k].to(dev) for k in ("bias", "gamma", "beta")}
    st = []
    for _ in range(S):
        a = {k: inp[k].to(dev) for k in ("x", "residual", "dy")}
        a["ez"] = ez_cpu.to(dev)
        for k in ("z", "y", "dres", "dxin"):
            a[k] = torch.empty((R, C), dtype=dt16, device=dev)
        a["mean"] = torch.empty(R, dtype=torch.float32, device=dev)
        a["rstd"] = torch.empty(R, dtype=torch.float32, device=dev)
        st.append(a)
    del inp
    wsd = mb.dropout_workspace(R, C, dev)
    pg = [torch.empty(C, dtype=torch.float32, device=dev) for _ in range(3)]

    def lfwd(i):
        a = st[i % S]
        mb.bias_dropout_residual_ln_fwd(a["x"], sh["bias"], a["residual"], sh["gamma"],
                                        sh["beta"], P_DROP, SEED, EPS, residual_out=a["z"],
                                        y=a["y"], mean=a["mean"], rstd=a["rstd"])

    def lbwd(i):
        a = st[(i + S // 2) % S]
        mb.bias_dropout_residual_ln_bwd(a["dy"], a["z"], sh["gamma"], a["mean"], a["rstd"],
                                        P_DROP, SEED, dz_extra=a["ez"], dresidual=a["dres"],
                                        dx=a["dxin"], dgamma=pg[0], dbeta=pg[1], dbias=pg[2],
                                        workspace=wsd)

    def layer(i):
        lfwd(i)
        lbwd(i)

    for i in range(S):
        lfwd(i)
    torch.cuda.synchronize()
    n = 200
    ms_b = timed(capture(lbwd, n), n)
    ms_l = timed(capture(layer, n), n)
    bb = 5 * R * C * 2 + C * 2 + 8 * R + 12 * C
    lb = algorithmic_bytes(R, C, 2)["fused_fwd"] + bb
    def pro_prep(n):
        i = {k: synth.as_f64(v) for k, v in synth.layer_inputs(n, C, dt16, seed=SEED).items()}
        ez = synth.as_f64(synth.layer_inputs(n, C, dt16, seed=SEED + 1, names=("dy",))["dy"])
        keep = orc.dropout_keep_rows(SEED, P_DROP, 0, n, C)
        z = orc.round_to(orc.bias_dropout_residual(i["x"], i["bias"], i["residual"], keep,
                                                   P_DROP), "bf16")
        _, mu, rs = orc.ln_fwd(z, i["gamma"], i["beta"], EPS)
        return i, ez, keep, z, np.float64(np.float32(mu)), np.float64(np.float32(rs))

    def pro_work(args):
        i, ez, keep, z, mu, rs = args
        dz = orc.ln_bwd_dx(i["dy"], z, i["gamma"], mu, rs) + ez
        orc.round_to(dz, "bf16")
        dxin, _, _ = orc.dropout_residual_bwd(dz, keep, P_DROP)
        orc.round_to(dxin, "bf16")
        orc.ln_bwd_params(i["dy"], z, mu, rs)

    emit({"workload": "fused backward of bias+dropout(p=0.1)+residual+LayerNorm "
                      "(dz_extra given), 8192x1280 bf16, rotated",
          "bytes_per_pass": bb, "us_per_pass": round(ms_b * 1e3, 3),
          "GBps": round(bb / (ms_b * 1e-3) / 1e9, 1),
          "pct_of_hbm_peak": round(100.0 * bb / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
          "cpu_baseline": oracle_rate(pro_prep, pro_work, 5 * C * 2, R)})
    emit({"workload": "training layer: fused forward + fused backward (p=0.1), "
                      "8192x1280 bf16, rotated",
          "bytes_per_pass": lb, "us_per_pass": round(ms_l * 1e3, 3),
          "GBps": round(lb / (ms_l * 1e-3) / 1e9, 1),
          "pct_of_hbm_peak": round(100.0 * lb / (ms_l * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)})
    del st, wsd
    torch.cuda.empty_cache()

    # attention softmax at the pages' shapes (fp16): batch 8 x 16 heads x
    # 512 x 512 with attention dropout p = 0.1, and 2 x 16 x 256 x 256 causal
    def softmax_case(rows, L, causal, p, label):
        dt = torch.float16
        d = synth.layer_inputs(rows, L, dt, seed=SEED, x_std=3.0, names=("x", "dy"))
        sets = []
        for _ in range(2):
            a = {"x": d["x"].to(dev), "dy": d["dy"].to(dev)}
            a["y"] = torch.empty_like(a["x"])
            a["yd"] = torch.empty_like(a["x"]) if p > 0 else None
            a["dx"] = torch.empty_like(a["x"])
            sets.append(a)
        del d
        scale = 0.125

        def f(i):
            a = sets[i % 2]
            mb.attn_softmax_fwd(a["x"], scale, causal=causal, p=p, seed=SEED, y=a["y"],
                                y_dropped=a["yd"])

        def b(i):
            a = sets[(i + 1) % 2]
            mb.attn_softmax_bwd(a["dy"], a["y"], scale, causal=causal, p=p, seed=SEED,
                                dx=a["dx"])

        for i in range(2):
            f(i)
        torch.cuda.synchronize()
        n = 50
        msf = timed(capture(f, n), n)
        msb = timed(capture(b, n), n)
        t = rows * L * 2
        read = t * (L + 1) / (2 * L) if causal else t     # scores past the query are not read
        fb = read + t * (2 if p > 0 else 1)
        bb = 2 * read + t
        def sm_prep(n):
            i = synth.layer_inputs(n, L, dt, seed=SEED, x_std=3.0, names=("x", "dy"))
            keep = orc.dropout_keep_rows(SEED, p, 0, n, L) if p > 0 else None
            return synth.as_f64(i["x"]), synth.as_f64(i["dy"]), keep

        def sm_work(args):
            x, dy, keep = args
            y = orc.attn_softmax_fwd(x, scale, causal=causal)
            if keep is not None:
                orc.round_to(np.where(keep == 1, y / (1.0 - p), 0.0), "f16")
            orc.attn_softmax_bwd(dy, orc.round_to(y, "f16"), keep, p, scale)

        cpu = None if causal else oracle_rate(sm_prep, sm_work, (fb + bb) / rows, rows)
        emit({"workload": label, "rows": rows, "cols": L, "storage": "float16",
              "causal": causal, "p": p, "cpu_baseline": cpu,
              "fwd_bytes": int(fb), "fwd_us": round(msf * 1e3, 3),
              "fwd_GBps": round(fb / (msf * 1e-3) / 1e9, 1),
              "fwd_pct_of_hbm_peak": round(100.0 * fb / (msf * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
              "bwd_bytes": int(bb), "bwd_us": round(msb * 1e3, 3),
              "bwd_GBps": round(bb / (msb * 1e-3) / 1e9, 1),
              "bwd_pct_of_hbm_peak": round(100.0 * bb / (msb * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                           2)})
        del sets
        torch.cuda.empty_cache()

    softmax_case(8 * 16 * 512, 512, False, 0.1,
                 "attention softmax fwd (y and dropped y) + bwd (with dropout), 8x16x512x512")
    softmax_case(2 * 16 * 256, 256, True, 0.0,
                 "attention softmax fwd + bwd, causal, 2x16x256x256")

    # fused residual add + RMSNorm (bf16): forward reads x and the residual
    # and writes z and y; backward reads dy, z and dz_extra and writes dz
    def rmsnorm_case(rows, cols, sets, iters, label, bwd=True):
        dt = torch.bfloat16
        d = synth.layer_inputs(rows, cols, dt, seed=SEED, names=("x", "residual", "gamma", "dy"))
        ez = synth.layer_inputs(rows, cols, dt, seed=SEED + 1, names=("dy",))["dy"]
        gamma = d["gamma"].to(dev)
        st = []
        for _ in range(sets):
            a = {k: d[k].to(dev) for k in ("x", "residual", "dy")}
            a["ez"] = ez.to(dev)
            for k in ("z", "y", "dz"):
                a[k] = torch.empty((rows, cols), dtype=dt, device=dev)
            a["rstd"] = torch.empty(rows, dtype=torch.float32, device=dev)
            st.append(a)
        del d, ez
        ws = mb.rmsnorm_workspace(rows, cols, dev)
        dg = torch.empty(cols, dtype=torch.float32, device=dev)

        def f(i):
            a = st[i % sets]
            mb.add_rmsnorm_fwd(a["x"], gamma, 1e-6, residual=a["residual"], residual_out=a["z"],
                               y=a["y"], rstd=a["rstd"])

        def b(i):
            a = st[(i + sets // 2) % sets]
            mb.add_rmsnorm_bwd(a["dy"], a["z"], gamma, a["rstd"], dz_extra=a["ez"], dz=a["dz"],
                               dgamma=dg, workspace=ws)

        for i in range(sets):
            f(i)
        torch.cuda.synchronize()
        t = rows * cols * 2
        fb = 4 * t + cols * 2 + 4 * rows
        msf = timed(capture(f, iters), iters)
        rec = {"workload": label, "rows": rows, "cols": cols, "storage": "bfloat16",
               "buffer_sets": sets, "iters": iters,
               "fwd_bytes": fb, "fwd_us": round(msf * 1e3, 3),
               "fwd_GBps": round(fb / (msf * 1e-3) / 1e9, 1),
               "fwd_pct_of_hbm_peak": round(100.0 * fb / (msf * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)}
        if bwd:
            bb = 4 * t + cols * 2 + 4 * rows + 4 * cols
            msb = timed(capture(b, iters), iters)
            rec.update({"bwd_bytes": bb, "bwd_us": round(msb * 1e3, 3),
                        "bwd_GBps": round(bb / (msb * 1e-3) / 1e9, 1),
                        "bwd_pct_of_hbm_peak": round(100.0 * bb / (msb * 1e-3) / 1e9
                                                     / HBM_PEAK_GBPS, 2)})

            def rms_prep(n):
                i = {k: synth.as_f64(v) for k, v in synth.layer_inputs(
                    n, cols, dt, seed=SEED, names=("x", "residual", "gamma", "dy")).items()}
                ez = synth.as_f64(synth.layer_inputs(n, cols, dt, seed=SEED + 1,
                                                     names=("dy",))["dy"])
                return i, ez

            def rms_work(args):
                i, ez = args
                z = orc.round_to(i["x"] + i["residual"], "bf16")
                y, rs = orc.rmsnorm_fwd(z, i["gamma"], 1e-6)
                orc.round_to(y, "bf16")
                dz, _, _ = orc.rmsnorm_bwd(i["dy"], z, i["gamma"], np.float64(np.float32(rs)))
                orc.round_to(dz + ez, "bf16")

            rec["cpu_baseline"] = oracle_rate(rms_prep, rms_work, 8 * cols * 2, rows)
        emit(rec)
        del st, ws
        torch.cuda.empty_cache()

    rmsnorm_case(2048, 4096, 4, 100,
                 "fused residual add + RMSNorm fwd + bwd (dz_extra given), 2048x4096, rotated")
    rmsnorm_case(64, 4096, 1, 1000, "fused residual add + RMSNorm forward, decode 64x4096",
                 bwd=False)

    # fused cross-entropy (loss + gradient) over a vocabulary-wide row
    def xent_case(rows, cols, ld, dt, label, two_pass=False, cpu=True):
        x = synth.logits(rows, ld, dt, seed=SEED).to(dev)
        lab = synth.class_labels(rows, cols, seed=SEED).to(dev)
        loss = torch.empty(rows, dtype=torch.float32, device=dev)
        dx = torch.empty_like(x)
        s = x.element_size()

        def f(i):
            mb.cross_entropy_fwd_bwd(x, lab, cols=cols, label_smoothing=0.1,
                                     grad_scale=1.0 / rows, loss=loss, dlogits=dx)

        def g(i):
            # the gradient over the logits (values change, the work does not)
            mb.cross_entropy_fwd_bwd(x, lab, cols=cols, label_smoothing=0.1,
                                     grad_scale=1.0 / rows, loss=loss, dlogits=x)

        mb.debug_force_two_pass(two_pass)
        try:
            for i in range(3):   # first touches of the fresh 0.4-3 GB buffers
                f(i)
            torch.cuda.synchronize()
            n = 20
            ms = timed(capture(f, n), n)
            ms_ip = timed(capture(g, n), n)
        finally:
            mb.debug_force_two_pass(False)
        b = 2 * rows * cols * s + 12 * rows

        def xe_prep(k):
            xs = synth.as_f64(synth.logits(k, ld, dt, seed=SEED))[:, :cols]
            return np.ascontiguousarray(xs), synth.class_labels(k, cols, seed=SEED).numpy()

        def xe_work(args):
            orc.cross_entropy(args[0], args[1], 0.1, 1.0 / rows)

        emit({"workload": label, "rows": rows, "cols": cols, "ld": ld,
              "storage": str(dt)[6:], "bytes_per_pass": b, "iters": n,
              "us_per_pass": round(ms * 1e3, 3), "GBps": round(b / (ms * 1e-3) / 1e9, 1),
              "pct_of_hbm_peak": round(100.0 * b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
              "in_place_us": round(ms_ip * 1e3, 3),
              "in_place_GBps": round(b / (ms_ip * 1e-3) / 1e9, 1),
              **({"cpu_baseline": oracle_rate(xe_prep, xe_work, b / rows, rows)} if cpu else {})})
        del x, dx, lab, loss
        torch.cuda.empty_cache()

    for dt in (torch.bfloat16, torch.float32):
        xent_case(8192, 50257, 50304, dt,
                  "fused cross-entropy loss + gradient, GPT-2 vocabulary, 8x1024 tokens")
    xent_case(2048, 256000, 256000, torch.bfloat16,
              "fused cross-entropy, 256000-class vocabulary (row held in registers and LDS), "
              "2048 tokens")
    xent_case(2048, 256000, 256000, torch.bfloat16,
              "fused cross-entropy, 256000-class vocabulary, forced onto the two-pass path, "
              "2048 tokens", two_pass=True, cpu=False)

    # softmax over long rows: the register layouts (32768 keys; also forced
    # onto the two-pass path, for comparison) and the two-pass path past them
    # (131072 keys)
    def long_softmax(rows, L, label, two_pass=False, p=0.0, rows_per_mask=0):
        d = synth.layer_inputs(rows, L, torch.float16, seed=SEED, x_std=3.0, names=("x", "dy"))
        a = {"x": d["x"].to(dev), "dy": d["dy"].to(dev)}
        del d
        a["mask"] = None
        if rows_per_mask:
            a["mask"] = synth.layer_inputs(rows // rows_per_mask, L, torch.float16, seed=SEED + 1,
                                           names=("dy",))["dy"].to(dev)
        a["y"] = torch.empty_like(a["x"])
        a["dx"] = torch.empty_like(a["x"])
        a["yd"] = torch.empty_like(a["x"]) if p > 0 else None

        def lf(i):
            mb.attn_softmax_fwd(a["x"], 0.125, mask=a["mask"], rows_per_mask=max(rows_per_mask, 1),
                                p=p, seed=SEED, y=a["y"], y_dropped=a["yd"])

        def lb(i):
            mb.attn_softmax_bwd(a["dy"], a["y"], 0.125, p=p, seed=SEED, dx=a["dx"])

        mb.debug_force_two_pass(two_pass)
        try:
            for i in range(3):
                lf(i)
                lb(i)
            torch.cuda.synchronize()
            n = 10
            msf = timed(capture(lf, n), n)
            msb = timed(capture(lb, n), n)
        finally:
            mb.debug_force_two_pass(False)
        t = rows * L * 2
        nf = 3 if p > 0 else 2   # x read; y (and the dropped copy) written
        fb = nf * t + (t // rows_per_mask if rows_per_mask else 0)   # and the mask rows
        emit({"workload": label, "rows": rows, "cols": L, "storage": "float16",
              "dropout": p, "rows_per_mask": rows_per_mask or None, "fwd_bytes": fb,
              "fwd_us": round(msf * 1e3, 3), "fwd_GBps": round(fb / (msf * 1e-3) / 1e9, 1),
              "bwd_bytes": 3 * t, "bwd_us": round(msb * 1e3, 3),
              "bwd_GBps": round(3 * t / (msb * 1e-3) / 1e9, 1)})
        del a
        torch.cuda.empty_cache()

    long_softmax(16 * 256, 32768,
                 "attention softmax fwd + bwd, 16x256 rows of 32768 keys (register layouts)")
    long_softmax(16 * 256, 32768,
                 "attention softmax fwd + bwd, 16x256 rows of 32768 keys, forced onto the "
                 "two-pass path", two_pass=True)
    long_softmax(8 * 256, 131072,
                 "attention softmax fwd + bwd, 8x256 rows of 131072 keys (forward without a mask "
                 "or dropped copy in registers, backward without dropout on chip)")
    long_softmax(8 * 256, 131072,
                 "attention softmax fwd + bwd, 8x256 rows of 131072 keys, forced onto the "
                 "two-pass path", two_pass=True)
    long_softmax(8 * 256, 131072,
                 "attention softmax fwd (y and the dropped copy) + bwd with dropout p = 0.1, "
                 "8x256 rows of 131072 keys (both on chip)", p=0.1)
    long_softmax(8 * 256, 131072,
                 "attention softmax fwd (y and the dropped copy) + bwd with dropout p = 0.1, "
                 "8x256 rows of 131072 keys, forced onto the two-pass path", two_pass=True, p=0.1)
    long_softmax(8 * 256, 131072,
                 "attention softmax fwd with a mask row per 16 rows + bwd, 8x256 rows of 131072 "
                 "keys (both on chip)", rows_per_mask=16)
    long_softmax(8 * 256, 131072,
                 "attention softmax fwd with a mask row per 16 rows + bwd, 8x256 rows of 131072 "
                 "keys, forced onto the two-pass path", two_pass=True, rows_per_mask=16)

    fwd_bwd(64, 768, torch.float32, 1, 1000,
            "LayerNorm forward + backward fp32 64x768 (launch-bound)")
    fwd_bwd(16384, 1024, torch.bfloat16, 4, 100,
            "LayerNorm backward (dx, dgamma, dbeta) bf16 16384x1024, rotated", fwd=False)
    for dtype in (torch.float32, torch.bfloat16):
        for rows, cols in ((4096, 16384), (65536, 1000)):
            fwd_bwd(rows, cols, dtype, 2, 20, "LayerNorm forward + backward, wide/ragged rows")
    # rows past the register layouts, staged in LDS
    fwd_bwd(4096, 32768, torch.bfloat16, 2, 20,
            "LayerNorm forward + backward, LDS-staged rows (widest 16-bit backward)")
    fwd_bwd(4096, 19968, torch.float32, 2, 20,
            "LayerNorm forward + backward, LDS-staged rows (widest fp32 backward)")
    for dtype in (torch.float32, torch.bfloat16):
        fwd_bwd(2048, 65536, dtype, 2, 20, "LayerNorm forward, LDS-staged rows (widest; fp32 "
                "slots past the stage read again for the output)", bwd=False)


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.configs:
        configs_report(cpp_launch=not args.no_cpp_launch)
        return
    if args.counter_sample:
        counter_sample()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the method's rows "
              "shard across GPUs with no communication except a [3, cols] parameter-gradient "
              "exchange, which this benchmark does not run.", file=sys.stderr)
        sys.exit(2)
    import torch
    import memory_bound_row_amd as mb
    from memory_bound_row_amd import synth

    torch.cuda.init()
    dev = torch.device("cuda", 0)
    dtype = torch.bfloat16
    K, W = args.steps, args.warmup
    S = 1 if args.warm_cache else max(2, args.sets)
    H = S // 2
    inp_cpu = synth.layer_inputs(ROWS, COLS, dtype, seed=SEED)
    # the gradient reaching z from the residual stream (drawn like dy)
    inp_cpu["ez"] = synth.layer_inputs(ROWS, COLS, dtype, seed=SEED + 1, names=("dy",))["dy"]
    shared = {k: inp_cpu[k].to(dev) for k in ("bias", "gamma", "beta")}
    sets = []
    for _ in range(S):
        st = {k: inp_cpu[k].to(dev) for k in ("x", "residual", "dy", "ez")}
        for k in ("z", "y", "dres", "dxin", "dx"):
            st[k] = torch.empty((ROWS, COLS), dtype=dtype, device=dev)
        st["mean"] = torch.empty(ROWS, dtype=torch.float32, device=dev)
        st["rstd"] = torch.empty(ROWS, dtype=torch.float32, device=dev)
        sets.append(st)
    wsd = mb.dropout_workspace(ROWS, COLS, dev)
    ws = mb.workspace(ROWS, COLS, dev)
    pg = [torch.empty(COLS, dtype=torch.float32, device=dev) for _ in range(3)]

    def fwd(a):
        mb.bias_dropout_residual_ln_fwd(a["x"], shared["bias"], a["residual"], shared["gamma"],
                                        shared["beta"], P_DROP, SEED, EPS, residual_out=a["z"],
                                        y=a["y"], mean=a["mean"], rstd=a["rstd"])

    def bwd(b):
        mb.bias_dropout_residual_ln_bwd_dx(b["dy"], b["z"], shared["gamma"], b["mean"],
                                           b["rstd"], P_DROP, SEED, workspace=wsd,
                                           dz_extra=b["ez"], dresidual=b["dres"], dx=b["dxin"])

    def fold():
        mb.bias_dropout_residual_ln_bwd_fold(wsd, ROWS, COLS, dgamma=pg[0], dbeta=pg[1],
                                             dbias=pg[2])

    def step(i):
        fwd(sets[i % S])
        bwd(sets[(i + H) % S])
        fold()

    # every set gets valid z/mean/rstd before any backward reads it
    for a in sets:
        fwd(a)
    for i in range(W):
        step(i)
    torch.cuda.synchronize()

    g_step = capture(step, K)
    ms_step = timed(g_step, K)
    dist = step_distribution(g_step, K, 20)
    # each kernel alone over the same rotation, timed with HIP events on the
    # stream it is launched on (the graph's)
    ms_fwd = timed(capture(lambda i: fwd(sets[i % S]), K), K)
    ms_bwd = timed(capture(lambda i: bwd(sets[(i + H) % S]), K), K)
    ms_fold = timed(capture(lambda i: fold(), K), K)

    # the metric case of the hot-path scope table: ln_fwd of x, then the
    # LayerNorm backward on x (dx with partials, then the fold)
    def ln_bwd_call(b, xk):
        mb.ln_bwd_dx(b["dy"], b[xk], shared["gamma"], b["mean"], b["rstd"], dx=b["dx"],
                     workspace=ws)
        mb.ln_bwd_dgamma_dbeta(ws, ROWS, COLS, dtype, partials_ready=True, dgamma=pg[0],
                               dbeta=pg[1])

    def plain_step(i):
        a = sets[i % S]
        mb.ln_fwd(a["x"], shared["gamma"], shared["beta"], EPS, y=a["y"], mean=a["mean"],
                  rstd=a["rstd"])
        ln_bwd_call(sets[(i + H) % S], "x")

    ms_plain = timed(capture(plain_step, K), K)

    # the fused forward followed by the plain LayerNorm backward of z
    def mixed_step(i):
        fwd(sets[i % S])
        ln_bwd_call(sets[(i + H) % S], "z")

    for a in sets:
        fwd(a)
    torch.cuda.synchronize()
    ms_mixed = timed(capture(mixed_step, K), K)
    ms_lnbwd = timed(capture(lambda i: ln_bwd_call(sets[(i + H) % S], "z"), K), K)

    nb = algorithmic_bytes(ROWS, COLS, 2)
    pb = plain_bytes(ROWS, COLS, 2)
    lb = ln_bwd_bytes(ROWS, COLS, 2)
    t = ROWS * COLS * 2
    # attainable bandwidth of each kernel's mix of reads and writes
    refs = stream_rates({"fused_fwd": (2, 2, 4 * t), "prologue_bwd": (3, 2, 5 * t),
                         "ln_fwd": (1, 1, 2 * t), "ln_bwd": (2, 1, 3 * t)}, S, dev, K)
    # calibration copy for the HBM traffic counters (256 MiB each way)
    big = [torch.randint(-2**31, 2**31 - 1, (COPY_BYTES // 4,), dtype=torch.int32, device=dev)
           for _ in range(2)]
    mb.hbm_copy(big[0], big[1])
    torch.cuda.synchronize()
    del big

    value = nb["step"] / (ms_step * 1e-3) / 1e9
    per_kernel = {
        "ln_fwd_kernel(fused)": (ms_fwd, nb["fused_fwd"]),
        "ln_bwd_kernel(prologue)": (ms_bwd, nb["prologue_bwd"]),
    }
    dom = max(per_kernel, key=lambda k: per_kernel[k][0])
    ms_dom, b_dom = per_kernel[dom]
    achieved = b_dom / (ms_dom * 1e-3) / 1e9
    src_hash = kernel_source_hash()
    traffic = load_traffic(dom, src_hash)
    ref_step_us = refs["fused_fwd"][1] + refs["prologue_bwd"][1]

    def gbps(nbytes, ms):
        return round(nbytes / (ms * 1e-3) / 1e9, 1)

    out = {
        "metric": "achieved HBM GB/s (% of peak) for fused LayerNorm fwd+bwd, 8192x1280 bf16",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "rows": ROWS, "cols": COLS, "storage": "bf16",
                   "arithmetic": "f32", "p": P_DROP, "buffer_sets": S,
                   "cache": "warm (one set)" if args.warm_cache else "rotated past 256 MB"},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "rows_per_s": round(ROWS / (ms_step * 1e-3), 1),
        "bytes_per_step": nb["step"],
        "kernel_us": {"fused_fwd": round(ms_fwd * 1e3, 3), "prologue_bwd": round(ms_bwd * 1e3, 3),
                      "fold": round(ms_fold * 1e3, 3)},
        "step_us": dist,
        "reference_GBps": {k: v[0] for k, v in refs.items()},
        "pct_of_reference": {
            "step": round(100.0 * ref_step_us / (ms_step * 1e3), 1),
            "fused_fwd": round(100.0 * refs["fused_fwd"][1] / (ms_fwd * 1e3), 1),
            "prologue_bwd": round(100.0 * refs["prologue_bwd"][1] / (ms_bwd * 1e3), 1)},
        "metric_case": {"workload": "ln_fwd, then ln_bwd_dx with partials and the fold, "
                                    "8192x1280 bf16 (the scope table's metric case)",
                        "bytes_per_step": pb["step"], "ms_per_step": round(ms_plain, 5),
                        "GBps": gbps(pb["step"], ms_plain),
                        "pct_of_hbm_peak": round(100.0 * pb["step"] / (ms_plain * 1e-3) / 1e9
                                                 / HBM_PEAK_GBPS, 2),
                        "pct_of_reference": round(
                            100.0 * (refs["ln_fwd"][1] + refs["ln_bwd"][1]) / (ms_plain * 1e3),
                            1)},
        "mixed_step": {"workload": "the fused forward, then the LayerNorm backward of z "
                                   "(dx with partials, fold)",
                       "bytes_per_step": nb["fused_fwd"] + lb, "ms_per_step": round(ms_mixed, 5),
                       "GBps": gbps(nb["fused_fwd"] + lb, ms_mixed),
                       "ln_bwd_with_fold_us": round(ms_lnbwd * 1e3, 3)},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "bytes_per_launch": b_dom,
                     "event_us": round(ms_dom * 1e3, 3), "source_hash": src_hash},
    }
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(inp_cpu, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
