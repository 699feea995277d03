"""Build libmbrow_ln.so (HIP, gfx950) in-tree with hipcc.

Each kernel file is compiled once per storage type in parallel; the objects
go to ``_build/`` next to this file and the library to
``memory_bound_row_amd/libmbrow_ln.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmbrow_ln.so")
LAUNCH_BENCH = os.path.join(HERE, "launch_bench")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # no packed-FP32 instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE,
]

UNITS = (
    [("ln_fwd.hip", ["-DMBROW_DT=%d" % d], "ln_fwd_%d.o" % d) for d in range(3)]
    + [("ln_bwd.hip", ["-DMBROW_DT=%d" % d], "ln_bwd_%d.o" % d) for d in range(3)]
    + [("softmax.hip", ["-DMBROW_DT=%d" % d], "softmax_%d.o" % d) for d in range(3)]
    + [("rmsnorm.hip", ["-DMBROW_DT=%d" % d], "rmsnorm_%d.o" % d) for d in range(3)]
    + [("xent.hip", ["-DMBROW_DT=%d" % d], "xent_%d.o" % d) for d in range(3)]
    + [("stream.hip", ["-DMBROW_DT=%d" % d], "stream_%d.o" % d) for d in range(3)]
    + [("ln_wide.hip", ["-DMBROW_DT=%d" % d], "ln_wide_%d.o" % d) for d in range(3)]
    + [("ln_fold.hip", [], "ln_fold.o"), ("copy.hip", [], "copy.o"),
       ("noalloc.hip", [], "noalloc.o"),
       ("ln_api.cpp", [], "ln_api.o")]
)


def _spilling_kernels(remarks: str):
    """Kernels whose resource-usage remarks report VGPR spills or scratch."""
    bad = []
    for block in re.split(r"remark: Function Name: ", remarks)[1:]:
        name = block.split()[0]
        spill = re.search(r"VGPRs Spill: (\d+)", block)
        scratch = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", block)
        if (spill and int(spill.group(1))) or (scratch and int(scratch.group(1))):
            bad.append(name)
    return bad


def _compile(unit, build_dir=BUILD, extra=(), csrc=CSRC):
    src, defs, obj = unit
    out = os.path.join(build_dir, obj)
    cmd = [HIPCC, *COMMON, "-I", csrc, *extra, *defs, "-Rpass-analysis=kernel-resource-usage",
           "-c", os.path.join(csrc, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    # every kernel must fit in registers: a spilling instance is a build error
    bad = _spilling_kernels(r.stderr)
    if bad:
        raise RuntimeError("%s: kernels spill registers:\n  %s" % (src, "\n  ".join(bad)))
    return out


def build(jobs: int | None = None, verbose: bool = False, extra_flags=(), out_lib: str = LIB,
          build_dir: str = BUILD, csrc: str = CSRC) -> str:
    """Compile every unit of `csrc` and link `out_lib`; `extra_flags` go to
    every hipcc compile."""
    os.makedirs(build_dir, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda u: _compile(u, build_dir, tuple(extra_flags), csrc), UNITS))
    tmp = out_lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp,
           "-L", os.path.join(ROCM, "lib"), "-lrocprofiler-sdk-roctx",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, out_lib)
    if verbose:
        print("built", out_lib)
    if out_lib == LIB:
        build_launch_bench(verbose)
    return out_lib


def build_launch_bench(verbose: bool = False) -> str:
    """The host-side launch-cost tool (``launch_bench``), linked against the
    library next to it."""
    tmp = LAUNCH_BENCH + ".tmp"
    cmd = [HIPCC, *COMMON, os.path.join(CSRC, "launch_bench.cpp"), "-o", tmp,
           "-L", HERE, "-lmbrow_ln", "-Wl,-rpath,$ORIGIN"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("launch_bench build failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LAUNCH_BENCH)
    if verbose:
        print("built", LAUNCH_BENCH)
    return LAUNCH_BENCH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
