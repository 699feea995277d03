"""Pin of the oracle's Philox4x32-10 round function (the dropout mask's
generator) against an independent implementation of the same published
generator: rocRAND's header-only host engine, built here with hipcc into a
small host program (tests/philox_library_ref.cpp).  CPU only.

The counters cover zero, all-ones words, the carry edges of each word and
seeded random values; keys cover zero, all-ones and random seeds.  rocRAND
reaches counter (x, y, z, w) as subsequence w:z and offset 4·(y:x), which
limits word y to below 2^30 here.  The mask's own layout on top of this
function (counter = (col >> 3, row lo, row hi, 0), 16-bit halves, the keep
threshold) is pinned in tests/test_oracle_pins.py; here the same layout is
also rebuilt from rocRAND's words for a block of rows and compared with the
oracle's mask bit for bit.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc")
                                  else None)
HEADER = "/opt/rocm/include/rocrand/rocrand_kernel.h"

pytestmark = pytest.mark.skipif(HIPCC is None or not os.path.exists(HEADER),
                                reason="hipcc or the rocRAND headers are not available")


@pytest.fixture(scope="module")
def ref_exe(tmp_path_factory):
    exe = tmp_path_factory.mktemp("philox") / "philox_library_ref"
    r = subprocess.run([HIPCC, "-O1", "-o", str(exe),
                        os.path.join(ROOT, "tests", "philox_library_ref.cpp")],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    return str(exe)


def library_blocks(exe, cases):
    """cases: iterable of (seed, (x, y, z, w)); returns an (n, 4) uint32 array."""
    lines = []
    for seed, (x, y, z, w) in cases:
        assert y < (1 << 30)
        lines.append(f"{seed} {(w << 32) | z} {4 * ((y << 32) | x)}")
    r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    out = np.array([[int(t) for t in ln.split()] for ln in r.stdout.split("\n") if ln.strip()],
                   dtype=np.uint64)
    assert out.shape == (len(lines), 4)
    return out.astype(np.uint32)


def oracle_block(seed, ctr):
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint32)
    return orc.philox4x32_10(np.array(ctr, np.uint32), key)


def test_round_function_matches_library(ref_exe):
    rng = np.random.default_rng(20240607)
    m32, m30 = 0xFFFFFFFF, (1 << 30) - 1
    seeds = [0, 1, m32, m32 << 32, (1 << 64) - 1, 0x0123456789ABCDEF]
    seeds += [int(s) for s in rng.integers(0, 1 << 63, size=6, dtype=np.int64)]
    ctrs = [(0, 0, 0, 0), (1, 0, 0, 0), (0, 1, 0, 0), (0, 0, 1, 0), (0, 0, 0, 1),
            (m32, 0, 0, 0), (m32, m30, m32, m32), (0, 0, m32, 0), (0, 0, 0, m32),
            (7, 12345, 0, 0)]
    ctrs += [tuple(int(v) for v in c) for c in
             zip(rng.integers(0, 1 << 32, 16, dtype=np.uint64),
                 rng.integers(0, 1 << 30, 16, dtype=np.uint64),
                 rng.integers(0, 1 << 32, 16, dtype=np.uint64),
                 rng.integers(0, 1 << 32, 16, dtype=np.uint64))]
    cases = [(s, c) for s in seeds for c in ctrs]
    lib = library_blocks(ref_exe, cases)
    ours = np.stack([oracle_block(s, c) for s, c in cases])
    bad = np.nonzero((lib != ours).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} of {len(cases)} blocks differ, first {cases[bad[0]]}"


def test_mask_rebuilt_from_library_words(ref_exe):
    """The oracle's dropout mask over rows 1000..1004 x 100 columns equals the
    layout applied to rocRAND's words: word (col & 7) >> 1 of the block for
    counter (col >> 3, row, 0, 0), its 16-bit half col & 1, kept iff that
    half is at least round(p * 65536)."""
    seed, p, row0, rows, cols = 0x5EED_1234_ABCD, 0.3, 1000, 5, 100
    keep = orc.dropout_keep_rows(seed, p, row0, rows, cols)
    thr = int(np.floor(p * 65536.0 + 0.5))
    blocks = (cols + 7) // 8
    lib = library_blocks(ref_exe, [(seed, (b, row0 + r, 0, 0))
                                   for r in range(rows) for b in range(blocks)])
    lib = lib.reshape(rows, blocks, 4)
    want = np.zeros((rows, cols), bool)
    for r in range(rows):
        for c in range(cols):
            word = int(lib[r, c >> 3, (c & 7) >> 1])
            half = (word >> (16 * (c & 1))) & 0xFFFF
            want[r, c] = half >= thr
    assert np.array_equal(np.asarray(keep, bool), want)
