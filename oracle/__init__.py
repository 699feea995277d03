"""float64 CPU oracle for fused LayerNorm forward/backward.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
never imports, links or calls it, and it shares no code with the GPU library.

The arithmetic lives in ``ln_oracle.c`` (plain C, float64); this module only
builds it with gcc and marshals numpy arrays through ctypes.  ``compare``
holds the tolerance rule used to check GPU outputs against it.

Parity unpinned: the Philox-based dropout mask is pinned by published
known-answer values of Philox4x32-10 and by statistics, but the choice of
counter/key layout is this library's own (the pages only say the mask is
regenerated from a seed); the GPU and oracle implementations of that layout
are written independently and checked against each other.
"""
from .oracle import *  # noqa: F401,F403
