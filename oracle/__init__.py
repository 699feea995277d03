"""float64 CPU oracle for fused LayerNorm forward/backward.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
never imports, links or calls it, and it shares no code with the GPU library.

The arithmetic lives in ``ln_oracle.c`` (plain C, float64); this module only
builds it with gcc and marshals numpy arrays through ctypes.  ``compare``
holds the tolerance rule used to check GPU outputs against it.

The Philox-based dropout mask: Philox4x32-10 is written here from its
published definition (Salmon et al., SC'11); the pages print no known-answer
values for it, so its round function is pinned against an independent
implementation of the same generator (rocRAND's host engine, in
tests/test_philox_pin.py).  The counter/key layout is this library's own
(the pages only say the mask is regenerated from a seed); the tests pin the
layout and the keep statistics, and the GPU and oracle implementations,
written independently, are checked against each other bit for bit.
"""
from .oracle import *  # noqa: F401,F403
