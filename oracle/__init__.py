"""CPU oracle for the KV-injection hot path — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, fp64 statement of what the hot path computes
(score, top-k, compose, Chunked RoPE, paged scatter, host fetch), and of the
attention read of the injected cache.  It exists to
check the GPU library against.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call it; the product
path (the C-ABI library and its Python binding) never does, and shares no code
with it.

Every function is pinned by ``-m "not gpu"`` tests against closed forms,
invariants, library routines or brute force (see ``tests/test_oracle_*.py``).
"""

from .fs_oracle import *  # noqa: F401,F403
