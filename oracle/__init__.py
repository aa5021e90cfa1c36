"""CPU oracle of the W4A8 decode GEMV path (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never does: it runs
entirely in the HIP library and fails loudly when that library is missing.
"""
from .oracle import *  # noqa: F401,F403
