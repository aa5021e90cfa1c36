"""MI355X-native W4A8 single-token decode GEMV (gfx950 HIP kernels behind a C ABI).

The compute lives in ``libbqd.so`` (``include/bqd.h``); ``bqd`` is its thin
ctypes binding with the same entry-point names, and ``inputs`` the seeded
synthetic input generator.
"""
from .bqd import *  # noqa: F401,F403
from .bqd import BQDError, LayerPlan, LinearW4A8, lib, make_linear  # noqa: F401
