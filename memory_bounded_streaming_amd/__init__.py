"""Stream-CQSA forward on MI355X (gfx950): CQS planner, stream engine and HIP kernels.

The compute path lives in the C-ABI library ``libcqsa.so`` built from ``csrc/``
(see ``include/cqsa.h``); ``cqsa`` is its ctypes binding and loads it lazily.
``inputs`` draws the seeded synthetic Q/K/V.  Importing this package does not
load the library.
"""
__all__ = ["cqsa", "inputs"]
