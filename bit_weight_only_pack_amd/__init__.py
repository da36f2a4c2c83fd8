"""Low-bit weight-only matmul for AMD Instinct MI355X (gfx950).

The compute lives in ``liblowbit.so`` (hand-written HIP kernels behind the C
ABI declared in ``include/lowbit.h``); ``_lib`` is a thin ctypes binding with
the same entry-point names.  PyTorch is used only for device memory and
streams.  ``synth`` draws the seeded synthetic workloads.
"""
from ._lib import *  # noqa: F401,F403
from ._lib import LowbitError, check, lib  # noqa: F401
