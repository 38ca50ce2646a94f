"""One tensor-parallel rank's share of a Transformer layer on an MI355X (gfx950).

The compute lives in libtpshard.so (hand-written HIP kernels behind a C ABI,
declared in include/tpshard.h); `tpshard` is its thin ctypes binding.  torch
is used for device memory and streams only.
"""
from . import tpshard  # noqa: F401
from .tpshard import *  # noqa: F401,F403

__all__ = [n for n in dir(tpshard) if n.startswith("tp_")] + ["TPError"]
