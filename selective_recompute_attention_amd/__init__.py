"""Selective-recompute KV-cache fusion for AMD Instinct MI355X (gfx950).

The compute path is libsra.so (hand-written HIP kernels behind the C ABI in include/sra.h);
this package only binds it. ``api`` holds one Python function per C entry point.
"""
from . import api  # noqa: F401
from .api import *  # noqa: F401,F403
