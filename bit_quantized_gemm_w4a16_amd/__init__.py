"""hq: MI355X-native (gfx950) quantized GEMM library.

The product is libhq.so (C ABI in include/hq.h); `hq` is its ctypes binding.
"""
from . import hq  # noqa: F401
from .hq import *  # noqa: F401,F403
