"""Block-quantized matrix multiplication with a selective high-precision
path on AMD Instinct MI355X (gfx950).

The compute path is librq.so -- hand-written HIP kernels behind the C ABI
declared in include/rq.h.  `_lib` is its ctypes binding (functions named
like the C entry points); `api` adds output allocation with torch device
memory.  Neither computes anything itself.
"""

from ._lib import *  # noqa: F401,F403
from . import api  # noqa: F401
