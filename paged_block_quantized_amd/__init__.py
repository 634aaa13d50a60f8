"""Block-quantized paged KV cache and fused dequantizing decode attention for
MI355X (gfx950).  The compute path is libpbq.so (HIP kernels behind the C ABI
in include/pbq.h); this package only marshals arguments to it.
"""

from . import _lib  # noqa: F401
from ._lib import PBQError, lib  # noqa: F401
from .pool import KVPool  # noqa: F401
