"""kvq: INT8-quantized KV cache with fused decode / prefill attention for MI355X.

The compute path is libkvq.so (hand-written HIP kernels for gfx950) behind the
C ABI in include/kvq.h; this package binds it with ctypes (``kvq``) and offers
a torch-owned storage wrapper (``Int8KVCache``).  Importing fails if the
library has not been built.
"""
from . import kvq  # noqa: F401  (loads libkvq.so or raises ImportError)
from .kvq import KvqError  # noqa: F401
from .cache import Int8KVCache, rolling_block_table  # noqa: F401

__all__ = ["kvq", "KvqError", "Int8KVCache", "rolling_block_table"]
