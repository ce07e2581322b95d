"""MI355X (gfx950) paged KV-cache decode attention.

Hand-written HIP kernels behind the C ABI in include/pagedkv.h, built in-tree
into libpagedkv.so; this package is the thin torch binding
(``paged_kv_cache_283_amd.ops``) plus the host-side block allocator
(``block_manager``).  The library is loaded on first use of an op and its
absence is an error, never a fallback.
"""
from .block_manager import BlockManager, OutOfBlocks  # noqa: F401

__all__ = ["BlockManager", "OutOfBlocks"]
