"""MI355X-native paged KV cache decode path.

libpagedkv.so (built in-tree by ``python -m paged_kv_cache_60_amd.build``)
holds the gfx950 kernels -- paged_kv_write, paged_block_copy,
paged_attn_decode -- and the C++ host block manager, behind the C ABI in
``include/pagedkv.h``. This package is the thin Python binding: ctypes
marshalling of torch tensors and a small engine that drives one decode step.
"""
from ._lib import PkvError, load  # noqa: F401
from .block_manager import BlockManager  # noqa: F401
from .ops import (decode_workers, paged_attn_decode, paged_block_copy,  # noqa: F401
                  paged_kv_write, workspace_bytes)

__all__ = ["BlockManager", "PkvError", "load", "paged_attn_decode", "paged_block_copy",
           "paged_kv_write", "workspace_bytes", "decode_workers"]
