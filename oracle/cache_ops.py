"""Paged cache writes: slot scatter and whole-block copy. TEST INFRASTRUCTURE.

Cache layout (both K and V): array [num_blocks, num_kv_heads, block_size, head_dim].
A slot is block * block_size + offset: the page-table mapping of
"From OOM to Smooth Inference (RAG memory management)", §2.1 (logical block i
of a sequence is stored in physical block table[i]; token t sits at offset
t mod block_size of logical block t // block_size).

fp16 caches store the value unchanged. fp8 caches (e4m3, or e5m2) store
encode(float32(x) * float32(inv_scale)) per "Where Did the VRAM Go (KV cache
tutorial)", §6.1-6.3 (see oracle.fp8); inv_scale is one value per tensor or
one per KV head.
"""
from __future__ import annotations

import numpy as np

from . import fp8


def scatter(k_cache, v_cache, k_new, v_new, slot_mapping, block_size,
            kv_dtype="f16", k_inv_scale=1.0, v_inv_scale=1.0):
    """Write token i's K/V rows into slot slot_mapping[i], in order; -1 skips.

    k_new, v_new: [T, num_kv_heads, head_dim] float16.
    """
    k_new = np.asarray(k_new)
    v_new = np.asarray(v_new)
    if kv_dtype in fp8.KV_FORMATS:
        fmt = fp8.KV_FORMATS[kv_dtype]
        k_src = fp8.quantize(k_new, k_inv_scale, fmt)
        v_src = fp8.quantize(v_new, v_inv_scale, fmt)
    else:
        k_src, v_src = k_new, v_new
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), block_size)
        k_cache[blk, :, off, :] = k_src[i]
        v_cache[blk, :, off, :] = v_src[i]


def block_copy(k_cache, v_cache, pairs):
    """cache[dst] = cache[src] for K and V, whole block, pairs applied in order.

    Copy-on-write duplicates the shared block before the write
    ("vLLM Architecture and Memory Use, ch. 3", §3.3).
    """
    for src, dst in pairs:
        k_cache[int(dst)] = k_cache[int(src)]
        v_cache[int(dst)] = v_cache[int(src)]


def block_swap(src_k, src_v, dst_k, dst_v, pairs):
    """dst[d] = src[s] for K and V, whole block, for every (s, d) pair.

    Swapping a preempted request copies its blocks to CPU memory and back
    ("Where Did the VRAM Go (KV cache tutorial)", §7.1-7.2; "From OOM to Smooth
    Inference", §5): out, src = device caches and dst = host caches; in, the
    other way round.
    """
    for s, d in pairs:
        dst_k[int(d)] = src_k[int(s)]
        dst_v[int(d)] = src_v[int(s)]
