"""Opt-in host checks for the preconditions the kernels rely on but cannot see.

Two valid tokens written to one slot race (the later store may land first),
and a block-copy pair whose destination is another pair's source or
destination races with that pair: both are stated preconditions of
paged_kv_write and paged_block_copy. Copy-on-write only ever copies a shared
block into a fresh one ("vLLM Architecture and Memory Use, ch. 3", §3.3), and
the block manager hands each new token its own slot ("From OOM to Smooth
Inference (RAG memory management)", §2.3), so the block manager never breaks
them; these checks are for callers that build slot mappings or pairs
themselves.

With debug checks on (set_debug_checks(True), or PKV_DEBUG_CHECKS=1 in the
environment), the wrappers in ops copy the slot mapping or the pairs to the
host (a synchronising copy) and raise PkvError before anything is queued if a
precondition fails. Off by default: the copy stalls the stream.
"""
from __future__ import annotations

import os

import numpy as np

_enabled = os.environ.get("PKV_DEBUG_CHECKS", "") not in ("", "0")


def set_debug_checks(on: bool) -> None:
    global _enabled
    _enabled = bool(on)


def debug_checks() -> bool:
    return _enabled


def slot_conflicts(slots, num_slots: int) -> np.ndarray:
    """Slots that two or more valid tokens write (valid: 0 <= slot < num_slots;
    -1 and out-of-range slots are skipped by the kernel). Sorted."""
    s = np.asarray(slots, dtype=np.int64).ravel()
    s = s[(s >= 0) & (s < num_slots)]
    u, counts = np.unique(s, return_counts=True)
    return u[counts > 1]


def pair_conflicts(pairs, num_src_blocks: int, num_dst_blocks: int | None = None) -> list:
    """Indices of copy pairs (src, dst) that race with an earlier or later pair:
    a destination written twice, or a destination that another pair reads.
    Pairs with an id out of range are skipped by the kernel and ignored here.
    num_dst_blocks differs from num_src_blocks when source and destination are
    different pools (swapping), where only duplicate destinations race."""
    p = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    same_pool = num_dst_blocks is None
    nd = num_src_blocks if same_pool else num_dst_blocks
    valid = (p[:, 0] >= 0) & (p[:, 0] < num_src_blocks) & (p[:, 1] >= 0) & (p[:, 1] < nd)
    idx = np.flatnonzero(valid)
    src, dst = p[idx, 0].tolist(), p[idx, 1].tolist()
    n_dst, n_src = {}, {}
    for s, d in zip(src, dst):
        n_dst[d] = n_dst.get(d, 0) + 1
        n_src[s] = n_src.get(s, 0) + 1
    bad = []
    for i, s, d in zip(idx.tolist(), src, dst):
        read_by_other = same_pool and n_src.get(d, 0) - (1 if s == d else 0) > 0
        if n_dst[d] > 1 or read_by_other:
            bad.append(i)
    return bad
