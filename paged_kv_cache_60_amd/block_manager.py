"""Python handle over the C++ block manager (pkv_bm_* in include/pagedkv.h)."""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from . import _lib
from ._lib import PkvError, check


@dataclass
class AppendResult:
    slots: list
    cow_src: int
    cow_dst: int


def _i32p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _i64p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


class BlockManager:
    """FIFO pool of physical blocks, block tables, refcounts and a prefix cache of
    full blocks (host, C++)."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        lib = _lib.load_block_manager()
        self._lib = lib
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        h = ctypes.c_void_p()
        if free_order is None:
            st = lib.pkv_bm_create(self.num_blocks, self.block_size, None, ctypes.byref(h))
        else:
            order = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
            if order.shape != (self.num_blocks,):
                raise PkvError(_lib.PKV_ERR_INVALID, "pkv_bm_create")
            st = lib.pkv_bm_create(self.num_blocks, self.block_size, _i32p(order), ctypes.byref(h))
        check(st, "pkv_bm_create")
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001
            pass

    # ------------------------------------------------------------ operations
    def allocate(self, seq: int, num_tokens: int) -> list:
        slots = np.empty(max(num_tokens, 0), dtype=np.int64)
        check(self._lib.pkv_bm_allocate(self._h, seq, num_tokens, _i64p(slots) if num_tokens > 0 else None),
              "pkv_bm_allocate")
        return slots.tolist()

    def allocate_np(self, seq: int, num_tokens: int) -> np.ndarray:
        slots = np.empty(max(num_tokens, 0), dtype=np.int64)
        check(self._lib.pkv_bm_allocate(self._h, seq, num_tokens, _i64p(slots) if num_tokens > 0 else None),
              "pkv_bm_allocate")
        return slots

    def allocate_prompt(self, seq: int, tokens) -> tuple:
        """New sequence for a prompt of token ids, reusing cached blocks.
        Returns (cached tokens, slots of the remaining tokens as an int64 array)."""
        toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
        n = len(toks)
        slots = np.empty(max(n, 1), dtype=np.int64)
        c = ctypes.c_int(0)
        check(self._lib.pkv_bm_allocate_prompt(self._h, seq, _i32p(toks) if n else None, n, ctypes.byref(c),
                                               _i64p(slots) if n else None), "pkv_bm_allocate_prompt")
        return c.value, slots[:n - c.value]

    def append(self, seq: int, n: int = 1) -> AppendResult:
        slots = np.empty(max(n, 0), dtype=np.int64)
        cs = ctypes.c_int32(-1)
        cd = ctypes.c_int32(-1)
        check(self._lib.pkv_bm_append(self._h, seq, n, _i64p(slots) if n > 0 else None,
                                      ctypes.byref(cs), ctypes.byref(cd)), "pkv_bm_append")
        return AppendResult(slots.tolist(), cs.value, cd.value)

    def append_batch(self, seqs: np.ndarray, slot_out: np.ndarray, cow_out: np.ndarray) -> int:
        """One token for each sequence; fills slot_out[n] and cow_out[2n]; returns #pairs."""
        n = ctypes.c_int(0)
        check(self._lib.pkv_bm_append_batch(self._h, _i64p(seqs), len(seqs), _i64p(slot_out),
                                            _i32p(cow_out), ctypes.byref(n)), "pkv_bm_append_batch")
        return n.value

    def decode_step(self, seqs: np.ndarray, slot_out: np.ndarray, cow_out: np.ndarray,
                    upd_out: np.ndarray, ctx_out: np.ndarray, max_blocks: int):
        """One token per sequence plus the block-table updates; returns (#pairs, #updates).
        Raises (state unchanged) if a table would need more than max_blocks entries."""
        n_cow = ctypes.c_int(0)
        n_upd = ctypes.c_int(0)
        check(self._lib.pkv_bm_decode_step(self._h, _i64p(seqs), len(seqs), _i64p(slot_out), _i32p(cow_out),
                                           ctypes.byref(n_cow), _i32p(upd_out), ctypes.byref(n_upd),
                                           _i32p(ctx_out), int(max_blocks)), "pkv_bm_decode_step")
        return n_cow.value, n_upd.value

    def fork(self, parent: int, child: int) -> None:
        check(self._lib.pkv_bm_fork(self._h, parent, child), "pkv_bm_fork")

    def share_prefix(self, src: int, num_blocks: int, dst: int) -> None:
        check(self._lib.pkv_bm_share_prefix(self._h, src, num_blocks, dst), "pkv_bm_share_prefix")

    def free_seq(self, seq: int) -> None:
        check(self._lib.pkv_bm_free(self._h, seq), "pkv_bm_free")

    # ------------------------------------------------------------ preemption and swapping
    def set_host_blocks(self, n: int) -> None:
        check(self._lib.pkv_bm_set_host_blocks(self._h, n), "pkv_bm_set_host_blocks")
        self.num_host_blocks = int(n)

    def _pairs_call(self, fn, where, seqs) -> list:
        ids = np.ascontiguousarray(np.asarray(list(seqs), dtype=np.int64))
        cap = max(1, self.num_blocks + getattr(self, "num_host_blocks", 0))
        out = np.empty(2 * cap, dtype=np.int32)
        n = ctypes.c_int(0)
        check(fn(self._h, _i64p(ids) if len(ids) else None, len(ids), _i32p(out), cap, ctypes.byref(n)), where)
        return [(int(out[2 * i]), int(out[2 * i + 1])) for i in range(n.value)]

    def swap_out(self, seqs) -> list:
        """Swap a group out; returns (device block, host block) pairs to copy."""
        return self._pairs_call(self._lib.pkv_bm_swap_out, "pkv_bm_swap_out", seqs)

    def swap_in(self, seqs) -> list:
        """Swap a group back in; returns (host block, device block) pairs to copy."""
        return self._pairs_call(self._lib.pkv_bm_swap_in, "pkv_bm_swap_in", seqs)

    def preempt_tail(self, running, need: int, mode: str = "recompute"):
        """Preempt from the tail of `running` until `need` blocks are available;
        returns (victims, swap pairs)."""
        ids = np.ascontiguousarray(np.asarray(list(running), dtype=np.int64))
        victims = np.empty(max(1, len(ids)), dtype=np.int64)
        cap = max(1, self.num_blocks)
        pairs = np.empty(2 * cap, dtype=np.int32)
        nv, npairs = ctypes.c_int(0), ctypes.c_int(0)
        m = _lib.PREEMPT_SWAP if mode == "swap" else _lib.PREEMPT_RECOMPUTE
        if mode not in ("swap", "recompute"):
            m = -1
        check(self._lib.pkv_bm_preempt_tail(self._h, _i64p(ids) if len(ids) else None, len(ids), int(need), m,
                                            _i64p(victims), ctypes.byref(nv), _i32p(pairs), cap,
                                            ctypes.byref(npairs)), "pkv_bm_preempt_tail")
        return ([int(v) for v in victims[:nv.value]],
                [(int(pairs[2 * i]), int(pairs[2 * i + 1])) for i in range(npairs.value)])

    def swapped_table(self, seq: int) -> list:
        n = ctypes.c_int(0)
        cap = max(1, getattr(self, "num_host_blocks", 0))
        out = np.empty(cap, dtype=np.int32)
        check(self._lib.pkv_bm_swapped_table(self._h, seq, _i32p(out), cap, ctypes.byref(n)),
              "pkv_bm_swapped_table")
        return out[:n.value].tolist()

    def swapped_tokens(self, seq: int) -> int:
        n = ctypes.c_int(0)
        check(self._lib.pkv_bm_swapped_tokens(self._h, seq, ctypes.byref(n)), "pkv_bm_swapped_tokens")
        return n.value

    def host_free_list(self) -> list:
        cap = max(1, getattr(self, "num_host_blocks", 0))
        out = np.empty(cap, dtype=np.int32)
        n = ctypes.c_int(0)
        check(self._lib.pkv_bm_host_free_list(self._h, _i32p(out), cap, ctypes.byref(n)), "pkv_bm_host_free_list")
        return out[:n.value].tolist()

    def host_refcount(self, h: int) -> int:
        rc = ctypes.c_int(0)
        check(self._lib.pkv_bm_host_refcount(self._h, h, ctypes.byref(rc)), "pkv_bm_host_refcount")
        return rc.value

    # ------------------------------------------------------------ queries
    def slots(self, seq: int, start: int, n: int) -> list:
        out = np.empty(max(n, 0), dtype=np.int64)
        check(self._lib.pkv_bm_slots(self._h, seq, start, n, _i64p(out) if n > 0 else None), "pkv_bm_slots")
        return out.tolist()

    def block_table(self, seq: int) -> list:
        n = ctypes.c_int(0)
        ntok = self.num_tokens(seq)
        cap = max(1, -(-ntok // self.block_size))
        out = np.empty(cap, dtype=np.int32)
        check(self._lib.pkv_bm_block_table(self._h, seq, _i32p(out), cap, ctypes.byref(n)),
              "pkv_bm_block_table")
        return out[:n.value].tolist()

    def num_tokens(self, seq: int) -> int:
        n = ctypes.c_int(0)
        check(self._lib.pkv_bm_num_tokens(self._h, seq, ctypes.byref(n)), "pkv_bm_num_tokens")
        return n.value

    def refcount(self, block: int) -> int:
        rc = ctypes.c_int(0)
        check(self._lib.pkv_bm_refcount(self._h, block, ctypes.byref(rc)), "pkv_bm_refcount")
        return rc.value

    def free_list(self) -> list:
        out = np.empty(self.num_blocks, dtype=np.int32)
        n = ctypes.c_int(0)
        check(self._lib.pkv_bm_free_list(self._h, _i32p(out), self.num_blocks, ctypes.byref(n)),
              "pkv_bm_free_list")
        return out[:n.value].tolist()

    def evictable_list(self) -> list:
        """Cached blocks with no reference, oldest (next to evict) first."""
        out = np.empty(self.num_blocks, dtype=np.int32)
        n = ctypes.c_int(0)
        check(self._lib.pkv_bm_evictable_list(self._h, _i32p(out), self.num_blocks, ctypes.byref(n)),
              "pkv_bm_evictable_list")
        return out[:n.value].tolist()

    def cache_entry(self, block: int):
        """(parent block, token ids) if the block is cached, else None."""
        cached = ctypes.c_int(0)
        parent = ctypes.c_int32(-1)
        toks = np.empty(self.block_size, dtype=np.int32)
        check(self._lib.pkv_bm_cache_entry(self._h, block, ctypes.byref(cached), ctypes.byref(parent),
                                           _i32p(toks)), "pkv_bm_cache_entry")
        return (parent.value, toks.tolist()) if cached.value else None

    def available_blocks(self) -> int:
        """Blocks a new allocation can take: the free queue plus evictable cached blocks."""
        st = self.stats()
        return st["free_blocks"] + st["evictable_blocks"]

    def stats(self) -> dict:
        s = _lib.PkvStats()
        check(self._lib.pkv_bm_stats(self._h, ctypes.byref(s)), "pkv_bm_stats")
        return {
            "free_blocks": s.free_blocks,
            "live_seqs": s.live_seqs,
            "used_blocks": s.used_blocks,
            "utilization": s.utilization,
            "filled_slots": s.filled_slots,
            "slot_utilization": s.slot_utilization,
            "evictable_blocks": s.evictable_blocks,
            "cached_blocks": s.cached_blocks,
            "prefix_query_tokens": s.prefix_query_tokens,
            "prefix_hit_tokens": s.prefix_hit_tokens,
            "host_blocks": s.host_blocks,
            "host_free_blocks": s.host_free_blocks,
            "swapped_seqs": s.swapped_seqs,
        }

    def export(self, seqs: np.ndarray, tables_out: np.ndarray, ctx_out: np.ndarray) -> None:
        """Fill tables_out [n, max_blocks] (-1 padded) and ctx_out [n] (int32)."""
        check(self._lib.pkv_bm_export(self._h, _i64p(seqs), len(seqs), _i32p(tables_out),
                                      tables_out.shape[1], _i32p(ctx_out)), "pkv_bm_export")

    def prefix_groups(self, seqs, max_members: int) -> np.ndarray:
        """Runs of the batch that share leading full blocks, as int32 [3, n]:
        first batch index, members, shared tokens of each group (the groups
        paged_attn_decode_shared reads once)."""
        seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        cap = max(1, len(seqs) // 2)
        first = np.empty(cap, dtype=np.int32)
        size = np.empty(cap, dtype=np.int32)
        prefix = np.empty(cap, dtype=np.int32)
        n = ctypes.c_int(0)
        check(self._lib.pkv_bm_prefix_groups(self._h, _i64p(seqs) if len(seqs) else None, len(seqs),
                                             int(max_members), _i32p(first), _i32p(size), _i32p(prefix), cap,
                                             ctypes.byref(n)), "pkv_bm_prefix_groups")
        return np.stack([first[:n.value], size[:n.value], prefix[:n.value]]).astype(np.int32)

    def state(self, seqs, swapped=()) -> dict:
        """Snapshot comparable with the oracle model's state() for the given
        resident and swapped-out ids."""
        tables = {int(s): self.block_table(int(s)) for s in sorted(seqs)}
        counts = {int(s): self.num_tokens(int(s)) for s in sorted(seqs)}
        nh = getattr(self, "num_host_blocks", 0)
        cache = {}
        for b in range(self.num_blocks):
            e = self.cache_entry(b)
            if e is not None:
                cache[b] = e
        return {
            "free": self.free_list(),
            "tables": tables,
            "counts": counts,
            "ref": [self.refcount(b) for b in range(self.num_blocks)],
            "evictable": self.evictable_list(),
            "cache": cache,
            "host_free": self.host_free_list() if nh else [],
            "host_ref": [self.host_refcount(h) for h in range(nh)],
            "host_tables": {int(s): self.swapped_table(int(s)) for s in sorted(swapped)},
            "host_counts": {int(s): self.swapped_tokens(int(s)) for s in sorted(swapped)},
        }
