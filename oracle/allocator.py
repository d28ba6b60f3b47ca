"""Block manager model: the reference semantics of the host allocator. TEST INFRASTRUCTURE.

Sources
  * "From OOM to Smooth Inference (RAG memory management)", §2.3: the Python
    KV cache manager. Free pool is a list popped from the front and extended
    at the back; a pool that is too small raises before anything is popped;
    block count is ceil(tokens / block_size); per-request token count.
  * "Inference Engine Memory Optimisation (KV Cache to Continuous Batching)",
    §3: the block manager with a FIFO queue of free blocks, block tables,
    per-block reference counts, allocate / append-token / free / share-prefix,
    available blocks and utilisation (used / total).
  * "vLLM Architecture and Memory Use, ch. 3", §3.2: sequences forked from one
    parent (beams, parallel samples) share blocks through reference counts; a
    block returns to the pool when its count reaches zero. §3.3: copy-on-write
    allocates a new block, copies the shared block into it, writes the new one
    and decrements the original's count.
  * "From OOM to Smooth Inference", §6.1: forked beams copy only the last block.
  * "Where Did the VRAM Go (KV cache tutorial)", §4.2-4.4: prefix caching. Each
    block gets a key built from its own token ids and everything before it; a
    new request looks its blocks up and maps hits straight into its block
    table, so only the missed part is prefilled; shared blocks carry reference
    counts and a block whose count reaches zero waits for reuse; eviction is
    least-recently-used; matching is exact at token level.

Readings taken where the pages are silent or garbled (each is tested):
  R1  Block ids are 0-based; the initial free order is caller-supplied
      (default ascending).
  R2  allocate() on an existing id is an error (EXISTS); growth goes through
      append(). A 0-token allocate is allowed and holds no block.
  R3  append(n) allocates ceil(count/bs) - len(table) new blocks at once, so
      n > block_size is handled (the Python sample pops only one block).
  R4  The fill of the last block is derived from a per-sequence token count,
      not from a per-block count, so that two sharers of a block never bump
      the same counter.
  R5  Copy-on-write: when an append's first new position lands inside the
      existing last block and that block's refcount is > 1, a fresh block is
      popped first, the old block's refcount drops by one, the table entry is
      replaced and the pair (old, new) is reported for a whole-block copy. A
      full last block is never copied: the next token goes to a new block.
  R6  share_prefix(src, n, dst) fails if n exceeds src's table length (the
      comparison sign was lost in the page's extraction) or dst exists. dst's
      token count is min(n * bs, src's count).
  R7  fork(parent, child) copies the whole table and the token count and adds
      one reference to every block.
  R8  free() walks the table in order; every block whose count reaches zero is
      appended to the back of the free queue.
  R9  A failing call changes no state: every check runs before any mutation.
  R10 Prefix cache. Only full blocks are cached. A block's key is (parent
      block, its bs token ids), parent = the previous block of the same prompt
      or -1: the chain "everything before it" is carried by the parent block,
      whose own key carries its parent, so a match is exact (no hash
      collisions can alias two contents). allocate_prompt(seq, tokens) maps
      the longest run of leading full blocks found in the cache, stops at the
      first miss, takes fresh blocks for the rest and registers every fresh
      full block under its parent. The partial last block is never cached.
  R11 A cached block whose count reaches zero keeps its key and joins the
      evictable list instead of the free queue; a later hit revives it. Fresh
      blocks come from the free queue first; when it is empty the oldest
      evictable block is evicted (its key dropped) and reused. The capacity
      check before any mutation counts free + evictable blocks, minus the
      evictable blocks the same call revives.
  R12 free() releases in table order; uncached blocks reaching zero go to the
      back of the free queue as before (R8), cached ones join the evictable
      list deepest block first. Since every sequence holding a block also
      holds its parent, a block never reaches zero after its parent, so the
      evictable list always holds a block's cached descendants before it and
      eviction removes children before parents (no key can name a parent
      block that was reused for other content).
  * "Where Did the VRAM Go (KV cache tutorial)", §7.1-7.2, and "From OOM to
    Smooth Inference", §5: when no new KV block can be had, running requests
    are preempted from the tail of the running set (the newest first) and
    their blocks released; a preempted request either drops its cache and is
    prefilled again later (recompute) or has its blocks copied to CPU memory
    and back (swap). "vLLM Architecture and Memory Use, ch. 3", §3.4: swap
    space in CPU memory for inactive blocks.
  R13 Host pool. set_host_blocks(n) gives host block ids 0..n-1 in a FIFO
      queue (ascending), allowed while nothing is swapped out.
  R14 swap_out(seqs) moves a group of resident sequences to host blocks. Every
      distinct device block of the group, in order of first appearance (the
      sequences in the order given, each table in order), gets one host block
      from the front of the host queue and one (device, host) pair to copy;
      a block the group's sequences share is copied once and its host block
      counts one reference per sharer. Then each sequence, in order, releases
      its device blocks exactly as free() does and keeps its token count and
      a table of host blocks. A device block still held by a sequence outside
      the group stays resident. Prefix-cache keys do not travel with the data.
  R15 swap_in(seqs) is the reverse: every distinct host block, in order of
      first appearance, gets a fresh device block (free queue, then the oldest
      evictable block) and one (host, device) pair; each sequence in order
      takes its device table and releases its host blocks (a host block whose
      count reaches zero goes to the back of the host queue).
  R16 A swapped-out sequence is not resident: calls that need its blocks on
      the device fail with NO_SEQ, its id stays taken (EXISTS), and free()
      releases its host blocks.
  R17 preempt_tail(running, need, mode) walks the running list from its tail
      (newest first) and picks victims until the blocks a new allocation can
      take (free + evictable) would reach `need`, counting only the device
      blocks each victim would actually release. mode "recompute" frees the
      victims (their requests are prefilled again later); mode "swap" swaps
      them out as one group. If even every listed sequence is not enough (or,
      for swap, the host pool is too small) nothing changes (OOM).
  * "vLLM Architecture and Memory Use, ch. 3", §3.2, and "Where Did the VRAM
    Go", §4.2-4.4: forked sequences and prefix-cache hits hold the same
    physical blocks at the same table positions, so their K/V there is one
    copy in memory.
  R18 prefix_groups(seqs, max_members) finds the runs of a decode batch that
      share leading blocks. Walking the batch in order, a group is a maximal
      run of consecutive entries, at most max_members long, whose first
      table entry is one block that every member holds in full (token count
      >= bs). Its prefix is bs times the number of leading table positions at
      which every member holds the same block, in full. A run of one entry is
      not a group. The result is (first batch index, members, prefix tokens)
      per group, in batch order.
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass

OK = 0
ERR_INVALID = -1
ERR_OOM = -2
ERR_NO_SEQ = -3
ERR_EXISTS = -4


class AllocError(Exception):
    """Raised for a rejected call; ``code`` is one of the ERR_* values."""

    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


@dataclass
class AppendResult:
    slots: list  # flat slot (block * bs + offset) of each appended token
    cow_src: int  # -1 when no copy-on-write happened
    cow_dst: int


class BlockAllocatorModel:
    """Pure-Python model of the paged KV block manager."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        # "From OOM to Smooth Inference", §2.3: sizes must be positive.
        if num_blocks <= 0 or block_size <= 0:
            raise AllocError(ERR_INVALID, "num_blocks and block_size must be positive")
        if free_order is None:
            order = list(range(num_blocks))
        else:
            order = [int(b) for b in free_order]
            if sorted(order) != list(range(num_blocks)):
                raise AllocError(ERR_INVALID, "free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.bs = block_size
        self.free = deque(order)
        self.tables: dict[int, list[int]] = {}
        self.counts: dict[int, int] = {}
        self.ref = [0] * num_blocks
        # prefix cache (R10-R12): key -> block, block -> key, evictable blocks oldest first
        self.cache: dict[tuple, int] = {}
        self.key_of: dict[int, tuple] = {}
        self.evictable: deque = deque()
        self.prefix_query_tokens = 0
        self.prefix_hit_tokens = 0
        # host pool for swapped-out sequences (R13-R16)
        self.num_host_blocks = 0
        self.host_free: deque = deque()
        self.host_ref: list = []
        self.host_tables: dict[int, list[int]] = {}
        self.host_counts: dict[int, int] = {}

    # ----------------------------------------------------------- helpers
    def _needed(self, tokens: int) -> int:
        # ceil(tokens / block_size), "From OOM to Smooth Inference", §2.3
        return (tokens + self.bs - 1) // self.bs

    def _capacity(self) -> int:
        return len(self.free) + len(self.evictable)

    def _pop(self, count: int) -> list[int]:
        """count fresh blocks: the free queue first, then the oldest evictable
        cached blocks, whose keys are dropped (R11)."""
        if self._capacity() < count:
            raise AllocError(ERR_OOM, f"need {count} blocks, {self._capacity()} available")
        out = []
        for _ in range(count):
            if self.free:
                out.append(self.free.popleft())
            else:
                b = self.evictable.popleft()
                del self.cache[self.key_of.pop(b)]
                out.append(b)
        return out

    def _taken(self, seq: int) -> bool:
        return seq in self.tables or seq in self.host_tables

    def _require(self, seq: int):
        if seq not in self.tables:
            raise AllocError(ERR_NO_SEQ, f"sequence {seq} does not exist")

    def _slot(self, table: list[int], pos: int) -> int:
        return table[pos // self.bs] * self.bs + pos % self.bs

    # ----------------------------------------------------------- operations
    def allocate(self, seq: int, num_tokens: int) -> list[int]:
        """New sequence holding num_tokens tokens; returns their slots."""
        if num_tokens < 0:
            raise AllocError(ERR_INVALID, "negative token count")
        if self._taken(seq):
            raise AllocError(ERR_EXISTS, f"sequence {seq} exists")
        blocks = self._pop(self._needed(num_tokens))
        for b in blocks:
            self.ref[b] += 1
        self.tables[seq] = blocks
        self.counts[seq] = num_tokens
        return [self._slot(blocks, p) for p in range(num_tokens)]

    def append(self, seq: int, n: int = 1) -> AppendResult:
        """Add n tokens to seq (R3, R5); returns their slots and any CoW pair."""
        self._require(seq)
        if n < 0:
            raise AllocError(ERR_INVALID, "negative token count")
        table = self.tables[seq]
        count = self.counts[seq]
        if n == 0:
            return AppendResult([], -1, -1)
        cow = bool(table) and count % self.bs != 0 and self.ref[table[-1]] > 1
        grow = self._needed(count + n) - len(table)
        need = grow + (1 if cow else 0)
        if self._capacity() < need:
            raise AllocError(ERR_OOM, f"need {need} blocks, {self._capacity()} available")
        cow_src = cow_dst = -1
        if cow:
            cow_src = table[-1]
            cow_dst = self._pop(1)[0]
            self.ref[cow_src] -= 1
            self.ref[cow_dst] += 1
            table[-1] = cow_dst
        for b in self._pop(grow):
            self.ref[b] += 1
            table.append(b)
        self.counts[seq] = count + n
        return AppendResult([self._slot(table, p) for p in range(count, count + n)], cow_src, cow_dst)

    def fork(self, parent: int, child: int) -> None:
        """child shares every block of parent (R7)."""
        self._require(parent)
        if self._taken(child):
            raise AllocError(ERR_EXISTS, f"sequence {child} exists")
        table = list(self.tables[parent])
        for b in table:
            self.ref[b] += 1
        self.tables[child] = table
        self.counts[child] = self.counts[parent]

    def share_prefix(self, src: int, num_blocks: int, dst: int) -> None:
        """dst's table is src's first num_blocks blocks (R6)."""
        self._require(src)
        if self._taken(dst):
            raise AllocError(ERR_EXISTS, f"sequence {dst} exists")
        table = self.tables[src]
        if num_blocks < 0 or num_blocks > len(table):
            raise AllocError(ERR_INVALID, "more shared blocks than the source holds")
        shared = list(table[:num_blocks])
        for b in shared:
            self.ref[b] += 1
        self.tables[dst] = shared
        self.counts[dst] = min(num_blocks * self.bs, self.counts[src])

    def free_seq(self, seq: int) -> None:
        """Release seq's blocks in table order (R8); cached blocks reaching zero
        join the evictable list deepest first (R12)."""
        if seq in self.host_tables:  # R16: a swapped-out sequence releases its host blocks
            self._release_host(self.host_tables.pop(seq))
            del self.host_counts[seq]
            return
        self._require(seq)
        self._release(self.tables.pop(seq))
        del self.counts[seq]

    def _release(self, table: list) -> None:
        """Drop one reference to every block of a table, in order (R8, R12)."""
        cached = []
        for b in table:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                if b in self.key_of:
                    cached.append(b)
                else:
                    self.free.append(b)
        self.evictable.extend(reversed(cached))

    def allocate_prompt(self, seq: int, tokens) -> tuple[int, list[int]]:
        """New sequence for a prompt of token ids, reusing cached blocks (R10).

        Returns (cached tokens, slots of the tokens after them): the caller
        writes K/V only for those."""
        tokens = [int(t) for t in tokens]
        n = len(tokens)
        if self._taken(seq):
            raise AllocError(ERR_EXISTS, f"sequence {seq} exists")
        bs = self.bs
        matched, parent = [], -1
        for i in range(n // bs):
            key = (parent, tuple(tokens[i * bs:(i + 1) * bs]))
            b = self.cache.get(key)
            if b is None:
                break
            matched.append(b)
            parent = b
        fresh_needed = self._needed(n) - len(matched)
        revived = sum(1 for b in matched if self.ref[b] == 0)
        if self._capacity() - revived < fresh_needed:
            raise AllocError(ERR_OOM, f"need {fresh_needed} blocks, {self._capacity() - revived} available")
        for b in matched:
            if self.ref[b] == 0:
                self.evictable.remove(b)
            self.ref[b] += 1
        fresh = self._pop(fresh_needed)
        for b in fresh:
            self.ref[b] += 1
        table = matched + fresh
        for i in range(len(matched), n // bs):
            key = (parent, tuple(tokens[i * bs:(i + 1) * bs]))
            b = table[i]
            self.cache[key] = b
            self.key_of[b] = key
            parent = b
        self.tables[seq] = table
        self.counts[seq] = n
        n_cached = len(matched) * bs
        self.prefix_query_tokens += n
        self.prefix_hit_tokens += n_cached
        return n_cached, [self._slot(table, p) for p in range(n_cached, n)]

    # ----------------------------------------------------------- swapping (R13-R17)
    def set_host_blocks(self, n: int) -> None:
        if n < 0:
            raise AllocError(ERR_INVALID, "negative host pool")
        if self.host_tables:
            raise AllocError(ERR_INVALID, "sequences are swapped out")
        self.num_host_blocks = n
        self.host_free = deque(range(n))
        self.host_ref = [0] * n

    def _release_host(self, table: list) -> None:
        for h in table:
            self.host_ref[h] -= 1
            if self.host_ref[h] == 0:
                self.host_free.append(h)

    @staticmethod
    def _distinct(tables) -> list:
        seen, out = set(), []
        for t in tables:
            for b in t:
                if b not in seen:
                    seen.add(b)
                    out.append(b)
        return out

    def _group(self, seqs, resident: bool) -> list:
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs):
            raise AllocError(ERR_INVALID, "a sequence is listed twice")
        where = self.tables if resident else self.host_tables
        for s_ in seqs:
            if s_ not in where:
                raise AllocError(ERR_NO_SEQ, f"sequence {s_} is not {'resident' if resident else 'swapped out'}")
        return seqs

    def swap_out(self, seqs) -> list:
        """Move a group of resident sequences to host blocks (R14); returns the
        (device block, host block) pairs to copy, before the released device
        blocks are written again."""
        seqs = self._group(seqs, True)
        blocks = self._distinct(self.tables[s_] for s_ in seqs)
        if len(self.host_free) < len(blocks):
            raise AllocError(ERR_OOM, f"need {len(blocks)} host blocks, {len(self.host_free)} free")
        to_host = {b: self.host_free.popleft() for b in blocks}
        for s_ in seqs:
            table = self.tables.pop(s_)
            host = [to_host[b] for b in table]
            for h in host:
                self.host_ref[h] += 1
            self.host_tables[s_] = host
            self.host_counts[s_] = self.counts.pop(s_)
            self._release(table)
        return [(b, to_host[b]) for b in blocks]

    def swap_in(self, seqs) -> list:
        """Bring a group of swapped-out sequences back (R15); returns the
        (host block, device block) pairs to copy before the group is used."""
        seqs = self._group(seqs, False)
        hosts = self._distinct(self.host_tables[s_] for s_ in seqs)
        if self._capacity() < len(hosts):
            raise AllocError(ERR_OOM, f"need {len(hosts)} blocks, {self._capacity()} available")
        fresh = self._pop(len(hosts))
        to_dev = dict(zip(hosts, fresh))
        for s_ in seqs:
            host = self.host_tables.pop(s_)
            table = [to_dev[h] for h in host]
            for b in table:
                self.ref[b] += 1
            self.tables[s_] = table
            self.counts[s_] = self.host_counts.pop(s_)
            self._release_host(host)
        return [(h, to_dev[h]) for h in hosts]

    def preempt_tail(self, running, need: int, mode: str = "recompute"):
        """Preempt from the tail of the running list until `need` blocks are
        available (R17); returns (victims in preemption order, swap pairs)."""
        running = [int(s_) for s_ in running]
        if mode not in ("recompute", "swap") or need < 0:
            raise AllocError(ERR_INVALID, "bad preemption request")
        if len(set(running)) != len(running):
            raise AllocError(ERR_INVALID, "a sequence is listed twice")
        for s_ in running:
            self._require(s_)
        ref = list(self.ref)
        avail = self._capacity()
        victims = []
        for s_ in reversed(running):
            if avail >= need:
                break
            victims.append(s_)
            for b in self.tables[s_]:
                ref[b] -= 1
                if ref[b] == 0:
                    avail += 1
        if avail < need:
            raise AllocError(ERR_OOM, f"need {need} blocks, {avail} even after preempting every listed sequence")
        if mode == "swap":
            return victims, self.swap_out(victims)
        for s_ in victims:
            self.free_seq(s_)
        return victims, []

    def swapped_table(self, seq: int) -> list:
        if seq not in self.host_tables:
            raise AllocError(ERR_NO_SEQ, f"sequence {seq} is not swapped out")
        return list(self.host_tables[seq])

    def host_free_list(self) -> list:
        return list(self.host_free)

    # ----------------------------------------------------------- queries
    def prefix_groups(self, seqs, max_members: int) -> list:
        """Runs of the batch that share leading full blocks (R18)."""
        seqs = [int(s_) for s_ in seqs]
        if max_members < 1:
            raise AllocError(ERR_INVALID, "max_members must be positive")
        for s_ in seqs:
            self._require(s_)

        def full_first(s_):
            return self.tables[s_][0] if self.counts[s_] >= self.bs else None

        groups = []
        i = 0
        while i < len(seqs):
            head = full_first(seqs[i])
            j = i + 1
            if head is not None:
                while j < len(seqs) and j - i < max_members and full_first(seqs[j]) == head:
                    j += 1
            if j - i >= 2:
                members = seqs[i:j]
                n = 0
                while all((n + 1) * self.bs <= self.counts[m] and self.tables[m][n] == self.tables[members[0]][n]
                          for m in members):
                    n += 1
                groups.append((i, j - i, n * self.bs))
            i = j
        return groups

    def slots(self, seq: int, start: int, n: int) -> list[int]:
        self._require(seq)
        if start < 0 or n < 0 or start + n > self.counts[seq]:
            raise AllocError(ERR_INVALID, "positions out of range")
        t = self.tables[seq]
        return [self._slot(t, p) for p in range(start, start + n)]

    def block_table(self, seq: int) -> list[int]:
        self._require(seq)
        return list(self.tables[seq])

    def num_tokens(self, seq: int) -> int:
        self._require(seq)
        return self.counts[seq]

    def refcount(self, block: int) -> int:
        if block < 0 or block >= self.num_blocks:
            raise AllocError(ERR_INVALID, "block id out of range")
        return self.ref[block]

    def free_list(self) -> list[int]:
        return list(self.free)

    def evictable_list(self) -> list[int]:
        """Cached blocks with no reference, oldest (next to evict) first."""
        return list(self.evictable)

    def cache_entry(self, block: int):
        """(parent block, token ids) if the block is cached, else None."""
        if block < 0 or block >= self.num_blocks:
            raise AllocError(ERR_INVALID, "block id out of range")
        key = self.key_of.get(block)
        return None if key is None else (key[0], list(key[1]))

    def available_blocks(self) -> int:
        """Blocks a new allocation can take: free plus evictable cached blocks."""
        return self._capacity()

    def utilization(self) -> float:
        """Blocks referenced by live sequences / total: the second page's
        (total - free) / total, with evictable cached blocks counted as free."""
        return (self.num_blocks - self._capacity()) / self.num_blocks

    def stats(self) -> dict:
        """Free blocks, live sequences, used blocks, physical utilisation,
        filled slots and slot utilisation.

        A used block's filled slots are the largest fill any sequence that
        references it sees in it, so a shared block counts its tokens once.
        """
        filled: dict[int, int] = {}
        for seq, table in self.tables.items():
            c = self.counts[seq]
            for i, b in enumerate(table):
                f = max(0, min(self.bs, c - i * self.bs))
                filled[b] = max(filled.get(b, 0), f)
        used = self.num_blocks - self._capacity()
        total_filled = sum(filled.values())
        return {
            "free_blocks": len(self.free),
            "live_seqs": len(self.tables),
            "used_blocks": used,
            "utilization": used / self.num_blocks,
            "filled_slots": total_filled,
            "slot_utilization": (total_filled / (used * self.bs)) if used else 0.0,
            "evictable_blocks": len(self.evictable),
            "cached_blocks": len(self.key_of),
            "prefix_query_tokens": self.prefix_query_tokens,
            "prefix_hit_tokens": self.prefix_hit_tokens,
            "host_blocks": self.num_host_blocks,
            "host_free_blocks": len(self.host_free),
            "swapped_seqs": len(self.host_tables),
        }

    def state(self) -> dict:
        """Full state snapshot for bit-exact comparison."""
        return {
            "free": list(self.free),
            "tables": {s: list(t) for s, t in sorted(self.tables.items())},
            "counts": dict(sorted(self.counts.items())),
            "ref": list(self.ref),
            "evictable": list(self.evictable),
            "cache": {b: (k[0], list(k[1])) for b, k in sorted(self.key_of.items())},
            "host_free": list(self.host_free),
            "host_ref": list(self.host_ref),
            "host_tables": {s_: list(t) for s_, t in sorted(self.host_tables.items())},
            "host_counts": dict(sorted(self.host_counts.items())),
        }
