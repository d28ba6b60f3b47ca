"""Paged KV cache on one GPU: device caches plus the host block manager.

One decode step, as the pages run it ("From OOM to Smooth Inference (RAG
memory management)", §2.3: allocate, append per generated token, release;
"vLLM Architecture and Memory Use, ch. 3", §3.2-3.3: sharing and
copy-on-write):

  1. host bookkeeping: append one token to every sequence of the batch
     (one C call); new blocks come from the FIFO pool; a write into a shared,
     partially filled last block triggers copy-on-write;
  2. the step's metadata (slot mapping, context lengths, copy pairs and the
     block-table entries that changed) stays in a pinned host buffer that the
     kernels read directly; the block tables themselves stay resident on the
     device and only their changed entries are written;
  3. paged_block_copy for the copy-on-write pairs, if any;
  4. paged_kv_write_step: the new tokens' K/V plus the step's context lengths
     and table entries, in one kernel;
  5. paged_attn_decode (pass 1 over equal shares of the KV, pass 2 for split segments).

Pinned metadata buffers form a ring of RING slots, so the host can prepare
the next steps while earlier steps' kernels are still queued. Before the host
overwrites a slot it waits for an event recorded after the step that last
read it. An event in the stream idles the GPU for a few microseconds (about
5.7 us between the step's last kernel and the next step's first, measured on
MI355X), so one event covers EVENT_EVERY steps and is recorded after the
step's last kernel, never between its kernels.
"""
from __future__ import annotations

import numpy as np
import torch

from . import ops
from .block_manager import BlockManager

F16_NAN_BITS = 0x7E00
FP8_NAN_BITS = 0x7F
RING = 32         # pinned metadata slots
EVENT_EVERY = 16  # steps covered by one completion event; RING is a multiple of it


class PagedKVEngine:
    def __init__(self, num_blocks, num_q_heads, num_kv_heads, head_dim, block_size, kv_dtype="f16",
                 free_order=None, k_scale=1.0, v_scale=1.0, k_inv_scale=1.0, v_inv_scale=1.0,
                 device="cuda", poison=True, num_host_blocks=0):
        self.num_blocks = int(num_blocks)
        self.hq, self.hkv, self.d, self.bs = int(num_q_heads), int(num_kv_heads), int(head_dim), int(block_size)
        self.kv_dtype = kv_dtype
        self.device = torch.device(device)
        # fp8 scales: one per tensor (numbers) or one per KV head (float32 device tensors)
        self.k_scale, self.v_scale, self.k_inv_scale, self.v_inv_scale = (
            self._scale(x) for x in (k_scale, v_scale, k_inv_scale, v_inv_scale))
        self.bm = BlockManager(self.num_blocks, self.bs, free_order)
        shape = (self.num_blocks, self.hkv, self.bs, self.d)
        dt = ops.cache_torch_dtype(kv_dtype)
        self.k_cache = torch.empty(shape, dtype=dt, device=self.device)
        self.v_cache = torch.empty(shape, dtype=dt, device=self.device)
        # host pool for swapped-out sequences: pinned, same layout, read and
        # written by paged_block_swap directly
        self.num_host_blocks = int(num_host_blocks)
        self.k_host = self.v_host = None
        if self.num_host_blocks:
            hshape = (self.num_host_blocks, self.hkv, self.bs, self.d)
            self.k_host = torch.empty(hshape, dtype=dt, pin_memory=True)
            self.v_host = torch.empty(hshape, dtype=dt, pin_memory=True)
            self.bm.set_host_blocks(self.num_host_blocks)
        if poison:
            self.poison()

    def _scale(self, x):
        a = np.asarray(x)
        if a.ndim == 0:
            return float(a)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(self.device)

    @property
    def block_bytes(self) -> int:
        return self.k_cache[0].numel() * self.k_cache.element_size()

    def poison(self):
        """Fill every slot with a NaN bit pattern (unused slots must never be read)."""
        if self.kv_dtype == "f16":
            for c in (self.k_cache, self.v_cache):
                c.view(torch.int16).fill_(F16_NAN_BITS)
        else:
            for c in (self.k_cache, self.v_cache):
                c.fill_(FP8_NAN_BITS)

    # ------------------------------------------------------ scripted rounds
    def apply_ops(self, ops_list):
        """Run block-manager ops in order; returns (slots int64 array of the
        allocate / append ops, cow pairs list, prompts list, swaps list). A
        prompt op goes through the prefix cache; its entry is (op, cached
        tokens, slots of the tokens after them), the ones whose K/V must still
        be written. A swap entry is ("out" | "in", pairs), in op order."""
        slots, pairs, prompts, swaps = [], [], [], []
        bm = self.bm
        for op in ops_list:
            if op.kind == "allocate":
                slots.append(bm.allocate_np(op.seq, op.n))
            elif op.kind == "append":
                r = bm.append(op.seq, op.n)
                slots.append(np.asarray(r.slots, dtype=np.int64))
                if r.cow_src >= 0:
                    pairs.append((r.cow_src, r.cow_dst))
            elif op.kind == "share_prefix":
                bm.share_prefix(op.src, op.n, op.seq)
            elif op.kind == "fork":
                bm.fork(op.src, op.seq)
            elif op.kind == "free":
                bm.free_seq(op.seq)
            elif op.kind == "prompt":
                c, sl = bm.allocate_prompt(op.seq, op.tokens)
                prompts.append((op, c, sl))
            elif op.kind == "swap_out":
                swaps.append(("out", bm.swap_out(op.group)))
            elif op.kind == "swap_in":
                swaps.append(("in", bm.swap_in(op.group)))
            elif op.kind == "preempt":
                _, sp = bm.preempt_tail(op.group, op.n, op.mode)
                if sp:
                    swaps.append(("out", sp))
            else:
                raise ValueError(op.kind)
        s = np.concatenate(slots) if slots else np.zeros(0, dtype=np.int64)
        return s, pairs, prompts, swaps

    def swap(self, direction, pairs):
        """Copy swapped blocks: "out" (device, host) pairs, "in" (host, device)."""
        if pairs:
            p = torch.tensor(pairs, dtype=torch.int32).to(self.device, non_blocking=False)
            ops.paged_block_swap(self.k_cache, self.v_cache, self.k_host, self.v_host, p, direction)

    def copy_blocks(self, pairs):
        if pairs:
            p = torch.tensor(pairs, dtype=torch.int32).to(self.device, non_blocking=False)
            ops.paged_block_copy(self.k_cache, self.v_cache, p)

    def write(self, slots, K, V):
        """Write host K/V [T, Hkv, D] fp16 (numpy or torch) at host slots [T]."""
        if len(slots) == 0:
            return
        kt = torch.as_tensor(K).to(self.device, non_blocking=False)
        vt = torch.as_tensor(V).to(self.device, non_blocking=False)
        st = torch.as_tensor(np.ascontiguousarray(slots, dtype=np.int64)).to(self.device)
        ops.paged_kv_write(kt, vt, self.k_cache, self.v_cache, st, self.kv_dtype,
                           self.k_inv_scale, self.v_inv_scale)

    # ------------------------------------------------------ decode steps
    def prepare_steps(self, batch_seqs, max_blocks, partition_tokens=0, shared_prefix=None):
        """Set up a decode batch: device-resident block tables (uploaded once
        here), the per-step metadata buffers (two pinned halves on the host,
        one set on the device) and the attention workspace. shared_prefix:
        find the runs of the batch that share leading full blocks (forked
        beams, common prefixes) and attend with paged_attn_decode_shared,
        which reads those blocks once per run; decode steps only append, so
        the runs stay valid until the batch is set up again. None (default):
        do so when the block manager finds a run of two or more sequences
        sharing at least one 32-token unit; True / False force either call.
        Without runs, a batch whose sequences hold no block in common attends
        through paged_attn_decode_shared with no groups, which declares that
        (paged_attn_decode's bits, its waves ordered for disjoint blocks)."""
        torch.cuda.synchronize(self.device)  # queued kernels may still read the previous buffers
        B = len(batch_seqs)
        self.batch = np.ascontiguousarray(np.asarray(batch_seqs, dtype=np.int64))
        self.max_blocks = int(max_blocks)
        self.partition_tokens = int(partition_tokens)
        # pinned layout (bytes): slots int64[B] | ctx int32[B] | cow int32[2B] | updates int32[3B]
        o_slots = 0
        o_ctx = o_slots + 8 * B
        o_cow = o_ctx + 4 * B
        o_upd = o_cow + 8 * B
        total = (o_upd + 12 * B + 255) // 256 * 256
        self._layout = (o_slots, o_ctx, o_cow, o_upd)
        self._pinned = [torch.empty(max(total, 256), dtype=torch.uint8, pin_memory=True) for _ in range(RING)]
        self._views = []
        for t in self._pinned:
            self._views.append((t[o_slots:o_ctx].view(torch.int64), t[o_ctx:o_cow].view(torch.int32),
                                t[o_cow:o_upd].view(torch.int32), t[o_upd:o_upd + 12 * B].view(torch.int32)))
        self._events = [None] * (RING // EVENT_EVERY)
        self._host_steps = 0
        self._device_steps = 0
        self.slots_dev = torch.empty(B, dtype=torch.int64, device=self.device)
        self.ctx_dev = torch.empty(B, dtype=torch.int32, device=self.device)
        self.cow_dev = torch.empty((B, 2), dtype=torch.int32, device=self.device)
        tab, ctx = self.host_tables()
        self.tables_dev = torch.from_numpy(tab).to(self.device)
        self.ctx_dev.copy_(torch.from_numpy(ctx))
        self.groups = None
        self.disjoint = None
        if shared_prefix is None:
            shared_prefix = B <= ops.SHARED_MAX_SEQS and self._sharing_found()
        if shared_prefix:
            g = self.bm.prefix_groups(self.batch, ops.SHARED_COLUMNS // (self.hq // self.hkv))
            self.groups = torch.from_numpy(np.ascontiguousarray(g)).to(self.device)
            wsb = ops.shared_workspace_bytes(B, self.hq, self.hkv, self.d)
        else:
            wsb = ops.workspace_bytes(B, self.hq, self.hkv, self.d, self.max_blocks, self.bs, self.partition_tokens)
            if 0 < B <= ops.SHARED_MAX_SEQS and self._blocks_disjoint(tab, ctx):
                # no block is read by two sequences: paged_attn_decode_shared
                # with no groups declares that, and orders the waves for it;
                # steps keep it true (appends take fresh blocks, and a
                # copy-on-write gives the writer a fresh one)
                self.disjoint = torch.empty((3, 0), dtype=torch.int32, device=self.device)
                wsb = max(wsb, ops.shared_workspace_bytes(B, self.hq, self.hkv, self.d))
        self.workspace = torch.empty(max(wsb, 4), dtype=torch.uint8, device=self.device)
        torch.cuda.synchronize(self.device)

    def _blocks_disjoint(self, tab, ctx) -> bool:
        """Whether no block of the batch's tables (the entries its context
        lengths reach) is held by two of its sequences."""
        n = (ctx.astype(np.int64) + self.bs - 1) // self.bs
        used = tab[np.arange(tab.shape[1])[None, :] < n[:, None]]
        return np.unique(used).size == used.size

    def _sharing_found(self) -> bool:
        """Whether the batch holds a run of sequences sharing leading blocks
        worth reading once (two or more members, 32 or more shared tokens)."""
        g = self.bm.prefix_groups(self.batch, ops.SHARED_COLUMNS // (self.hq // self.hkv))
        return bool(((g[1] >= 2) & (g[2] >= 32)).any()) if g.shape[1] else False

    def host_step(self):
        """Step part 1: host bookkeeping into the next pinned slot.
        Returns (slot, n_cow, n_updates)."""
        k = self._host_steps
        self._host_steps += 1
        slot = k % RING
        if k >= RING:
            # the event of the group holding step k - RING, the slot's last reader
            ev = self._events[((k - RING) // EVENT_EVERY) % len(self._events)]
            ev.synchronize()
        slots, ctx, cow, upd = (v.numpy() for v in self._views[slot])
        n_cow, n_upd = self.bm.decode_step(self.batch, slots, cow, upd, ctx, self.max_blocks)
        return slot, n_cow, n_upd

    def _end_device_step(self):
        """Called after a step's last kernel: every EVENT_EVERY steps, record the
        event that releases the pinned slots of that group of steps."""
        k = self._device_steps
        self._device_steps += 1
        if k % EVENT_EVERY == EVENT_EVERY - 1:
            ev = torch.cuda.Event()
            ev.record()
            self._events[(k // EVENT_EVERY) % len(self._events)] = ev

    def upload(self, slot, n_cow, n_upd):
        """Step part 2 on its own: one small kernel reads the pinned slot and
        updates the device slot mapping, context lengths, copy pairs and table
        entries (paged_step_metadata). device_step() does this inside the write
        kernel instead; this form serves callers that write tokens separately
        (it ends the step for the slot ring)."""
        slots, ctx, cow, upd = self._views[slot]
        ops.paged_step_metadata(slots, self.slots_dev, ctx, self.ctx_dev, len(self.batch), cow,
                                self.cow_dev, n_cow, upd, n_upd, self.tables_dev)
        self._end_device_step()

    def device_step(self, slot, n_cow, n_upd, k_new, v_new, q, out, passes=3, between=None):
        """Step parts 2-5 on the current stream: copy-on-write copies (pairs read
        from the pinned slot), then one kernel that writes the new tokens and
        applies the step's metadata, then attention. `between` (optional) is
        called after the write, before attention, and again between the passes."""
        if n_cow:
            cow = self._views[slot][2]
            ops.paged_block_copy(self.k_cache, self.v_cache, cow[:2 * n_cow].view(n_cow, 2))
        self.write_step(slot, n_upd, k_new, v_new)
        self.last_step = (slot, n_cow, n_upd)
        if between is None:
            self.attend(q, out, passes)
        else:
            between(0)
            self.attend(q, out, 1)
            between(1)
            self.attend(q, out, 2)
        self._end_device_step()

    def write_step(self, slot, n_upd, k_new, v_new):
        """The write kernel of a step: new K/V rows to their slots, plus the
        step's context lengths and block-table entries, all read from pinned
        slot `slot`. Applying it twice is harmless (same values, same places)."""
        slots, ctx, _, upd = self._views[slot]
        ops.paged_kv_write_step(k_new, v_new, self.k_cache, self.v_cache, slots, ctx, self.ctx_dev, upd,
                                n_upd, self.tables_dev, self.kv_dtype, self.k_inv_scale, self.v_inv_scale)

    def attend(self, q, out, passes=3):
        """Attention of the step; passes: 1 = pass 1 (with the shared-prefix
        pass when groups are set), 2 = pass 2 (the merge), 3 = both."""
        sm_scale = 1.0 / float(self.d) ** 0.5
        groups = self.groups if self.groups is not None else self.disjoint
        if groups is not None:
            bits = (3 if passes & 1 else 0) | (4 if passes & 2 else 0)
            ops.paged_attn_decode_shared(out, q, self.k_cache, self.v_cache, self.tables_dev, self.ctx_dev,
                                         groups, sm_scale, self.kv_dtype, self.k_scale, self.v_scale,
                                         self.partition_tokens, self.workspace, bits)
            return
        ops.paged_attn_decode(out, q, self.k_cache, self.v_cache, self.tables_dev, self.ctx_dev, sm_scale,
                              self.kv_dtype, self.k_scale, self.v_scale, self.partition_tokens, self.workspace,
                              passes)

    def decode_step(self, k_new, v_new, q, out):
        """Full decode step: append one token per batch sequence, write it, attend."""
        slot, n_cow, n_upd = self.host_step()
        self.device_step(slot, n_cow, n_upd, k_new, v_new, q, out)
        return n_cow

    # ------------------------------------------------------ prefill
    def prepare_prefill(self, batch_seqs, max_blocks):
        """Device block tables and context lengths of a prefill batch, read
        from the block manager (each sequence's chunk K/V must be written)."""
        B = len(batch_seqs)
        seqs = np.ascontiguousarray(np.asarray(batch_seqs, dtype=np.int64))
        tab = np.empty((B, int(max_blocks)), dtype=np.int32)
        ctx = np.empty(B, dtype=np.int32)
        self.bm.export(seqs, tab, ctx)
        return torch.from_numpy(tab).to(self.device), torch.from_numpy(ctx).to(self.device)

    def prefill(self, tables_dev, ctx_dev, q, q_start_dev, out):
        """Chunked causal prefill attention for the batch (paged_attn_prefill)."""
        ops.paged_attn_prefill(out, q, self.k_cache, self.v_cache, tables_dev, ctx_dev, q_start_dev,
                               1.0 / float(self.d) ** 0.5, self.kv_dtype, self.k_scale, self.v_scale)

    def host_tables(self):
        """(tables [B, maxb], ctx [B]) of the current batch, read back from the manager."""
        B = len(self.batch)
        tab = np.empty((B, self.max_blocks), dtype=np.int32)
        ctx = np.empty(B, dtype=np.int32)
        self.bm.export(self.batch, tab, ctx)
        return tab, ctx
