"""Drive a workload script through the oracle. TEST INFRASTRUCTURE.

One round = apply its block-manager operations in order, copy every
copy-on-write pair the round produced, then write the round's new tokens at
their slots. This is the lifecycle of "From OOM to Smooth Inference (RAG
memory management)", §2.3 (allocate, append, release) with the sharing and
copy-on-write of "vLLM Architecture and Memory Use, ch. 3", §3.2-3.3.
A decode step is one such round (one appended token per sequence) followed by
decode attention over the batch. A prefill run is the setup rounds followed by
causal attention for each sequence's chunk of query rows.

Unused cache slots start as a NaN bit pattern (0x7E00 for float16, 0x7F for
e4m3fn) so that a kernel reading past a sequence's tokens shows up.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from contextlib import nullcontext
from dataclasses import dataclass, field

import numpy as np

from .allocator import BlockAllocatorModel
from .attention import decode_attention
from .cache_ops import block_copy, block_swap, scatter
from .prefill import prefill_attention

F16_NAN_BITS = 0x7E00
FP8_NAN_BITS = 0x7F


def empty_cache(num_blocks, num_kv_heads, block_size, head_dim, kv_dtype):
    shape = (num_blocks, num_kv_heads, block_size, head_dim)
    if kv_dtype != "f16":  # 0x7F is a NaN in both e4m3fn and e5m2
        return np.full(shape, FP8_NAN_BITS, dtype=np.uint8)
    return np.full(shape, F16_NAN_BITS, dtype=np.uint16).view(np.float16)


@dataclass
class RoundResult:
    slots: list
    cow_pairs: list
    prompts: list = field(default_factory=list)  # (op, cached tokens, slots of the other tokens)
    swaps: list = field(default_factory=list)    # ("out" | "in", pairs), in op order


@dataclass
class OracleRun:
    alloc: BlockAllocatorModel
    k_cache: np.ndarray
    v_cache: np.ndarray
    outputs: list = field(default_factory=list)  # per decode step, [B, Hq, D] float64
    tables: list = field(default_factory=list)  # per decode step, list of tables
    ctx_lens: list = field(default_factory=list)  # per decode step
    rounds: list = field(default_factory=list)  # RoundResult per applied round


def apply_ops(alloc: BlockAllocatorModel, ops) -> RoundResult:
    slots, pairs, prompts, swaps = [], [], [], []
    for op in ops:
        if op.kind == "allocate":
            slots += alloc.allocate(op.seq, op.n)
        elif op.kind == "append":
            r = alloc.append(op.seq, op.n)
            slots += r.slots
            if r.cow_src >= 0:
                pairs.append((r.cow_src, r.cow_dst))
        elif op.kind == "share_prefix":
            alloc.share_prefix(op.src, op.n, op.seq)
        elif op.kind == "fork":
            alloc.fork(op.src, op.seq)
        elif op.kind == "free":
            alloc.free_seq(op.seq)
        elif op.kind == "prompt":
            # prefix cache ("Where Did the VRAM Go (KV cache tutorial)", §4.2): only
            # the tokens after the cached blocks are written
            c, sl = alloc.allocate_prompt(op.seq, op.tokens)
            prompts.append((op, c, list(sl)))
        elif op.kind == "swap_out":
            swaps.append(("out", alloc.swap_out(op.group)))
        elif op.kind == "swap_in":
            swaps.append(("in", alloc.swap_in(op.group)))
        elif op.kind == "preempt":
            # "Where Did the VRAM Go (KV cache tutorial)", §7.1: newest first
            _, sp = alloc.preempt_tail(op.group, op.n, op.mode)
            if sp:
                swaps.append(("out", sp))
        else:
            raise ValueError(op.kind)
    return RoundResult(slots, pairs, prompts, swaps)


def run_round(wl, alloc, k_cache, v_cache, ops, host=None) -> RoundResult:
    """One round: the ops, then their swap copies (in op order, before any
    write can reuse a released block), copy-on-write copies, then writes.
    host = (k_host, v_host) caches of the host pool, if the script swaps."""
    res = apply_ops(alloc, ops)
    for direction, sp in res.swaps:
        if direction == "out":
            block_swap(k_cache, v_cache, host[0], host[1], sp)
        else:
            block_swap(host[0], host[1], k_cache, v_cache, sp)
    block_copy(k_cache, v_cache, res.cow_pairs)
    K, V = wl.round_kv(ops)
    scatter(k_cache, v_cache, K, V, res.slots, wl.block_size, wl.kv_dtype,
            wl.k_inv_scale, wl.v_inv_scale)
    for op, c, sl in res.prompts:
        K, V = wl.prompt_kv(op, c)
        scatter(k_cache, v_cache, K, V, sl, wl.block_size, wl.kv_dtype, wl.k_inv_scale, wl.v_inv_scale)
    return res


def _host_pool(wl, alloc):
    """Host caches for the script's swap space (None when it has none)."""
    n = getattr(wl, "num_host_blocks", 0)
    if not n:
        return None
    alloc.set_host_blocks(n)
    return (empty_cache(n, wl.num_kv_heads, wl.block_size, wl.head_dim, wl.kv_dtype),
            empty_cache(n, wl.num_kv_heads, wl.block_size, wl.head_dim, wl.kv_dtype))


def _blas_one_thread():
    """Keep BLAS to one thread while sequences are spread over Python threads."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover - threadpoolctl ships with scikit-learn
        return nullcontext()
    return threadpool_limits(1)


def per_sequence(fn, seqs, threads: int):
    """Call fn(s) for every s in seqs, on `threads` threads when threads > 1.

    Sequences are independent (each reads the caches and writes its own output
    rows), so spreading them over threads changes no arithmetic: every
    sequence's result is the same call as in a serial loop."""
    seqs = list(seqs)
    if threads <= 1 or len(seqs) <= 1:
        for s in seqs:
            fn(s)
        return
    with _blas_one_thread(), ThreadPoolExecutor(max_workers=threads) as ex:
        for _ in ex.map(fn, seqs):
            pass


def _decode_step(wl, step, kc, vc, tables, lens, seqs, heads, threads):
    q = wl.queries(step)
    if threads <= 1:
        return decode_attention(q, kc, vc, tables, lens, wl.block_size, wl.sm_scale, wl.kv_dtype,
                                wl.k_scale, wl.v_scale, seqs=seqs, heads=heads)
    out = np.full((len(wl.batch), wl.num_q_heads, wl.head_dim), np.nan, dtype=np.float64)

    def one(s):
        out[s] = decode_attention(q, kc, vc, tables, lens, wl.block_size, wl.sm_scale, wl.kv_dtype,
                                  wl.k_scale, wl.v_scale, seqs=[s], heads=heads)[s]

    per_sequence(one, range(len(wl.batch)) if seqs is None else seqs, threads)
    return out


def run(wl, steps: int = 1, seqs=None, heads=None, keep_rounds: bool = False, threads: int = 1) -> OracleRun:
    """Apply the setup rounds and `steps` decode steps; attention after each step.

    seqs / heads restrict attention to a sample of batch positions / query heads.
    threads > 1 spreads the sequences of each step's attention over threads.
    """
    alloc = BlockAllocatorModel(wl.num_blocks, wl.block_size, wl.free_order)
    kc = empty_cache(wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim, wl.kv_dtype)
    vc = empty_cache(wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim, wl.kv_dtype)
    run_ = OracleRun(alloc, kc, vc)
    host = _host_pool(wl, alloc)
    for ops in wl.setup_rounds:
        r = run_round(wl, alloc, kc, vc, ops, host)
        if keep_rounds:
            run_.rounds.append(r)
    for step in range(steps):
        ops = wl.step_ops(step)
        r = run_round(wl, alloc, kc, vc, ops, host)
        if keep_rounds:
            run_.rounds.append(r)
        tables = [alloc.block_table(s) for s in wl.batch]
        lens = [alloc.num_tokens(s) for s in wl.batch]
        out = _decode_step(wl, step, kc, vc, tables, lens, seqs, heads, threads)
        run_.outputs.append(out)
        run_.tables.append(tables)
        run_.ctx_lens.append(lens)
    return run_


@dataclass
class PrefillRun:
    alloc: BlockAllocatorModel
    k_cache: np.ndarray
    v_cache: np.ndarray
    cached: dict          # prompt sequence -> tokens found in the prefix cache
    chunks: list          # query rows per batch sequence
    q_start: np.ndarray   # int64 [B + 1]
    tables: list
    ctx_lens: list
    rows: dict            # batch index -> float64 [chunk, Hq, D] (sampled sequences only)

    @property
    def output(self) -> np.ndarray:
        """[total_q, Hq, D] float64, NaN for rows of sequences outside the sample."""
        first = next(iter(self.rows.values()), None)
        hq, d = (first.shape[1], first.shape[2]) if first is not None else (0, 0)
        out = np.full((int(self.q_start[-1]), hq, d), np.nan)
        for i, r in self.rows.items():
            out[self.q_start[i]:self.q_start[i + 1]] = r
        return out


def run_prefill(wl, seqs=None, threads: int = 1) -> PrefillRun:
    """Apply the setup rounds, then one prefill pass: every batch sequence's
    chunk (the positions its prompt did not find in the prefix cache, or its
    scripted last positions) attends causally over its context
    ("Where Did the VRAM Go (KV cache tutorial)", §4.2). seqs restricts
    attention to a sample of batch positions; threads > 1 spreads the
    sequences over threads."""
    alloc = BlockAllocatorModel(wl.num_blocks, wl.block_size, wl.free_order)
    kc = empty_cache(wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim, wl.kv_dtype)
    vc = empty_cache(wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim, wl.kv_dtype)
    cached = {}
    host = _host_pool(wl, alloc)
    for ops in wl.setup_rounds:
        r = run_round(wl, alloc, kc, vc, ops, host)
        for op, c, _ in r.prompts:
            cached[op.seq] = c
    chunks = wl.chunk_lengths(cached)
    q_start = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int64)
    tables = [alloc.block_table(s) for s in wl.batch]
    lens = [alloc.num_tokens(s) for s in wl.batch]
    rows = {}

    def one(i):
        s, n = wl.batch[i], chunks[i]
        q = wl.prefill_queries(s, n)
        rows[i] = prefill_attention(q, [0, n], kc, vc, [tables[i]], [lens[i]], wl.block_size, wl.sm_scale,
                                    wl.kv_dtype, wl.k_scale, wl.v_scale)

    per_sequence(one, range(len(wl.batch)) if seqs is None else seqs, threads)
    rows = dict(sorted(rows.items()))
    return PrefillRun(alloc, kc, vc, cached, chunks, q_start, tables, lens, rows)
