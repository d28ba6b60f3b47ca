"""Replays a scripted workload on the GPU through PagedKVEngine.

A script (see the ``workloads`` package) is a list of setup rounds of block
manager operations followed by decode steps. Each round runs all of its
operations on the host block manager first, then the round's swap copies (in
op order), copy-on-write block copies, then writes the round's new tokens (in chunks of at most
``chunk_tokens`` tokens, so host staging stays bounded); this is the same
order in which a serving loop would issue them.

The script object is duck-typed: it needs ``setup_rounds``, ``round_kv(ops)``,
``step_ops(i)``, ``queries(i)`` (decode) or ``chunk_lengths`` and
``prefill_queries`` (prefill) and the shape attributes used below.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from .engine import PagedKVEngine


def make_engine(wl, device="cuda", poison=True) -> PagedKVEngine:
    return PagedKVEngine(wl.num_blocks, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size,
                         wl.kv_dtype, wl.free_order, wl.k_scale, wl.v_scale, wl.k_inv_scale,
                         wl.v_inv_scale, device=device, poison=poison,
                         num_host_blocks=getattr(wl, "num_host_blocks", 0))


def replay_round(eng: PagedKVEngine, wl, ops, chunk_tokens: int = 1 << 18):
    slots, pairs, prompts, swaps = eng.apply_ops(ops)
    for direction, sp in swaps:  # in op order, before any write reuses a released block
        eng.swap(direction, sp)
    eng.copy_blocks(pairs)
    # rows after the cached blocks only; the draws run in threads (the
    # generator releases the GIL), a bounded number of prompts at a time
    with ThreadPoolExecutor(max_workers=8) as ex:
        for g0 in range(0, len(prompts), 32):
            group = prompts[g0:g0 + 32]
            for (op, c, sl), (K, V) in zip(group, ex.map(lambda p: wl.prompt_kv(p[0], p[1]), group)):
                eng.write(sl, K, V)
    creating = [o for o in ops if o.kind in ("allocate", "append") and o.n > 0]
    pos = i = 0
    while i < len(creating):
        chunk, acc = [creating[i]], creating[i].n
        i += 1
        while i < len(creating) and acc + creating[i].n <= chunk_tokens:
            chunk.append(creating[i])
            acc += creating[i].n
            i += 1
        K, V = wl.round_kv(chunk)
        eng.write(slots[pos:pos + acc], K, V)
        pos += acc
    assert pos == len(slots)
    return slots, pairs, prompts


def replay_setup(eng: PagedKVEngine, wl, chunk_tokens: int = 1 << 18) -> dict:
    """Replay the setup rounds; returns {prompt seq: tokens found in the prefix cache}."""
    cached = {}
    for ops in wl.setup_rounds:
        _, _, prompts = replay_round(eng, wl, ops, chunk_tokens)
        for op, c, _ in prompts:
            cached[op.seq] = int(c)
    torch.cuda.synchronize()
    return cached


def prefill_inputs(wl, cached, device="cuda"):
    """(q [total_q, Hq, D] fp16, q_start [B + 1] int32, chunk lengths) on device
    for a prefill run after the setup."""
    chunks = wl.chunk_lengths(cached)
    q_start = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = np.empty((int(q_start[-1]), wl.num_q_heads, wl.head_dim), dtype=np.float16)

    def fill(i):
        q[q_start[i]:q_start[i + 1]] = wl.prefill_queries(wl.batch[i], chunks[i])

    with ThreadPoolExecutor(max_workers=8) as ex:  # the generator releases the GIL
        list(ex.map(fill, range(len(chunks))))
    return torch.from_numpy(q).to(device), torch.from_numpy(q_start).to(device), chunks


def run_prefill(eng: PagedKVEngine, wl, cached, device="cuda"):
    """One prefill pass over every batch sequence's chunk; returns (out on
    device, q_start host array, host tables, host context lengths)."""
    q, q_start, chunks = prefill_inputs(wl, cached, device)
    tables, ctx = eng.prepare_prefill(wl.batch, wl.max_blocks_per_seq)
    out = torch.empty_like(q)
    eng.prefill(tables, ctx, q, q_start, out)
    return out, q_start.cpu().numpy(), tables.cpu().numpy(), ctx.cpu().numpy()


def step_inputs(wl, step, device="cuda"):
    """(k_new, v_new, q) on device for decode step `step`."""
    K, V = wl.round_kv(wl.step_ops(step))
    q = wl.queries(step)
    return (torch.from_numpy(K).to(device), torch.from_numpy(V).to(device),
            torch.from_numpy(q).to(device))


def run_steps(eng: PagedKVEngine, wl, steps: int, partition_tokens: int = 0, device="cuda",
              shared_prefix: bool = False):
    """Decode `steps` steps; returns per-step outputs (host fp16 arrays) and (tables, ctx).
    shared_prefix: attend with the shared-prefix decode (runs of the batch that
    share leading blocks read them once)."""
    eng.prepare_steps(wl.batch, wl.max_blocks_per_seq, partition_tokens, shared_prefix=shared_prefix)
    outs, metas = [], []
    B = len(wl.batch)
    for s in range(steps):
        k, v, q = step_inputs(wl, s, device)
        out = torch.empty((B, wl.num_q_heads, wl.head_dim), dtype=torch.float16, device=device)
        eng.decode_step(k, v, q, out)
        outs.append(out.cpu().numpy())
        metas.append(eng.host_tables())
    return outs, metas
