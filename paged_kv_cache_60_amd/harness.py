"""Replays a scripted workload on the GPU through PagedKVEngine.

A script (see the ``workloads`` package) is a list of setup rounds of block
manager operations followed by decode steps. Each round runs all of its
operations on the host block manager first, then the round's copy-on-write
block copies, then writes the round's new tokens (in chunks of at most
``chunk_tokens`` tokens, so host staging stays bounded); this is the same
order in which a serving loop would issue them.

The script object is duck-typed: it needs ``setup_rounds``, ``round_kv(ops)``,
``step_ops(i)``, ``queries(i)`` and the shape attributes used below.
"""
from __future__ import annotations

import numpy as np
import torch

from .engine import PagedKVEngine


def make_engine(wl, device="cuda", poison=True) -> PagedKVEngine:
    return PagedKVEngine(wl.num_blocks, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size,
                         wl.kv_dtype, wl.free_order, wl.k_scale, wl.v_scale, wl.k_inv_scale,
                         wl.v_inv_scale, device=device, poison=poison)


def replay_round(eng: PagedKVEngine, wl, ops, chunk_tokens: int = 1 << 18):
    slots, pairs, prompts = eng.apply_ops(ops)
    eng.copy_blocks(pairs)
    for op, c, sl in prompts:  # rows after the cached blocks only
        K, V = wl.prompt_kv(op, c)
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
    return slots, pairs


def replay_setup(eng: PagedKVEngine, wl, chunk_tokens: int = 1 << 18):
    for ops in wl.setup_rounds:
        replay_round(eng, wl, ops, chunk_tokens)
    torch.cuda.synchronize()


def step_inputs(wl, step, device="cuda"):
    """(k_new, v_new, q) on device for decode step `step`."""
    K, V = wl.round_kv(wl.step_ops(step))
    q = wl.queries(step)
    return (torch.from_numpy(K).to(device), torch.from_numpy(V).to(device),
            torch.from_numpy(q).to(device))


def run_steps(eng: PagedKVEngine, wl, steps: int, partition_tokens: int = 0, device="cuda"):
    """Decode `steps` steps; returns per-step outputs (host fp16 arrays) and (tables, ctx)."""
    eng.prepare_steps(wl.batch, wl.max_blocks_per_seq, partition_tokens)
    outs, metas = [], []
    B = len(wl.batch)
    for s in range(steps):
        k, v, q = step_inputs(wl, s, device)
        out = torch.empty((B, wl.num_q_heads, wl.head_dim), dtype=torch.float16, device=device)
        eng.decode_step(k, v, q, out)
        outs.append(out.cpu().numpy())
        metas.append(eng.host_tables())
    return outs, metas
