"""Decode attention over a paged KV cache, in float64. TEST INFRASTRUCTURE.

What is computed (one new query token per sequence):
  1. Gather: walk the sequence's block table, logical block i -> physical
     block table[i], and copy tokens 0..L-1 into a contiguous buffer
     ("From OOM to Smooth Inference (RAG memory management)", §2.1;
     "Inference Engine Memory Optimisation", §2.2). fp16 values convert to
     float64 exactly; fp8 bytes (e4m3 or e5m2) become decode(byte) * scale
     with one scale per tensor or per KV head ("Where Did the VRAM Go (KV
     cache tutorial)", §6.1-6.3).
  2. For query head h, the KV head is h // (Hq / Hkv) (contiguous groups; the
     pages do not say, this is the reading taken).
  3. z_t = sm_scale * <q_h, K_t>;  p_t = exp(z_t - max z);  out = sum p_t V_t / sum p_t.
     This is plain softmax attention, which the pages take as given.
  4. A sequence of length 0 has output 0 (0/0 read as 0).
"""
from __future__ import annotations

import numpy as np

from . import fp8


def gather_sequence(cache, table, length, block_size, kv_dtype="f16", scale=1.0):
    """Contiguous [length, Hkv, D] float64 copy of one sequence's K or V.

    Position t lives in physical block table[t // block_size] at offset
    t % block_size: take the sequence's first ceil(length / block_size) table
    entries, pick those blocks out of the pool in table order, lay their
    slots end to end and keep the first `length` positions."""
    cache = np.asarray(cache)
    hkv, d = cache.shape[1], cache.shape[3]
    nblk = -(-length // block_size)
    phys = np.asarray(table[:nblk], dtype=np.int64)
    blocks = cache[phys]                       # [nblk, Hkv, bs, D] stored values, logical block order
    rows = np.transpose(blocks, (0, 2, 1, 3)).reshape(nblk * block_size, hkv, d)[:length]
    if kv_dtype in fp8.KV_FORMATS:
        return fp8.dequantize(rows, scale, fp8.KV_FORMATS[kv_dtype], head_axis=1)  # per tensor or KV head
    return rows.astype(np.float64)


def attend_one(q_h, K, V, sm_scale):
    """softmax(sm_scale * K q) weighted sum of V rows, float64. K, V: [L, D]."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    z = sm_scale * (K @ np.asarray(q_h, dtype=np.float64))
    p = np.exp(z - z.max())
    return (p @ V) / p.sum()


def decode_attention(q, k_cache, v_cache, block_tables, ctx_lens, block_size,
                     sm_scale, kv_dtype="f16", k_scale=1.0, v_scale=1.0,
                     seqs=None, heads=None):
    """Reference output [B, Hq, D] float64 for one decode token per sequence.

    q: [B, Hq, D] float16. block_tables: per-sequence lists (or rows of an
    array) of physical block ids. seqs / heads restrict the computation to
    a sample (other entries are left NaN).
    """
    q = np.asarray(q)
    B, Hq, D = q.shape
    hkv = np.asarray(k_cache).shape[1]
    if Hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // hkv
    out = np.full((B, Hq, D), np.nan, dtype=np.float64)
    seq_ids = range(B) if seqs is None else seqs
    for s in seq_ids:
        L = int(ctx_lens[s])
        K = gather_sequence(k_cache, block_tables[s], L, block_size, kv_dtype, k_scale)
        V = gather_sequence(v_cache, block_tables[s], L, block_size, kv_dtype, v_scale)
        for h in (range(Hq) if heads is None else heads):
            kv = h // group
            out[s, h] = attend_one(q[s, h], K[:, kv, :], V[:, kv, :], sm_scale)
    return out
