"""Prefill (multi-token, causal) attention over a paged KV cache, in float64.
TEST INFRASTRUCTURE.

What is computed. A request whose leading blocks were found in the prefix
cache maps them into its block table and prefills only the positions that
missed ("Where Did the VRAM Go (KV cache tutorial)", §4.2; §5 measures the
time to first token it saves). The same holds for a prompt cut into chunks:
each chunk's query tokens attend over everything already in the cache plus
the chunk itself. So, for sequence s:
  * its context holds L = ctx_lens[s] tokens, reached through its block table
    exactly as in decode ("From OOM to Smooth Inference (RAG memory
    management)", §2.1), and includes the n query tokens of the chunk (their
    K/V are in the cache before attention runs);
  * the chunk's query rows are q[q_start[s] : q_start[s+1]], n = q_start[s+1]
    - q_start[s]; row i sits at position p = L - n + i, i.e. the chunk is the
    last n positions of the context (the reading taken: the pages never write
    the positions out);
  * row i attends over positions 0..p (causal: a token sees itself and what
    came before it). A row with p < 0 (a chunk longer than its context) has
    nothing to attend and its output is 0, as for an empty decode context.
For each query head h and its KV head h // (Hq / Hkv):
  out[row, h] = sum_{t<=p} exp(z_t - max z) V_t / sum_{t<=p} exp(z_t - max z),
  z_t = sm_scale * <q[row, h], K_t>.
That is plain causal softmax attention restricted to the chunk's rows; the
pages take attention itself as given.
"""
from __future__ import annotations

import numpy as np

from .attention import gather_sequence


def prefill_sequence(q_rows, K, V, L, sm_scale, group):
    """Outputs [n, Hq, D] float64 for the n query rows of one sequence.

    q_rows: [n, Hq, D]; K, V: [L, Hkv, D] float64 (the sequence's gathered
    context). Row i attends positions 0 .. L - n + i.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    n, hq, d = q_rows.shape
    out = np.zeros((n, hq, d), dtype=np.float64)
    if n == 0:
        return out
    pos = L - n + np.arange(n)                       # position of each query row
    visible = np.arange(L)[None, :] <= pos[:, None]  # [n, L] causal mask
    live = pos >= 0                                  # rows with something to attend
    if not live.any():                               # an empty context: every row is 0
        return out
    for h in range(hq):
        kv = h // group
        z = sm_scale * (q_rows[live, h, :] @ K[:, kv, :].T)  # [rows, L]
        z = np.where(visible[live], z, -np.inf)
        p = np.exp(z - z.max(axis=1, keepdims=True))          # masked entries -> 0
        out[live, h] = (p @ V[:, kv, :]) / p.sum(axis=1, keepdims=True)
    return out


def prefill_attention(q, q_start, k_cache, v_cache, block_tables, ctx_lens, block_size,
                      sm_scale, kv_dtype="f16", k_scale=1.0, v_scale=1.0, seqs=None):
    """Reference output [total_q, Hq, D] float64 for chunked prefill.

    q: [total_q, Hq, D] float16, rows of sequence s at q_start[s] .. q_start[s+1]-1.
    block_tables: per-sequence lists of physical block ids. seqs restricts
    the computation to a sample of sequences (other rows are left NaN).
    """
    q = np.asarray(q)
    total, hq, d = q.shape
    hkv = np.asarray(k_cache).shape[1]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    B = len(ctx_lens)
    if len(q_start) != B + 1 or q_start[0] != 0 or q_start[B] != total:
        raise ValueError("q_start must be [0, ..., total_q] with one entry per sequence + 1")
    out = np.full((total, hq, d), np.nan, dtype=np.float64)
    for s in (range(B) if seqs is None else seqs):
        r0, r1 = int(q_start[s]), int(q_start[s + 1])
        L = int(ctx_lens[s])
        K = gather_sequence(k_cache, block_tables[s], L, block_size, kv_dtype, k_scale)
        V = gather_sequence(v_cache, block_tables[s], L, block_size, kv_dtype, v_scale)
        out[r0:r1] = prefill_sequence(q[r0:r1], K, V, L, sm_scale, hq // hkv)
    return out
