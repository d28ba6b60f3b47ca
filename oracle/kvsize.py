"""Closed forms for KV cache size, pool sizing and reservation waste. TEST INFRASTRUCTURE.

  * KV bytes = 2 (K and V) x layers x kv_heads x head_dim x seq_len x bytes per
    element ("Inference Engine Memory Optimisation", §2.1; "Where Did the VRAM
    Go (KV cache tutorial)", §1.4). The symbolic formula on "From OOM to
    Smooth Inference", §1.1 did not survive extraction; its numeric form uses
    hidden size x layers, which equals kv_heads x head_dim x layers for a
    model without grouped KV heads.
  * Pool size = floor(KV budget / bytes of one block), one block holding
    block_size tokens of every layer ("vLLM Architecture and Memory Use,
    ch. 3", §3.3; that page writes the per-block size with attention heads,
    read here as KV heads so that grouped-query models size correctly).
  * Reservation waste = (reserved - used) / reserved ("From OOM to Smooth
    Inference", §1.2).
  * Internal fragmentation of one sequence = allocated slots - tokens, at most
    block_size - 1 ("From OOM to Smooth Inference", §2.1).
"""
from __future__ import annotations


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return 2 * layers * kv_heads * head_dim * elem_bytes


def kv_bytes(layers: int, kv_heads: int, head_dim: int, seq_len: int, elem_bytes: int,
             batch: int = 1) -> int:
    return kv_bytes_per_token(layers, kv_heads, head_dim, elem_bytes) * seq_len * batch


def pool_blocks(budget_bytes: int, block_size: int, layers: int, kv_heads: int,
                head_dim: int, elem_bytes: int) -> int:
    block_bytes = block_size * kv_bytes_per_token(layers, kv_heads, head_dim, elem_bytes)
    return budget_bytes // block_bytes


def reservation_waste(used_tokens: int, reserved_tokens: int) -> float:
    return (reserved_tokens - used_tokens) / reserved_tokens


def internal_fragmentation(tokens: int, block_size: int) -> int:
    """Unused slots in the last block of a sequence holding `tokens` tokens."""
    blocks = (tokens + block_size - 1) // block_size
    return blocks * block_size - tokens
