"""Torch-facing wrappers of the kernel entry points (argument marshalling only).

Every function checks shapes, dtypes and devices, then passes raw device
pointers and the current HIP stream to libpagedkv.so. All computation happens
in the library's kernels.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib, guards
from ._lib import PkvError, check

F16 = "f16"
FP8 = "fp8"            # OCP e4m3fn
FP8_E5M2 = "fp8_e5m2"  # OCP e5m2


def kv_dtype_code(kv_dtype: str) -> int:
    if kv_dtype == F16:
        return _lib.KV_F16
    if kv_dtype == FP8:
        return _lib.KV_FP8_E4M3
    if kv_dtype == FP8_E5M2:
        return _lib.KV_FP8_E5M2
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


def cache_torch_dtype(kv_dtype: str) -> torch.dtype:
    return torch.float16 if kv_dtype == F16 else torch.uint8


def _per_head(scale) -> bool:
    """A scale given as a device tensor holds one value per KV head (the *_scaled
    entry points); a Python number is one value for the whole tensor."""
    return isinstance(scale, torch.Tensor)


def _scales_ok(k, v, hkv) -> bool:
    return all(t.is_cuda and t.dtype == torch.float32 and t.is_contiguous() and t.shape == (hkv,) for t in (k, v))


def _stream_ptr(stream=None) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _p(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _require(cond: bool, where: str, what: str):
    if not cond:
        raise PkvError(_lib.PKV_ERR_INVALID, f"{where}: {what}")


def _guard_slots(slot_mapping, T, num_slots, where):
    """With debug checks on: no two valid tokens may share a slot."""
    if guards.debug_checks() and T > 0:
        dup = guards.slot_conflicts(slot_mapping[:T].cpu().numpy(), num_slots)
        _require(len(dup) == 0, where, f"slots written by more than one token: {dup[:8].tolist()}")


def _guard_pairs(pairs, n_src, n_dst, where):
    """With debug checks on: no pair's destination is another pair's source or destination."""
    if guards.debug_checks() and pairs.shape[0] > 0:
        bad = guards.pair_conflicts(pairs.cpu().numpy(), n_src, n_dst)
        _require(len(bad) == 0, where, f"copy pairs that race with another pair: {bad[:8]}")


def _cache_ok(c: torch.Tensor, kv_dtype: str) -> bool:
    if not (c.is_cuda and c.is_contiguous() and c.dim() == 4):
        return False
    return c.dtype == torch.float16 if kv_dtype == F16 else c.element_size() == 1


def paged_kv_write(k_new, v_new, k_cache, v_cache, slot_mapping, kv_dtype=F16,
                   k_inv_scale=1.0, v_inv_scale=1.0, stream=None):
    """Scatter k_new/v_new [T, Hkv, D] (fp16) into the caches at slot_mapping [T] (int64).
    fp8 multipliers: Python numbers (one per tensor) or float32 device tensors [Hkv] (one per KV head)."""
    w = "paged_kv_write"
    _require(k_new.is_cuda and k_new.dtype == torch.float16 and k_new.is_contiguous(), w, "k_new")
    _require(v_new.shape == k_new.shape and v_new.dtype == torch.float16 and v_new.is_contiguous(), w, "v_new")
    _require(_cache_ok(k_cache, kv_dtype) and _cache_ok(v_cache, kv_dtype), w, "caches")
    _require(k_cache.shape == v_cache.shape, w, "cache shapes")
    nb, hkv, bs, d = k_cache.shape
    T = k_new.shape[0]
    _require(k_new.dim() == 3 and k_new.shape[1] == hkv and k_new.shape[2] == d, w, "k_new shape")
    _require(slot_mapping.is_cuda and slot_mapping.dtype == torch.int64 and slot_mapping.shape == (T,)
             and slot_mapping.is_contiguous(), w, "slot_mapping")
    _guard_slots(slot_mapping, T, nb * bs, w)
    lib = _lib.load()
    if _per_head(k_inv_scale):
        _require(_scales_ok(k_inv_scale, v_inv_scale, hkv), w, "per-head inverse scales")
        check(lib.paged_kv_write_scaled(_p(k_new), _p(v_new), _p(k_cache), _p(v_cache), _p(slot_mapping), T, nb,
                                        hkv, d, bs, kv_dtype_code(kv_dtype), _p(k_inv_scale), _p(v_inv_scale),
                                        _stream_ptr(stream)), w)
        return
    check(lib.paged_kv_write(_p(k_new), _p(v_new), _p(k_cache), _p(v_cache), _p(slot_mapping), T, nb,
                             hkv, d, bs, kv_dtype_code(kv_dtype), float(k_inv_scale), float(v_inv_scale),
                             _stream_ptr(stream)), w)


def _device_readable(t) -> bool:
    """On the GPU, or pinned host memory the kernels can read directly."""
    return t.is_cuda or t.is_pinned()


def paged_block_copy(k_cache, v_cache, pairs, stream=None):
    """Copy whole blocks pairs[i] = (src, dst) (int32 [n, 2], device or pinned) in both caches."""
    w = "paged_block_copy"
    _require(k_cache.is_cuda and v_cache.is_cuda and k_cache.is_contiguous() and v_cache.is_contiguous()
             and k_cache.shape == v_cache.shape and k_cache.dim() == 4, w, "caches")
    _require(_device_readable(pairs) and pairs.dtype == torch.int32 and pairs.dim() == 2
             and pairs.shape[1] == 2 and pairs.is_contiguous(), w, "pairs")
    nb = k_cache.shape[0]
    block_bytes = k_cache[0].numel() * k_cache.element_size()
    _guard_pairs(pairs, nb, None, w)
    lib = _lib.load()
    check(lib.paged_block_copy(_p(k_cache), _p(v_cache), _p(pairs), pairs.shape[0], nb, block_bytes,
                               _stream_ptr(stream)), w)


def paged_block_swap(k_cache, v_cache, k_host, v_host, pairs, direction, stream=None):
    """Whole-block copies between the device caches and pinned host caches of the same
    layout. direction "out": pairs (device, host), host <- device; "in": pairs (host,
    device), device <- host. pairs: int32 [n, 2], device or pinned."""
    w = "paged_block_swap"
    _require(k_cache.is_cuda and v_cache.is_cuda and k_cache.is_contiguous() and v_cache.is_contiguous()
             and k_cache.shape == v_cache.shape and k_cache.dim() == 4, w, "caches")
    _require(k_host.is_pinned() and v_host.is_pinned() and k_host.is_contiguous() and v_host.is_contiguous()
             and k_host.shape == v_host.shape and k_host.shape[1:] == k_cache.shape[1:]
             and k_host.dtype == k_cache.dtype and v_host.dtype == v_cache.dtype, w, "host caches")
    _require(_device_readable(pairs) and pairs.dtype == torch.int32 and pairs.dim() == 2
             and pairs.shape[1] == 2 and pairs.is_contiguous(), w, "pairs")
    _require(direction in ("out", "in"), w, "direction")
    n_dev, n_host = k_cache.shape[0], k_host.shape[0]
    _guard_pairs(pairs, *((n_dev, n_host) if direction == "out" else (n_host, n_dev)), w)
    block_bytes = k_cache[0].numel() * k_cache.element_size()
    lib = _lib.load()
    check(lib.paged_block_swap(_p(k_cache), _p(v_cache), _p(k_host), _p(v_host), _p(pairs), pairs.shape[0],
                               k_cache.shape[0], k_host.shape[0], block_bytes,
                               _lib.SWAP_OUT if direction == "out" else _lib.SWAP_IN, _stream_ptr(stream)), w)


def paged_kv_write_step(k_new, v_new, k_cache, v_cache, slot_mapping, ctx_src, ctx_dst, updates,
                        n_updates, block_tables, kv_dtype=F16, k_inv_scale=1.0, v_inv_scale=1.0,
                        stream=None):
    """paged_kv_write plus the step metadata (context lengths, table updates) in one launch.

    slot_mapping / ctx_src / updates may be pinned host tensors (read directly by the kernel).
    """
    w = "paged_kv_write_step"
    _require(k_new.is_cuda and k_new.dtype == torch.float16 and k_new.is_contiguous(), w, "k_new")
    _require(v_new.shape == k_new.shape and v_new.dtype == torch.float16 and v_new.is_contiguous(), w, "v_new")
    _require(_cache_ok(k_cache, kv_dtype) and _cache_ok(v_cache, kv_dtype) and k_cache.shape == v_cache.shape,
             w, "caches")
    nb, hkv, bs, d = k_cache.shape
    T = k_new.shape[0]
    _require(k_new.dim() == 3 and k_new.shape[1] == hkv and k_new.shape[2] == d, w, "k_new shape")
    _require(_device_readable(slot_mapping) and slot_mapping.dtype == torch.int64 and slot_mapping.numel() >= T,
             w, "slot_mapping")
    _require(_device_readable(ctx_src) and ctx_src.dtype == torch.int32 and ctx_dst.is_cuda
             and ctx_dst.dtype == torch.int32 and ctx_src.numel() >= ctx_dst.numel(), w, "ctx")
    _require(_device_readable(updates) and updates.dtype == torch.int32 and updates.numel() >= 3 * n_updates,
             w, "updates")
    _require(block_tables.is_cuda and block_tables.dtype == torch.int32 and block_tables.dim() == 2, w, "tables")
    rows, maxb = block_tables.shape
    _guard_slots(slot_mapping, T, nb * bs, w)
    lib = _lib.load()
    if _per_head(k_inv_scale):
        _require(_scales_ok(k_inv_scale, v_inv_scale, hkv), w, "per-head inverse scales")
        check(lib.paged_kv_write_step_scaled(_p(k_new), _p(v_new), _p(k_cache), _p(v_cache), _p(slot_mapping), T,
                                             nb, hkv, d, bs, kv_dtype_code(kv_dtype), _p(k_inv_scale),
                                             _p(v_inv_scale), _p(ctx_src), _p(ctx_dst), ctx_dst.numel(),
                                             _p(updates), int(n_updates), _p(block_tables), rows, maxb,
                                             _stream_ptr(stream)), w)
        return
    check(lib.paged_kv_write_step(_p(k_new), _p(v_new), _p(k_cache), _p(v_cache), _p(slot_mapping), T, nb,
                                  hkv, d, bs, kv_dtype_code(kv_dtype), float(k_inv_scale), float(v_inv_scale),
                                  _p(ctx_src), _p(ctx_dst), ctx_dst.numel(), _p(updates), int(n_updates),
                                  _p(block_tables), rows, maxb, _stream_ptr(stream)), w)


def workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size,
                    partition_tokens=0) -> int:
    return int(_lib.load().paged_attn_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                             max_blocks_per_seq, block_size,
                                                             partition_tokens))


def decode_workers(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                   kv_dtype=F16, partition_tokens=0) -> int:
    """Workers (waves) that pass 1 of paged_attn_decode uses for this shape on the current device."""
    n = int(_lib.load().paged_attn_decode_workers(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                                  max_blocks_per_seq, kv_dtype_code(kv_dtype),
                                                  partition_tokens))
    check(min(n, 0), "paged_attn_decode_workers")
    return n


def time_next_pass1(start=None, stop=None) -> None:
    """Arm the library's measurement hook: the next pass-1 launch of this
    thread records `start` and `stop` (torch.cuda.Event with timing enabled,
    each already recorded once so that its handle exists) as its own start and
    stop; `start.elapsed_time(stop)` after a synchronize is then that kernel's
    duration alone. No arguments: disarm."""
    if (start is None) != (stop is None):
        raise ValueError("time_next_pass1 takes both events or neither")
    h0 = h1 = None
    if start is not None:
        h0, h1 = int(start.cuda_event), int(stop.cuda_event)
        if not h0 or not h1:
            raise ValueError("record each event once before arming the hook (its handle is created then)")
    check(_lib.load().pkv_time_next_pass1(h0, h1), "pkv_time_next_pass1")


def paged_attn_decode(out, q, k_cache, v_cache, block_tables, ctx_lens, sm_scale, kv_dtype=F16,
                      k_scale=1.0, v_scale=1.0, partition_tokens=0, workspace=None, passes=3,
                      stream=None):
    """out/q [B, Hq, D] fp16; block_tables [B, max_blocks] int32; ctx_lens [B] int32.
    workspace: device buffer of at least workspace_bytes(...) bytes; allocated here if None."""
    w = "paged_attn_decode"
    _require(q.is_cuda and q.dtype == torch.float16 and q.is_contiguous() and q.dim() == 3, w, "q")
    _require(out.is_cuda and out.dtype == torch.float16 and out.is_contiguous() and out.shape == q.shape, w, "out")
    _require(_cache_ok(k_cache, kv_dtype) and _cache_ok(v_cache, kv_dtype) and k_cache.shape == v_cache.shape,
             w, "caches")
    B, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    _require(d == d2, w, "head_dim")
    _require(block_tables.is_cuda and block_tables.dtype == torch.int32 and block_tables.dim() == 2
             and block_tables.shape[0] == B and block_tables.is_contiguous(), w, "block_tables")
    _require(ctx_lens.is_cuda and ctx_lens.dtype == torch.int32 and ctx_lens.shape == (B,)
             and ctx_lens.is_contiguous(), w, "ctx_lens")
    maxb = block_tables.shape[1]
    need = workspace_bytes(B, hq, hkv, d, maxb, bs, partition_tokens) if B > 0 else 0
    ws_ptr, ws_bytes = ctypes.c_void_p(0), 0
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        _require(workspace.is_cuda and workspace.numel() * workspace.element_size() >= need, w,
                 "workspace too small")
        ws_ptr, ws_bytes = _p(workspace), workspace.numel() * workspace.element_size()
    lib = _lib.load()
    if _per_head(k_scale):
        _require(_scales_ok(k_scale, v_scale, hkv), w, "per-head scales")
        check(lib.paged_attn_decode_scaled(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables), maxb,
                                           _p(ctx_lens), B, hq, hkv, d, bs, nb, float(sm_scale),
                                           kv_dtype_code(kv_dtype), _p(k_scale), _p(v_scale),
                                           int(partition_tokens), ws_ptr, ws_bytes, int(passes),
                                           _stream_ptr(stream)), w)
        return
    check(lib.paged_attn_decode_passes(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables), maxb,
                                       _p(ctx_lens), B, hq, hkv, d, bs, nb, float(sm_scale),
                                       kv_dtype_code(kv_dtype), float(k_scale), float(v_scale),
                                       int(partition_tokens), ws_ptr, ws_bytes, int(passes),
                                       _stream_ptr(stream)), w)


def paged_attn_decode_noalloc(out, q, k_cache, v_cache, block_tables, ctx_lens, sm_scale, kv_dtype=F16,
                              k_scale=1.0, v_scale=1.0, partition_tokens=0, stream=None):
    """paged_attn_decode with no workspace: the library's per-device scratch array
    holds the partials, and neither this wrapper nor the call allocates device
    memory. Calls that overlap on one device race (they share the array)."""
    w = "paged_attn_decode_noalloc"
    _require(q.is_cuda and q.dtype == torch.float16 and q.is_contiguous() and q.dim() == 3, w, "q")
    _require(out.is_cuda and out.dtype == torch.float16 and out.is_contiguous() and out.shape == q.shape, w, "out")
    _require(_cache_ok(k_cache, kv_dtype) and _cache_ok(v_cache, kv_dtype) and k_cache.shape == v_cache.shape,
             w, "caches")
    B, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    _require(d == d2, w, "head_dim")
    _require(block_tables.is_cuda and block_tables.dtype == torch.int32 and block_tables.dim() == 2
             and block_tables.shape[0] == B and block_tables.is_contiguous(), w, "block_tables")
    _require(ctx_lens.is_cuda and ctx_lens.dtype == torch.int32 and ctx_lens.shape == (B,)
             and ctx_lens.is_contiguous(), w, "ctx_lens")
    _require(not _per_head(k_scale), w, "per-tensor scales only")
    check(_lib.load().paged_attn_decode_noalloc(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables),
                                                block_tables.shape[1], _p(ctx_lens), B, hq, hkv, d, bs, nb,
                                                float(sm_scale), kv_dtype_code(kv_dtype), float(k_scale),
                                                float(v_scale), int(partition_tokens), _stream_ptr(stream)), w)


# query columns (sequence, query head) of one part of a group: the columns
# that one read of the group's shared blocks serves; a group of more than
# SHARED_COLUMNS / G members is cut into several parts
SHARED_COLUMNS = 32
SHARED_MAX_SEQS = 4096  # paged_attn_decode_shared takes batches up to this size


def shared_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim) -> int:
    """Bytes of device workspace paged_attn_decode_shared needs (0 for a bad shape)."""
    return int(_lib.load().paged_attn_decode_shared_workspace_bytes(num_seqs, num_q_heads, num_kv_heads,
                                                                    head_dim))


def paged_attn_decode_shared(out, q, k_cache, v_cache, block_tables, ctx_lens, groups, sm_scale, kv_dtype=F16,
                             k_scale=1.0, v_scale=1.0, partition_tokens=0, workspace=None, passes=7,
                             stream=None):
    """paged_attn_decode for a batch whose runs of sequences share leading
    blocks: groups is a device int32 tensor [3, num_groups] holding, per
    group, its first batch index, its member count and its shared tokens (as
    BlockManager.prefix_groups returns them); with no groups ([3, 0]) the
    caller declares that no block is held by two sequences, and the call is
    paged_attn_decode with its waves ordered for disjoint blocks (the same
    bits). passes: bit 0 or 1 the grouped pass 1, bit 2 the merge of parts
    split between workers."""
    w = "paged_attn_decode_shared"
    _require(q.is_cuda and q.dtype == torch.float16 and q.is_contiguous() and q.dim() == 3, w, "q")
    _require(out.is_cuda and out.dtype == torch.float16 and out.is_contiguous() and out.shape == q.shape, w, "out")
    _require(_cache_ok(k_cache, kv_dtype) and _cache_ok(v_cache, kv_dtype) and k_cache.shape == v_cache.shape,
             w, "caches")
    B, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    _require(d == d2, w, "head_dim")
    _require(block_tables.is_cuda and block_tables.dtype == torch.int32 and block_tables.dim() == 2
             and block_tables.shape[0] == B and block_tables.is_contiguous(), w, "block_tables")
    _require(ctx_lens.is_cuda and ctx_lens.dtype == torch.int32 and ctx_lens.shape == (B,)
             and ctx_lens.is_contiguous(), w, "ctx_lens")
    _require(groups.is_cuda and groups.dtype == torch.int32 and groups.dim() == 2 and groups.shape[0] == 3
             and groups.is_contiguous(), w, "groups")
    ng = groups.shape[1]
    maxb = block_tables.shape[1]
    ws_ptr, ws_bytes = ctypes.c_void_p(0), 0
    if B > 0:
        need = shared_workspace_bytes(B, hq, hkv, d)
        _require(need > 0, w, "shape")
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        _require(workspace.is_cuda and workspace.numel() * workspace.element_size() >= need, w,
                 "workspace too small")
        ws_ptr, ws_bytes = _p(workspace), workspace.numel() * workspace.element_size()
    per_head = _per_head(k_scale)
    if per_head:
        _require(_scales_ok(k_scale, v_scale, hkv), w, "per-head scales")
    gp = [ctypes.c_void_p(groups.data_ptr() + r * ng * 4) if ng else ctypes.c_void_p(0) for r in range(3)]
    check(_lib.load().paged_attn_decode_shared(
        _p(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables), maxb, _p(ctx_lens), B, hq, hkv, d, bs, nb,
        float(sm_scale), kv_dtype_code(kv_dtype), 1.0 if per_head else float(k_scale),
        1.0 if per_head else float(v_scale), _p(k_scale) if per_head else ctypes.c_void_p(0),
        _p(v_scale) if per_head else ctypes.c_void_p(0), gp[0], gp[1], gp[2], ng, int(partition_tokens),
        ws_ptr, ws_bytes, int(passes), _stream_ptr(stream)), w)


def paged_attn_prefill(out, q, k_cache, v_cache, block_tables, ctx_lens, q_start, sm_scale, kv_dtype=F16,
                       k_scale=1.0, v_scale=1.0, stream=None):
    """Chunked causal prefill. out/q [total_q, Hq, D] fp16; block_tables [B, max_blocks] int32;
    ctx_lens [B] int32 (context including the chunk); q_start [B + 1] int32 (row offsets)."""
    w = "paged_attn_prefill"
    _require(q.is_cuda and q.dtype == torch.float16 and q.is_contiguous() and q.dim() == 3, w, "q")
    _require(out.is_cuda and out.dtype == torch.float16 and out.is_contiguous() and out.shape == q.shape, w, "out")
    _require(_cache_ok(k_cache, kv_dtype) and _cache_ok(v_cache, kv_dtype) and k_cache.shape == v_cache.shape,
             w, "caches")
    total, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    _require(d == d2, w, "head_dim")
    _require(block_tables.is_cuda and block_tables.dtype == torch.int32 and block_tables.dim() == 2
             and block_tables.is_contiguous(), w, "block_tables")
    B = block_tables.shape[0]
    _require(ctx_lens.is_cuda and ctx_lens.dtype == torch.int32 and ctx_lens.shape == (B,)
             and ctx_lens.is_contiguous(), w, "ctx_lens")
    _require(q_start.is_cuda and q_start.dtype == torch.int32 and q_start.shape == (B + 1,)
             and q_start.is_contiguous(), w, "q_start")
    lib = _lib.load()
    if _per_head(k_scale):
        _require(_scales_ok(k_scale, v_scale, hkv), w, "per-head scales")
        check(lib.paged_attn_prefill_scaled(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables),
                                            block_tables.shape[1], _p(ctx_lens), _p(q_start), B, total, hq, hkv,
                                            d, bs, nb, float(sm_scale), kv_dtype_code(kv_dtype), _p(k_scale),
                                            _p(v_scale), _stream_ptr(stream)), w)
        return
    check(lib.paged_attn_prefill(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables),
                                 block_tables.shape[1], _p(ctx_lens), _p(q_start), B, total, hq, hkv, d, bs,
                                 nb, float(sm_scale), kv_dtype_code(kv_dtype), float(k_scale), float(v_scale),
                                 _stream_ptr(stream)), w)


def paged_step_metadata(slots_src, slots_dst, ctx_src, ctx_dst, n_seqs, cow_src, cow_dst, n_cow,
                        updates_src, n_updates, block_tables, stream=None):
    """Apply a decode step's metadata (sources: pinned host tensors or device tensors)."""
    rows, maxb = block_tables.shape
    lib = _lib.load()
    check(lib.paged_step_metadata(_p(slots_src), _p(slots_dst), _p(ctx_src), _p(ctx_dst), int(n_seqs),
                                  _p(cow_src), _p(cow_dst), int(n_cow), _p(updates_src), int(n_updates),
                                  _p(block_tables), rows, maxb, _stream_ptr(stream)), "paged_step_metadata")
