"""ctypes loader for libpagedkv.so (argument marshalling only).

The library is built in-tree (``python -m paged_kv_cache_60_amd.build``) and
loaded from this package's directory. There is no fallback: if the library is
missing the import of the GPU entry points fails loudly.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

PKV_OK = 0
PKV_ERR_INVALID = -1
PKV_ERR_OOM = -2
PKV_ERR_NO_SEQ = -3
PKV_ERR_EXISTS = -4
PKV_ERR_HIP = -5

KV_F16 = 0
KV_FP8_E4M3 = 1
KV_FP8_E5M2 = 2

SWAP_OUT = 0
SWAP_IN = 1
PREEMPT_RECOMPUTE = 0
PREEMPT_SWAP = 1

DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20  # PKV_DECODE_NOALLOC_SCRATCH_BYTES

_c_int = ctypes.c_int
_c_i64 = ctypes.c_int64
_c_f = ctypes.c_float
_c_sz = ctypes.c_size_t
_vp = ctypes.c_void_p
_p_i32 = ctypes.POINTER(ctypes.c_int32)
_p_i64 = ctypes.POINTER(ctypes.c_int64)
_p_int = ctypes.POINTER(ctypes.c_int)


class PkvStats(ctypes.Structure):
    _fields_ = [
        ("total_blocks", ctypes.c_int32),
        ("free_blocks", ctypes.c_int32),
        ("used_blocks", ctypes.c_int32),
        ("live_seqs", ctypes.c_int32),
        ("filled_slots", ctypes.c_int64),
        ("utilization", ctypes.c_double),
        ("slot_utilization", ctypes.c_double),
        ("evictable_blocks", ctypes.c_int32),
        ("cached_blocks", ctypes.c_int32),
        ("prefix_query_tokens", ctypes.c_int64),
        ("prefix_hit_tokens", ctypes.c_int64),
        ("host_blocks", ctypes.c_int32),
        ("host_free_blocks", ctypes.c_int32),
        ("swapped_seqs", ctypes.c_int32),
    ]


# name -> (restype, argtypes); every symbol include/pagedkv.h declares.
SIGNATURES = {
    "pkv_status_str": (ctypes.c_char_p, [_c_int]),
    "paged_kv_write": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                _c_int, _c_f, _c_f, _vp]),
    "paged_kv_write_step": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                     _c_int, _c_f, _c_f, _vp, _vp, _c_int, _vp, _c_int, _vp, _c_int,
                                     _c_int, _vp]),
    "paged_kv_write_scaled": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_int, _vp, _vp, _vp]),
    "paged_kv_write_step_scaled": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                            _c_int, _vp, _vp, _vp, _vp, _c_int, _vp, _c_int, _vp, _c_int,
                                            _c_int, _vp]),
    "paged_attn_decode_scaled": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _vp, _c_int, _c_int, _c_int,
                                          _c_int, _c_int, _c_int, _c_f, _c_int, _vp, _vp, _c_int, _vp, _c_sz,
                                          _c_int, _vp]),
    "paged_attn_prefill_scaled": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _c_int, _c_int,
                                           _c_int, _c_int, _c_int, _c_int, _c_int, _c_f, _c_int, _vp, _vp,
                                           _vp]),
    "paged_block_copy": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_sz, _vp]),
    "paged_block_swap": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_sz, _c_int, _vp]),
    "paged_attn_decode_workspace_bytes": (_c_sz, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "paged_attn_decode": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _vp, _c_int, _c_int, _c_int,
                                   _c_int, _c_int, _c_int, _c_f, _c_int, _c_f, _c_f, _c_int, _vp,
                                   _c_sz, _vp]),
    "paged_attn_decode_passes": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _vp, _c_int, _c_int,
                                          _c_int, _c_int, _c_int, _c_int, _c_f, _c_int, _c_f, _c_f,
                                          _c_int, _vp, _c_sz, _c_int, _vp]),
    "paged_attn_decode_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _vp, _c_int, _c_int, _c_int, _c_int,
                                           _c_int, _c_int, _c_f, _c_int, _c_f, _c_f, _c_int, _vp]),
    "paged_attn_decode_workers": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "pkv_time_next_pass1": (_c_int, [_vp, _vp]),
    "paged_attn_decode_shared_workspace_bytes": (_c_sz, [_c_int, _c_int, _c_int, _c_int]),
    "paged_attn_decode_shared": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _vp, _c_int, _c_int, _c_int,
                                          _c_int, _c_int, _c_int, _c_f, _c_int, _c_f, _c_f, _vp,
                                          _vp, _vp, _vp, _vp, _c_int, _c_int, _vp, _c_sz, _c_int, _vp]),
    "paged_attn_prefill": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _c_int, _c_int, _c_int,
                                    _c_int, _c_int, _c_int, _c_int, _c_f, _c_int, _c_f, _c_f, _vp]),
    "paged_step_metadata": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _vp, _vp, _c_int, _vp, _c_int, _vp,
                                     _c_int, _c_int, _vp]),
    "pkv_bm_create": (_c_int, [_c_int, _c_int, _p_i32, ctypes.POINTER(_vp)]),
    "pkv_bm_destroy": (None, [_vp]),
    "pkv_bm_allocate": (_c_int, [_vp, _c_i64, _c_int, _p_i64]),
    "pkv_bm_allocate_prompt": (_c_int, [_vp, _c_i64, _p_i32, _c_int, _p_int, _p_i64]),
    "pkv_bm_append": (_c_int, [_vp, _c_i64, _c_int, _p_i64, _p_i32, _p_i32]),
    "pkv_bm_append_batch": (_c_int, [_vp, _p_i64, _c_int, _p_i64, _p_i32, _p_int]),
    "pkv_bm_decode_step": (_c_int, [_vp, _p_i64, _c_int, _p_i64, _p_i32, _p_int, _p_i32, _p_int, _p_i32, _c_int]),
    "pkv_bm_fork": (_c_int, [_vp, _c_i64, _c_i64]),
    "pkv_bm_share_prefix": (_c_int, [_vp, _c_i64, _c_int, _c_i64]),
    "pkv_bm_free": (_c_int, [_vp, _c_i64]),
    "pkv_bm_slots": (_c_int, [_vp, _c_i64, _c_int, _c_int, _p_i64]),
    "pkv_bm_block_table": (_c_int, [_vp, _c_i64, _p_i32, _c_int, _p_int]),
    "pkv_bm_num_tokens": (_c_int, [_vp, _c_i64, _p_int]),
    "pkv_bm_refcount": (_c_int, [_vp, ctypes.c_int32, _p_int]),
    "pkv_bm_free_list": (_c_int, [_vp, _p_i32, _c_int, _p_int]),
    "pkv_bm_evictable_list": (_c_int, [_vp, _p_i32, _c_int, _p_int]),
    "pkv_bm_cache_entry": (_c_int, [_vp, ctypes.c_int32, _p_int, _p_i32, _p_i32]),
    "pkv_bm_num_free": (_c_int, [_vp]),
    "pkv_bm_stats": (_c_int, [_vp, ctypes.POINTER(PkvStats)]),
    "pkv_bm_export": (_c_int, [_vp, _p_i64, _c_int, _p_i32, _c_int, _p_i32]),
    "pkv_bm_prefix_groups": (_c_int, [_vp, _p_i64, _c_int, _c_int, _p_i32, _p_i32, _p_i32, _c_int, _p_int]),
    "pkv_bm_set_host_blocks": (_c_int, [_vp, _c_int]),
    "pkv_bm_swap_out": (_c_int, [_vp, _p_i64, _c_int, _p_i32, _c_int, _p_int]),
    "pkv_bm_swap_in": (_c_int, [_vp, _p_i64, _c_int, _p_i32, _c_int, _p_int]),
    "pkv_bm_preempt_tail": (_c_int, [_vp, _p_i64, _c_int, _c_int, _c_int, _p_i64, _p_int, _p_i32, _c_int, _p_int]),
    "pkv_bm_swapped_table": (_c_int, [_vp, _c_i64, _p_i32, _c_int, _p_int]),
    "pkv_bm_swapped_tokens": (_c_int, [_vp, _c_i64, _p_int]),
    "pkv_bm_host_free_list": (_c_int, [_vp, _p_i32, _c_int, _p_int]),
    "pkv_bm_host_refcount": (_c_int, [_vp, ctypes.c_int32, _p_int]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libpagedkv.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_60_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


_bm_lib = None


def load_block_manager() -> ctypes.CDLL:
    """The library whose pkv_bm_* functions BlockManager calls: libpagedkv.so,
    unless $PKV_BM_LIB names a host-only build of the block manager (the tests
    build one with the address and undefined-behaviour sanitizers and run the
    block-manager suite against it). Only the block manager's symbols (pkv_bm_*
    and pkv_status_str) are bound then."""
    global _bm_lib
    path = os.environ.get("PKV_BM_LIB")
    if not path:
        return load()
    if _bm_lib is None:
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            if name.startswith("pkv_bm_") or name == "pkv_status_str":
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
        _bm_lib = lib
    return _bm_lib


class PkvError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = load_block_manager().pkv_status_str(code).decode()
        super().__init__(f"{where}: {msg} ({code})")
        self.code = code


def check(code: int, where: str) -> None:
    if code != PKV_OK:
        raise PkvError(code, where)
