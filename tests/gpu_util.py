"""Helpers for the GPU parity tests (the HIP path through the C ABI vs the oracle)."""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import torch

TOL = {"f16": (2e-3, 1e-2), "fp8": (3e-2, 1e-2), "fp8_e5m2": (3e-2, 1e-2)}  # (atol, rtol) per KV dtype

# Threads for the oracle's per-sequence attention at full size (the host share
# of a one-GPU MI355X node is 16 cores); PKV_ORACLE_THREADS overrides.
ORACLE_THREADS = int(os.environ.get("PKV_ORACLE_THREADS", "16"))

# Block slice for bit-exact cache comparisons (bounded host memory: a slice of
# 1024 blocks is 160 MiB at 40 KV heads x 32 slots x 128 x fp16).
CACHE_SLICE_BLOCKS = 1024
# seeded random draws per randomized parity test (more with PKV_RANDOM_DRAWS)
RANDOM_DRAWS = int(os.environ.get("PKV_RANDOM_DRAWS", "24"))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def record_error(what, kv_dtype, max_abs, max_rel_excess, n):
    """Append one observed-error record to $PKV_ERR_RECORD (JSON lines), if set."""
    path = os.environ.get("PKV_ERR_RECORD")
    if not path:
        return
    with open(path, "a") as f:
        f.write(json.dumps({"what": what, "kv_dtype": kv_dtype, "max_abs_err": max_abs,
                            "max_err_over_bound": max_rel_excess, "n": n}) + "\n")


def assert_close_to_oracle(gpu_out, ref, kv_dtype, what="", partial=False):
    """|gpu - ref| <= atol + rtol*|ref| elementwise.

    Every GPU output must be finite (unused cache slots are NaN, so this also
    shows that no output read one). The reference must define every entry
    unless partial=True (then only the entries it defines are compared).
    Returns the largest absolute error."""
    atol, rtol = TOL[kv_dtype]
    g = np.asarray(gpu_out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, f"{what}: shape {g.shape} vs {ref.shape}"
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output ({int((~np.isfinite(g)).sum())} entries)"
    mask = ~np.isnan(ref)
    if not partial:
        assert mask.all(), f"{what}: the oracle left {int((~mask).sum())} entries undefined"
    if not mask.any():
        return 0.0
    err = np.abs(g[mask] - ref[mask])
    bound = atol + rtol * np.abs(ref[mask])
    worst = float((err - bound).max())
    assert (err <= bound).all(), f"{what}: max excess {worst:.3e}, max abs err {err.max():.3e}"
    ratio = float((err / bound).max())
    record_error(what, kv_dtype, float(err.max()), ratio, int(mask.sum()))
    return float(err.max())


def assert_caches_bit_exact(gpu_cache: torch.Tensor, oracle_cache: np.ndarray, what=""):
    """Bit-for-bit comparison of a device cache with the oracle's, one slice of
    blocks at a time so host memory stays bounded for pools of several GiB."""
    nb = gpu_cache.shape[0]
    assert tuple(gpu_cache.shape) == tuple(oracle_cache.shape), f"{what}: cache shape"
    ob = oracle_bits(oracle_cache)
    for b0 in range(0, nb, CACHE_SLICE_BLOCKS):
        b1 = min(nb, b0 + CACHE_SLICE_BLOCKS)
        got = cache_bits(gpu_cache[b0:b1])
        if not np.array_equal(got, ob[b0:b1]):
            bad = np.argwhere((got != ob[b0:b1]).reshape(b1 - b0, -1).any(axis=1)).ravel()
            raise AssertionError(f"{what}: blocks differ, first {[int(b0 + i) for i in bad[:8]]}")


def cache_bits(t: torch.Tensor) -> np.ndarray:
    c = t.cpu()
    if c.dtype == torch.float16:
        return c.view(torch.int16).numpy().view(np.uint16)
    return c.numpy()


def oracle_bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint16) if a.dtype == np.float16 else a


