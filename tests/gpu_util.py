"""Helpers for the GPU parity tests (the HIP path through the C ABI vs the oracle)."""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL = {"f16": (2e-3, 1e-2), "fp8": (3e-2, 1e-2), "fp8_e5m2": (3e-2, 1e-2)}  # (atol, rtol) per KV dtype


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def assert_close_to_oracle(gpu_out, ref, kv_dtype, what=""):
    """|gpu - ref| <= atol + rtol*|ref| elementwise, on the entries ref defines."""
    atol, rtol = TOL[kv_dtype]
    g = np.asarray(gpu_out, dtype=np.float64)
    mask = ~np.isnan(ref)
    assert mask.any()
    err = np.abs(g[mask] - ref[mask])
    bound = atol + rtol * np.abs(ref[mask])
    worst = float((err - bound).max())
    assert np.isfinite(g[mask]).all(), f"{what}: non-finite GPU output"
    assert (err <= bound).all(), f"{what}: max excess {worst:.3e}, max abs err {err.max():.3e}"
    return float(err.max())


def cache_bits(t: torch.Tensor) -> np.ndarray:
    c = t.cpu()
    if c.dtype == torch.float16:
        return c.view(torch.int16).numpy().view(np.uint16)
    return c.numpy()


def oracle_bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint16) if a.dtype == np.float16 else a


def sample_seqs(lengths, n=6, seed=0):
    """Shortest, longest and a few seeded others (batch positions)."""
    L = np.asarray(lengths)
    pick = {int(L.argmin()), int(L.argmax())}
    g = np.random.default_rng(seed)
    while len(pick) < min(n, len(L)):
        pick.add(int(g.integers(len(L))))
    return sorted(pick)
