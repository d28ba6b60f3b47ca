"""GPU parity of paged_kv_write and paged_block_copy against the oracle (bit-exact).

Runs the HIP kernels through the C ABI (paged_kv_cache_60_amd.ops -> ctypes)
and compares every byte of both caches with the oracle's scatter / block copy
applied to the same NaN-poisoned starting caches.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import cache_ops, fp8, runner
from paged_kv_cache_60_amd import ops
from tests.gpu_util import RANDOM_DRAWS, cache_bits, log, oracle_bits

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _caches(nb, hkv, bs, d, kv_dtype):
    o_k = runner.empty_cache(nb, hkv, bs, d, kv_dtype)
    o_v = runner.empty_cache(nb, hkv, bs, d, kv_dtype)
    if kv_dtype == "f16":
        g_k = torch.from_numpy(o_k.view(np.int16).copy()).view(torch.float16).to(DEV)
        g_v = torch.from_numpy(o_v.view(np.int16).copy()).view(torch.float16).to(DEV)
    else:
        g_k = torch.from_numpy(o_k.copy()).to(DEV)
        g_v = torch.from_numpy(o_v.copy()).to(DEV)
    return o_k, o_v, g_k, g_v


@pytest.mark.parametrize("kv_dtype", ["f16", "fp8", "fp8_e5m2"])
@pytest.mark.parametrize("hkv,d,bs", [(8, 64, 16), (32, 128, 16), (40, 128, 32), (8, 128, 64)])
def test_kv_write_bit_exact(kv_dtype, hkv, d, bs):
    log(f"kv_write {kv_dtype} hkv={hkv} d={d} bs={bs}")
    g = np.random.default_rng(hkv * 1000 + d + bs)
    nb = 24
    T = 150
    slots = g.permutation(nb * bs)[:T].astype(np.int64)
    slots[::17] = -1                       # skipped tokens
    slots[5] = nb * bs + 3                 # out of range: skipped
    slots[6] = -7                          # negative: skipped
    K = g.standard_normal((T, hkv, d), dtype=np.float32).astype(np.float16)
    V = (3 * g.standard_normal((T, hkv, d), dtype=np.float32)).astype(np.float16)
    kinv, vinv = (1.0, 1.0) if kv_dtype == "f16" else (float(np.float32(448) / np.float32(4.5)), 37.0)
    o_k, o_v, g_k, g_v = _caches(nb, hkv, bs, d, kv_dtype)
    o_slots = np.where((slots >= 0) & (slots < nb * bs), slots, -1)
    cache_ops.scatter(o_k, o_v, K, V, o_slots, bs, kv_dtype, kinv, vinv)
    ops.paged_kv_write(torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV), g_k, g_v,
                       torch.from_numpy(slots).to(DEV), kv_dtype, kinv, vinv)
    torch.cuda.synchronize()
    assert np.array_equal(cache_bits(g_k), oracle_bits(o_k))
    assert np.array_equal(cache_bits(g_v), oracle_bits(o_v))


@pytest.mark.parametrize("kv_dtype,inv_scale", [("fp8", 1.0), ("fp8", 448.0 / 5.25), ("fp8", 0.731), ("fp8", 81.37),
                                               ("fp8_e5m2", 1.0), ("fp8_e5m2", 57344.0 / 5.25),
                                               ("fp8_e5m2", 0.731), ("fp8_e5m2", 4096.0)])
def test_kv_write_fp8_every_fp16_value(kv_dtype, inv_scale):
    """Every fp16 bit pattern through the device encoder, against the oracle codec:
    finite values round to nearest even and saturate, infinities saturate with
    their sign, NaNs become 0x7F."""
    log(f"{kv_dtype} exhaustive inv_scale={inv_scale}")
    fmt = fp8.KV_FORMATS[kv_dtype]
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16)
    d, hkv, bs = 128, 1, 16
    n = len(x)
    T = -(-n // d)
    pad = np.zeros(T * d - n, dtype=np.float16)
    K = np.concatenate([x, pad]).reshape(T, hkv, d)
    V = -K
    nb = -(-T // bs)
    slots = np.arange(T, dtype=np.int64)
    kinv = float(np.float32(inv_scale))
    o_k, o_v, g_k, g_v = _caches(nb, hkv, bs, d, kv_dtype)
    ops.paged_kv_write(torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV), g_k, g_v,
                       torch.from_numpy(slots).to(DEV), kv_dtype, kinv, kinv)
    torch.cuda.synchronize()
    got = cache_bits(g_k).reshape(-1)[:T * d][:n]
    want = fp8.quantize(x, kinv, fmt)
    assert np.array_equal(got, want)
    gotv = cache_bits(g_v).reshape(-1)[:T * d][:n]
    assert np.array_equal(gotv, fp8.quantize(-x, kinv, fmt))


@pytest.mark.parametrize("kv_dtype", ["fp8", "fp8_e5m2"])
def test_kv_write_per_head_scales_bit_exact(kv_dtype):
    """One multiplier per KV head (paged_kv_write_scaled), against the oracle."""
    g = np.random.default_rng(21)
    nb, hkv, bs, d, T = 20, 8, 16, 128, 200
    slots = g.permutation(nb * bs)[:T].astype(np.int64)
    K = (g.standard_normal((T, hkv, d), dtype=np.float32) * np.arange(1, hkv + 1)[None, :, None]).astype(np.float16)
    V = g.standard_normal((T, hkv, d), dtype=np.float32).astype(np.float16)
    fmax = np.float32(448 if kv_dtype == "fp8" else 57344)
    kinv = fmax / np.abs(K.astype(np.float32)).max(axis=(0, 2))
    vinv = (fmax / np.abs(V.astype(np.float32)).max(axis=(0, 2))).astype(np.float32)
    kinv = kinv.astype(np.float32)
    o_k, o_v, g_k, g_v = _caches(nb, hkv, bs, d, kv_dtype)
    cache_ops.scatter(o_k, o_v, K, V, slots, bs, kv_dtype, kinv, vinv)
    ops.paged_kv_write(torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV), g_k, g_v,
                       torch.from_numpy(slots).to(DEV), kv_dtype, torch.from_numpy(kinv).to(DEV),
                       torch.from_numpy(vinv).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(cache_bits(g_k), oracle_bits(o_k))
    assert np.array_equal(cache_bits(g_v), oracle_bits(o_v))


@pytest.mark.parametrize("kv_dtype", ["f16", "fp8"])
def test_block_copy_bit_exact(kv_dtype):
    g = np.random.default_rng(3)
    nb, hkv, bs, d = 40, 8, 64, 128
    o_k, o_v, g_k, g_v = _caches(nb, hkv, bs, d, kv_dtype)
    # fill some blocks with data first
    T = 20 * bs
    slots = np.arange(T, dtype=np.int64)
    K = g.standard_normal((T, hkv, d), dtype=np.float32).astype(np.float16)
    V = g.standard_normal((T, hkv, d), dtype=np.float32).astype(np.float16)
    cache_ops.scatter(o_k, o_v, K, V, slots, bs, kv_dtype, 50.0, 50.0)
    ops.paged_kv_write(torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV), g_k, g_v,
                       torch.from_numpy(slots).to(DEV), kv_dtype, 50.0, 50.0)
    pairs = [(0, 30), (5, 31), (19, 25), (3, 39), (7, -1), (50, 2)]  # last two skipped
    cache_ops.block_copy(o_k, o_v, [p for p in pairs if 0 <= p[0] < nb and 0 <= p[1] < nb])
    ops.paged_block_copy(g_k, g_v, torch.tensor(pairs, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert np.array_equal(cache_bits(g_k), oracle_bits(o_k))
    assert np.array_equal(cache_bits(g_v), oracle_bits(o_v))


def test_block_copy_config5_scale():
    """Copy-on-write pairs of the beam workload, replayed on both sides."""
    wl = workloads.beam_fp8(prompts=4, max_steps=1)
    from paged_kv_cache_60_amd import harness
    eng = harness.make_engine(wl)
    harness.replay_setup(eng, wl)
    o = runner.run(wl, steps=0)
    assert np.array_equal(cache_bits(eng.k_cache), oracle_bits(o.k_cache))
    assert np.array_equal(cache_bits(eng.v_cache), oracle_bits(o.v_cache))


def _meta_case(seed, B=37, maxb=11, n_upd=20):
    g = np.random.default_rng(seed)
    tables = g.integers(-1, 500, size=(B, maxb), dtype=np.int32)
    upd = np.stack([g.integers(0, B, n_upd), g.integers(0, maxb, n_upd), g.integers(0, 500, n_upd)], 1)
    upd = upd.astype(np.int32)
    upd[3] = (B, 0, 7)          # row out of range: skipped
    upd[4] = (0, maxb, 7)       # index out of range: skipped
    upd[5] = (-1, 2, 7)
    # later updates win when two address the same entry; keep entries distinct here
    _, first = np.unique(upd[:, 0] * 1000 + upd[:, 1], return_index=True)
    upd = upd[np.sort(first)]
    expect = tables.copy()
    for r, i, b in upd.tolist():
        if 0 <= r < B and 0 <= i < maxb:
            expect[r, i] = b
    ctx = g.integers(0, 4000, size=B, dtype=np.int32)
    return tables, upd, ctx, expect


def _pinned(a):
    t = torch.from_numpy(np.ascontiguousarray(a)).pin_memory()
    return t


def test_step_metadata_bit_exact():
    tables, upd, ctx, expect = _meta_case(1)
    B = len(ctx)
    slots = np.random.default_rng(2).integers(-1, 10 ** 6, size=B).astype(np.int64)
    cow = np.random.default_rng(3).integers(0, 100, size=(5, 2)).astype(np.int32)
    t_dev = torch.from_numpy(tables).to(DEV)
    s_dev = torch.empty(B, dtype=torch.int64, device=DEV)
    c_dev = torch.empty(B, dtype=torch.int32, device=DEV)
    cw_dev = torch.empty((5, 2), dtype=torch.int32, device=DEV)
    ops.paged_step_metadata(_pinned(slots), s_dev, _pinned(ctx), c_dev, B, _pinned(cow), cw_dev, 5,
                            _pinned(upd.reshape(-1)), len(upd), t_dev)
    torch.cuda.synchronize()
    assert np.array_equal(t_dev.cpu().numpy(), expect)
    assert np.array_equal(s_dev.cpu().numpy(), slots)
    assert np.array_equal(c_dev.cpu().numpy(), ctx)
    assert np.array_equal(cw_dev.cpu().numpy(), cow)


@pytest.mark.parametrize("kv_dtype", ["f16", "fp8"])
@pytest.mark.parametrize("where,B,n_upd", [("pinned", 37, 20), ("pinned", 128, 128), ("pinned", 200, 150),
                                           ("device", 37, 20)])
def test_kv_write_step_bit_exact(kv_dtype, where, B, n_upd):
    """The write kernel of a decode step: small steps with pinned metadata
    travel in the launch's arguments (up to 128 tokens, lengths and updates),
    larger ones and device metadata are read by the kernel; same bits."""
    tables, upd, ctx, expect = _meta_case(4, B=B, n_upd=n_upd)
    g = np.random.default_rng(5)
    nb, hkv, bs, d = 40, 8, 16, 128
    slots = g.permutation(nb * bs)[:B].astype(np.int64)
    slots[::7] = -1
    slots[5] = nb * bs + 3   # past the pool: skipped
    slots[12] = 1 << 40      # past 32 bits: skipped
    K = g.standard_normal((B, hkv, d), dtype=np.float32).astype(np.float16)
    V = g.standard_normal((B, hkv, d), dtype=np.float32).astype(np.float16)
    o_k, o_v, g_k, g_v = _caches(nb, hkv, bs, d, kv_dtype)
    cache_ops.scatter(o_k, o_v, K, V, np.where(slots < nb * bs, slots, -1), bs, kv_dtype, 61.0, 61.0)
    t_dev = torch.from_numpy(tables).to(DEV)
    c_dev = torch.full((B,), -5, dtype=torch.int32, device=DEV)
    put = _pinned if where == "pinned" else (lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV))
    ops.paged_kv_write_step(torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV), g_k, g_v, put(slots),
                            put(ctx), c_dev, put(upd.reshape(-1)), len(upd), t_dev, kv_dtype, 61.0, 61.0)
    torch.cuda.synchronize()
    assert np.array_equal(cache_bits(g_k), oracle_bits(o_k))
    assert np.array_equal(cache_bits(g_v), oracle_bits(o_v))
    assert np.array_equal(t_dev.cpu().numpy(), expect)
    assert np.array_equal(c_dev.cpu().numpy(), ctx)


def test_debug_checks_refuse_racing_slots_and_pairs_before_queuing():
    """With the opt-in race guards on, a slot mapping with two valid tokens on one
    slot, or copy pairs where one pair writes another's source, raise before any
    launch and leave the caches untouched; valid inputs still run and match the
    oracle with the guards on."""
    from paged_kv_cache_60_amd import guards
    from paged_kv_cache_60_amd._lib import PkvError
    log("debug checks: racing slots and pairs refused")
    nb, hkv, bs, d = 8, 4, 16, 64
    o_k, o_v, g_k, g_v = _caches(nb, hkv, bs, d, "f16")
    before_k, before_v = cache_bits(g_k), cache_bits(g_v)
    g = np.random.default_rng(7)
    k_new = torch.from_numpy(g.standard_normal((3, hkv, d)).astype(np.float16)).to(DEV)
    v_new = torch.from_numpy(g.standard_normal((3, hkv, d)).astype(np.float16)).to(DEV)
    was = guards.debug_checks()
    try:
        guards.set_debug_checks(True)
        dup = torch.tensor([5, 17, 5], dtype=torch.int64, device=DEV)
        with pytest.raises(PkvError):
            ops.paged_kv_write(k_new, v_new, g_k, g_v, dup)
        pairs = torch.tensor([[0, 3], [3, 6]], dtype=torch.int32, device=DEV)
        with pytest.raises(PkvError):
            ops.paged_block_copy(g_k, g_v, pairs)
        torch.cuda.synchronize()
        assert np.array_equal(cache_bits(g_k), before_k) and np.array_equal(cache_bits(g_v), before_v)
        # valid inputs pass the guards and give the oracle's bytes
        slots = np.array([5, 17, -1], dtype=np.int64)
        ops.paged_kv_write(k_new, v_new, g_k, g_v, torch.from_numpy(slots).to(DEV))
        ok_pairs = np.array([[0, 3], [1, 6]], dtype=np.int32)
        ops.paged_block_copy(g_k, g_v, torch.from_numpy(ok_pairs).to(DEV))
        torch.cuda.synchronize()
    finally:
        guards.set_debug_checks(was)
    cache_ops.scatter(o_k, o_v, k_new.cpu().numpy(), v_new.cpu().numpy(), slots, bs)
    cache_ops.block_copy(o_k, o_v, ok_pairs)
    assert np.array_equal(cache_bits(g_k), oracle_bits(o_k))
    assert np.array_equal(cache_bits(g_v), oracle_bits(o_v))



@pytest.mark.parametrize("seed", range(RANDOM_DRAWS))
def test_random_writes_and_copies(seed):
    """Seeded random scatters and copies, bit-exact against the oracle: a
    shape (1-40 KV heads, D 64/128, block size 16/32/64, fp16/e4m3/e5m2 with
    a random multiplier per tensor or per KV head), 0-3000 tokens on distinct
    slots of which some are -1, negative or past the pool, then disjoint copy
    pairs of which some point outside the pool."""
    g = np.random.default_rng(9000 + seed)
    hkv = int(g.choice([1, 2, 8, 32, 40]))
    d = int(g.choice([64, 128]))
    bs = int(g.choice([16, 32, 64]))
    kv = str(g.choice(["f16", "fp8", "fp8_e5m2"]))
    nb = int(g.integers(2, 80))
    T = int(g.integers(0, min(3000, nb * bs) + 1))
    log(f"random write {seed}: hkv={hkv} d={d} bs={bs} {kv} nb={nb} T={T}")
    slots = g.permutation(nb * bs)[:T].astype(np.int64)
    bad = g.random(T)
    slots[bad < 0.05] = -1
    slots[(bad >= 0.05) & (bad < 0.08)] = -3
    slots[(bad >= 0.08) & (bad < 0.10)] = nb * bs + 5
    K = (g.standard_normal((T, hkv, d), dtype=np.float32) * float(g.choice([0.1, 1.0, 30.0]))).astype(np.float16)
    V = g.standard_normal((T, hkv, d), dtype=np.float32).astype(np.float16)
    o_k, o_v, g_k, g_v = _caches(nb, hkv, bs, d, kv)
    o_slots = np.where((slots >= 0) & (slots < nb * bs), slots, -1)
    if kv != "f16" and g.random() < 0.5:
        kinv = (g.random(hkv) * 200 + 0.5).astype(np.float32)
        vinv = (g.random(hkv) * 200 + 0.5).astype(np.float32)
        ka, va = torch.from_numpy(kinv).to(DEV), torch.from_numpy(vinv).to(DEV)
    else:
        kinv = vinv = 1.0 if kv == "f16" else float(np.float32(g.random() * 200 + 0.5))
        ka = va = kinv
    cache_ops.scatter(o_k, o_v, K, V, o_slots, bs, kv, kinv, vinv)
    if T:
        ops.paged_kv_write(torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV), g_k, g_v,
                           torch.from_numpy(slots).to(DEV), kv, ka, va)
    # disjoint pairs: sources and destinations drawn without repeats
    perm = g.permutation(nb)
    n = int(g.integers(0, nb // 2 + 1))
    pairs = [(int(perm[i]), int(perm[nb - 1 - i])) for i in range(n)]
    for i in range(len(pairs)):
        r = g.random()
        if r < 0.1:
            pairs[i] = (pairs[i][0], nb + 3)
        elif r < 0.2:
            pairs[i] = (-2, pairs[i][1])
    cache_ops.block_copy(o_k, o_v, [p for p in pairs if 0 <= p[0] < nb and 0 <= p[1] < nb])
    if pairs:
        ops.paged_block_copy(g_k, g_v, torch.tensor(pairs, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert np.array_equal(cache_bits(g_k), oracle_bits(o_k))
    assert np.array_equal(cache_bits(g_v), oracle_bits(o_v))
