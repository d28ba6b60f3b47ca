"""Pins for the oracle's cache writes, gather and decode attention.

* Library pin: PyTorch's scaled_dot_product_attention in float64 on the
  logical (contiguous) K/V, including grouped-query heads (enable_gqa, which
  maps query head h to KV head h // group).
* Closed forms: one token gives V[0]; constant V gives V; identical keys give
  the mean of V.
* The block-table figure of "From OOM to Smooth Inference", §2.1 for the
  slot -> (block, offset) mapping.
* Whole pipeline (allocator + scatter + copy-on-write + gather + attention)
  against SDPA on K/V assembled from the workload script's own meaning
  (shared prefix, forked prompt, private tails), at reduced sizes.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import attention, cache_ops, fp8, runner
from tests import alloc_driver


def sdpa64(q, K, V, scale):
    """q [Hq, D], K/V [L, Hkv, D] -> [Hq, D] via torch SDPA in float64."""
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))[None, :, None, :]  # [1,Hq,1,D]
    kt = torch.from_numpy(np.ascontiguousarray(np.transpose(K, (1, 0, 2)), dtype=np.float64))[None]
    vt = torch.from_numpy(np.ascontiguousarray(np.transpose(V, (1, 0, 2)), dtype=np.float64))[None]
    gqa = qt.shape[1] != kt.shape[1]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=gqa)
    return o[0, :, 0, :].numpy()


def _random_paged(seed, lengths, hq, hkv, d, bs, nb):
    g = np.random.default_rng(seed)
    perm = g.permutation(nb)
    kc = runner.empty_cache(nb, hkv, bs, d, "f16")
    vc = runner.empty_cache(nb, hkv, bs, d, "f16")
    tables, logical, pos = [], [], 0
    for L in lengths:
        nblk = -(-L // bs)
        t = perm[pos:pos + nblk].tolist()
        pos += nblk
        K = g.standard_normal((L, hkv, d)).astype(np.float16)
        V = g.standard_normal((L, hkv, d)).astype(np.float16)
        slots = [t[p // bs] * bs + p % bs for p in range(L)]
        cache_ops.scatter(kc, vc, K, V, slots, bs)
        tables.append(t)
        logical.append((K, V))
    q = g.standard_normal((len(lengths), hq, d)).astype(np.float16)
    return q, kc, vc, tables, logical


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (6, 1)])
def test_paged_matches_sdpa(hq, hkv):
    lengths = [1, 5, 16, 17, 40]
    d, bs = 32, 4 if hq != 6 else 16
    nb = sum(-(-L // bs) for L in lengths) + 3
    q, kc, vc, tables, logical = _random_paged(11, lengths, hq, hkv, d, bs, nb)
    scale = 1.0 / np.sqrt(d)
    out = attention.decode_attention(q, kc, vc, tables, lengths, bs, scale)
    for s, (K, V) in enumerate(logical):
        ref = sdpa64(q[s].astype(np.float64), K.astype(np.float64), V.astype(np.float64), scale)
        np.testing.assert_allclose(out[s], ref, rtol=1e-12, atol=1e-12)


def test_single_token_gives_v0():
    q, kc, vc, tables, logical = _random_paged(3, [1, 1], 4, 4, 16, 4, 4)
    out = attention.decode_attention(q, kc, vc, tables, [1, 1], 4, 0.25)
    for s in range(2):
        assert np.array_equal(out[s], logical[s][1][0].astype(np.float64))


def test_constant_v_and_identical_keys():
    g = np.random.default_rng(5)
    L, d = 37, 16
    q = g.standard_normal(d)
    K = g.standard_normal((L, d))
    V = np.tile(g.standard_normal(d), (L, 1))
    np.testing.assert_allclose(attention.attend_one(q, K, V, 0.3), V[0], rtol=1e-14, atol=1e-14)
    K2 = np.tile(g.standard_normal(d), (L, 1))
    V2 = g.standard_normal((L, d))
    np.testing.assert_allclose(attention.attend_one(q, K2, V2, 0.3), V2.mean(0), rtol=1e-13, atol=1e-13)


def test_zero_and_negative_scales():
    """Scale 0: every visible token weighs the same (the mean of V). A negative
    scale is the positive one applied to -q. Both against a direct evaluation
    of the softmax by an independent route (scipy's logsumexp)."""
    from scipy.special import logsumexp
    g = np.random.default_rng(11)
    L, d = 53, 32
    q, K, V = g.standard_normal(d), g.standard_normal((L, d)), g.standard_normal((L, d))
    np.testing.assert_allclose(attention.attend_one(q, K, V, 0.0), V.mean(0), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(attention.attend_one(q, K, V, -0.4), attention.attend_one(-q, K, V, 0.4),
                               rtol=1e-13, atol=1e-13)
    z = -0.4 * (K @ q)
    w = np.exp(z - logsumexp(z))
    np.testing.assert_allclose(attention.attend_one(q, K, V, -0.4), w @ V, rtol=1e-12, atol=1e-12)


def test_zero_length_is_zero():
    assert np.array_equal(attention.attend_one(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)), 1.0),
                          np.zeros(4))


def test_block_table_figure():
    fx = alloc_driver.load("block_table_figure.json")
    bs, nb = fx["block_size"], fx["num_blocks"]
    kc = runner.empty_cache(nb, 1, bs, 2, "f16")
    vc = runner.empty_cache(nb, 1, bs, 2, "f16")
    n = fx["tokens"]
    K = np.arange(n, dtype=np.float16).reshape(n, 1, 1).repeat(2, axis=2)
    V = -K
    slots = [fx["table"][t // bs] * bs + t % bs for t in range(n)]
    cache_ops.scatter(kc, vc, K, V, slots, bs)
    for lo, hi, phys in fx["expected_block_of_token_ranges"]:
        assert np.array_equal(kc[phys, 0, :, 0], np.arange(lo, hi + 1, dtype=np.float16))
        assert np.array_equal(vc[phys, 0, :, 1], -np.arange(lo, hi + 1, dtype=np.float16))
    got = attention.gather_sequence(kc, fx["table"], n, bs)
    assert np.array_equal(got[:, 0, 0], np.arange(n, dtype=np.float64))


def test_scatter_skips_minus_one_and_block_copy():
    kc = runner.empty_cache(4, 2, 4, 8, "f16")
    vc = runner.empty_cache(4, 2, 4, 8, "f16")
    before_k = kc.view(np.uint16).copy()
    K = np.ones((3, 2, 8), np.float16)
    cache_ops.scatter(kc, vc, K, K * 2, [5, -1, 14], 4)
    # slot 5 -> block 1 offset 1, slot 14 -> block 3 offset 2; nothing else changes
    changed = np.argwhere((kc.view(np.uint16) != before_k).any(axis=(1, 3)))
    assert changed.tolist() == [[1, 1], [3, 2]]
    assert np.all(kc[1, :, 1] == 1) and np.all(kc[3, :, 2] == 1) and np.all(vc[3, :, 2] == 2)
    cache_ops.block_copy(kc, vc, [(3, 0)])
    assert np.array_equal(kc[0].view(np.uint16), kc[3].view(np.uint16))
    assert np.array_equal(vc[0].view(np.uint16), vc[3].view(np.uint16))


@pytest.mark.parametrize("kv_dtype,per_head", [("fp8", False), ("fp8_e5m2", False), ("fp8", True),
                                               ("fp8_e5m2", True)])
def test_fp8_cache_matches_sdpa_on_dequantized_values(kv_dtype, per_head):
    """fp8 caches (e4m3 or e5m2, one scale per tensor or per KV head) attend like
    SDPA on the values torch's own fp8 conversion gives for the same scaled data."""
    g = np.random.default_rng(9)
    L, hkv, hq, d, bs = 23, 2, 8, 16, 8
    K = g.standard_normal((L, hkv, d)).astype(np.float16)
    V = g.standard_normal((L, hkv, d)).astype(np.float16)
    V[:, 1] *= 40  # the heads' ranges differ, so per-head scales differ
    fmax = np.float32(448 if kv_dtype == "fp8" else 57344)
    tdt = torch.float8_e4m3fn if kv_dtype == "fp8" else torch.float8_e5m2
    if per_head:
        ks = np.abs(K).max(axis=(0, 2)).astype(np.float32) / fmax
        vs = np.abs(V).max(axis=(0, 2)).astype(np.float32) / fmax
    else:
        ks, vs = np.float32(np.abs(K).max()) / fmax, np.float32(np.abs(V).max()) / fmax
    kinv, vinv = np.float32(1) / ks, np.float32(1) / vs
    kc = runner.empty_cache(4, hkv, bs, d, kv_dtype)
    vc = runner.empty_cache(4, hkv, bs, d, kv_dtype)
    table = [2, 0, 3]
    slots = [table[p // bs] * bs + p % bs for p in range(L)]
    cache_ops.scatter(kc, vc, K, V, slots, bs, kv_dtype, kinv, vinv)
    q = g.standard_normal((1, hq, d)).astype(np.float16)
    out = attention.decode_attention(q, kc, vc, [table], [L], bs, 0.25, kv_dtype, ks, vs)
    # library route for the same quantised values: torch's fp8 conversion, per head
    bk = np.broadcast_to(kinv, (hkv,)).astype(np.float32)[None, :, None]
    bv = np.broadcast_to(vinv, (hkv,)).astype(np.float32)[None, :, None]
    sk = np.broadcast_to(ks, (hkv,)).astype(np.float64)[None, :, None]
    sv = np.broadcast_to(vs, (hkv,)).astype(np.float64)[None, :, None]
    kq = torch.from_numpy(K.astype(np.float32) * bk).to(tdt).to(torch.float64).numpy() * sk
    vq = torch.from_numpy(V.astype(np.float32) * bv).to(tdt).to(torch.float64).numpy() * sv
    ref = sdpa64(q[0].astype(np.float64), kq, vq, 0.25)
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-12)
    # and close to the unquantised result (relative precision ~1/16 for e4m3, ~1/8 for e5m2)
    ref16 = sdpa64(q[0].astype(np.float64), K.astype(np.float64), V.astype(np.float64), 0.25)
    assert np.abs(out[0] - ref16).max() < (0.1 if kv_dtype == "fp8" else 0.2) * np.abs(V).max() / 4


# ---------------------------------------------------- whole-pipeline pins
def logical_kv(wl, steps):
    """Per batch sequence, its K/V rows in logical order, assembled from what
    the script means (who owns which tokens), with no allocator involved."""
    owned = {}  # seq -> list of (K, V) segments
    for ops in wl.setup_rounds + [wl.step_ops(s) for s in range(steps)]:
        for op in ops:
            if op.kind in ("allocate", "append"):
                if op.kind == "allocate":
                    owned[op.seq] = []
                if op.n:
                    owned[op.seq].append(wl.op_kv(op))
            elif op.kind == "fork":
                owned[op.seq] = list(owned[op.src])
            elif op.kind == "share_prefix":
                # the workloads share whole blocks of a prefix that is the
                # source's first allocation
                segs, need, out = owned[op.src], op.n * wl.block_size, []
                for k, v in segs:
                    take = min(need, k.shape[0])
                    if take:
                        out.append((k[:take], v[:take]))
                    need -= take
                owned[op.seq] = out
    res = []
    for s in wl.batch:
        K = np.concatenate([k for k, _ in owned[s]])
        V = np.concatenate([v for _, v in owned[s]])
        res.append((K, V))
    return res


def _check_pipeline(wl, steps, sample=None):
    run = runner.run(wl, steps=steps)
    lk = logical_kv(wl, steps)
    out = run.outputs[-1]
    q = wl.queries(steps - 1)
    seqs = range(len(wl.batch)) if sample is None else sample
    for s in seqs:
        K, V = lk[s]
        assert K.shape[0] == run.ctx_lens[-1][s]
        if wl.kv_dtype != "f16":
            # torch's own fp8 conversion of the scaled values; scales per tensor or per KV head
            tdt = torch.float8_e4m3fn if wl.kv_dtype == "fp8" else torch.float8_e5m2
            hs = lambda x, dt: np.broadcast_to(np.asarray(x, dtype=dt), (wl.num_kv_heads,))[None, :, None]  # noqa: E731
            K = torch.from_numpy(K.astype(np.float32) * hs(wl.k_inv_scale, np.float32)).to(
                tdt).to(torch.float64).numpy() * hs(wl.k_scale, np.float64)
            V = torch.from_numpy(V.astype(np.float32) * hs(wl.v_inv_scale, np.float32)).to(
                tdt).to(torch.float64).numpy() * hs(wl.v_scale, np.float64)
        ref = sdpa64(q[s].astype(np.float64), K.astype(np.float64), V.astype(np.float64), wl.sm_scale)
        np.testing.assert_allclose(out[s], ref, rtol=1e-11, atol=1e-12)
    return run


def test_pipeline_tiny_two_steps():
    wl = workloads.tiny()
    run = _check_pipeline(wl, 2)
    assert run.ctx_lens[-1] == [38, 101, 17, 251]
    assert [len(t) for t in run.tables[-1]] == [3, 7, 2, 16]


def test_pipeline_shared_prefix_small():
    wl = workloads.qwen3_prefix(batch=5, max_steps=2)
    run = _check_pipeline(wl, 1)
    for s in range(1, 5):
        assert run.tables[-1][s][:64] == run.tables[-1][0][:64]
    assert run.alloc.refcount(run.tables[-1][0][0]) == 5


@pytest.mark.parametrize("kv_dtype,per_head", [("fp8", False), ("fp8_e5m2", True)])
def test_pipeline_beam_fp8_small(kv_dtype, per_head):
    wl = workloads.beam_fp8(prompts=3, max_steps=2, kv_dtype=kv_dtype, per_head=per_head)
    run = _check_pipeline(wl, 1)
    # every beam shares its prompt's full blocks
    for i in range(3):
        full = wl.meta["prompts"][i] // wl.block_size
        t0 = run.tables[-1][4 * i]
        for b in range(1, 4):
            assert run.tables[-1][4 * i + b][:full] == t0[:full]


def test_kv_fp8_scale_maps_max_to_448():
    wl = workloads.beam_fp8(prompts=2, max_steps=1)
    kmax = 0.0
    for r in wl.setup_rounds + [wl.step_ops(0)]:
        for op in r:
            if op.creates_tokens:
                k, _ = wl.op_kv(op)
                kmax = max(kmax, float(np.abs(k.astype(np.float32)).max()))
    assert fp8.encode(np.float32(kmax) * np.float32(wl.k_inv_scale)) == 0x7E
