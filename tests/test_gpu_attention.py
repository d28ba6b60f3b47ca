"""GPU parity of paged_attn_decode (and the whole decode step) against the oracle.

Each workload script is replayed on the GPU through the engine (C++ block
manager + paged_block_copy + paged_kv_write + paged_attn_decode through the C
ABI) and through the oracle. Caches are compared bit for bit after the setup;
attention outputs are compared elementwise with |gpu - ref| <= atol + rtol|ref|,
(2e-3, 1e-2) for fp16 KV and (3e-2, 1e-2) for fp8 KV (the oracle runs on the same
fp8 bytes). Every output of every sequence, head and step is compared, at full
size too (the oracle spreads sequences over host threads there), and every GPU
output must be finite. All caches start NaN-poisoned, so a finite output also
shows no unused slot was read. Full-size caches are compared bit for bit one
slice of blocks at a time.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import attention as oattn
from oracle import runner
from paged_kv_cache_60_amd import harness, ops
from tests.gpu_util import (ORACLE_THREADS, RANDOM_DRAWS, assert_caches_bit_exact, assert_close_to_oracle, cache_bits, log,
                            oracle_bits)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gpu_run(wl, steps, partition_tokens=0):
    eng = harness.make_engine(wl)
    harness.replay_setup(eng, wl, chunk_tokens=1 << 16)
    outs, metas = harness.run_steps(eng, wl, steps, partition_tokens)
    torch.cuda.synchronize()
    return eng, outs, metas


def _check(wl, steps, compare_caches=True, partition_tokens=0, disjoint=None):
    log(f"{wl.name}: gpu run ({steps} step(s))")
    eng, outs, metas = _gpu_run(wl, steps, partition_tokens)
    if disjoint is not None:
        # batches whose sequences hold no block in common attend through the
        # zero-group call (waves in head groups where the shape allows); those
        # with shared blocks through plain decode
        assert (eng.disjoint is not None) == disjoint
    log(f"{wl.name}: oracle run")
    o = runner.run(wl, steps=steps, threads=ORACLE_THREADS)
    for s in range(steps):
        tab, ctx = metas[s]
        assert ctx.tolist() == o.ctx_lens[s]
        for i, t in enumerate(o.tables[s]):
            assert tab[i, :len(t)].tolist() == t
            assert (tab[i, len(t):] == -1).all()
        err = assert_close_to_oracle(outs[s], o.outputs[s], wl.kv_dtype, f"{wl.name} step {s}")
        log(f"{wl.name} step {s}: max abs err {err:.2e}")
    # the device-resident tables and lengths, kept current by the write kernel's
    # updates, equal the manager's (and so the oracle's) after the last step
    assert np.array_equal(eng.tables_dev.cpu().numpy(), metas[-1][0])
    assert np.array_equal(eng.ctx_dev.cpu().numpy(), metas[-1][1])
    if compare_caches:
        assert_caches_bit_exact(eng.k_cache, o.k_cache, f"{wl.name} K cache")
        assert_caches_bit_exact(eng.v_cache, o.v_cache, f"{wl.name} V cache")
    return eng, outs


def test_config1_tiny_two_steps():
    _check(workloads.tiny(), steps=2, disjoint=True)


@pytest.mark.parametrize("part", [16, 48, 128, 512, 4096])
def test_config1_partition_sizes(part):
    _check(workloads.tiny(), steps=2, partition_tokens=part, compare_caches=False)


def test_config2_llama2_full_size():
    _check(workloads.llama2_7b(max_steps=2), steps=2, disjoint=True)


def test_config3_qwen3_prefix_full_size():
    _check(workloads.qwen3_prefix(max_steps=1), steps=1, disjoint=False)


@pytest.mark.timeout(600)
def test_config4_opt13b_full_size():
    """Two steps over 128 sequences of ~3000 tokens; both 4.4 GB caches are
    compared bit for bit (pools past 4 GiB per array)."""
    _check(workloads.opt13b_rag(max_steps=2), steps=2, disjoint=True)


def test_config5_beam_fp8_full_size():
    _check(workloads.beam_fp8(max_steps=2), steps=2, disjoint=False)


@pytest.mark.parametrize("kv_dtype,per_head", [("fp8_e5m2", False), ("fp8", True), ("fp8_e5m2", True)])
def test_config5_beam_fp8_variants_full_size(kv_dtype, per_head):
    """The beam workload with e5m2 storage and/or one scale per KV head."""
    _check(workloads.beam_fp8(max_steps=2, kv_dtype=kv_dtype, per_head=per_head), steps=2)


def test_per_head_scales_all_equal_match_per_tensor_bits():
    """Per-head scales that are all equal give the per-tensor results bit for bit
    (the same fp32 products in the same order)."""
    wl = workloads.beam_fp8(prompts=6, max_steps=1)
    eng, outs, _ = _gpu_run(wl, 1)
    hkv = wl.num_kv_heads
    wl2 = workloads.beam_fp8(prompts=6, max_steps=1)
    for name in ("k_scale", "v_scale", "k_inv_scale", "v_inv_scale"):
        setattr(wl2, name, np.full(hkv, getattr(wl, name), dtype=np.float32))
    eng2, outs2, _ = _gpu_run(wl2, 1)
    assert np.array_equal(cache_bits(eng.k_cache), cache_bits(eng2.k_cache))
    assert np.array_equal(outs[0].view(np.uint16), outs2[0].view(np.uint16))


def test_copy_on_write_inside_decode_steps():
    """Every beam's first tail token is written by a decode step: the step's
    copy-on-write pairs go through paged_step_metadata and paged_block_copy."""
    wl = workloads.beam_fp8(max_steps=3, prompts=6, tail_max=1)
    _check(wl, steps=3)


@pytest.mark.parametrize("hq,hkv,d,bs,kv", [(8, 8, 64, 16, "f16"), (16, 8, 128, 16, "f16"),
                                           (32, 8, 128, 32, "f16"), (64, 8, 128, 64, "fp8"),
                                           (8, 2, 64, 64, "fp8"), (16, 16, 128, 64, "fp8"),
                                           (32, 8, 128, 16, "fp8_e5m2"), (16, 16, 64, 32, "fp8_e5m2")])
def test_small_shapes_all_outputs(hq, hkv, d, bs, kv):
    # ragged lengths: 1, block boundaries +-1, many splits, one long
    L = [1, 2, bs - 1, bs, bs + 1, 63, 64, 65, 511, 512, 513, 1500]
    wl = workloads.small_custom(seed=hq + hkv + d + bs, lengths=L, num_q_heads=hq, num_kv_heads=hkv,
                                head_dim=d, block_size=bs, kv_dtype=kv, max_steps=1)
    for part in (16, 80, 0):
        _check(wl, steps=1, partition_tokens=part, compare_caches=(part == 16))


@pytest.mark.parametrize("g", [4, 8])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kv", ["f16", "fp8", "fp8_e5m2"])
def test_matrix_core_path_every_variant(g, d, kv):
    """Every instantiation of the matrix-core decode kernel (4 or 8 query heads
    per KV head, head_dim 64 or 128, each KV format): ragged lengths around the
    32-token unit and the block, at the default worker count."""
    L = [1, 31, 32, 33, 95, 96, 97, 300]
    wl = workloads.small_custom(seed=200 + g + d, lengths=L, num_q_heads=2 * g, num_kv_heads=2, head_dim=d,
                                block_size=32, kv_dtype=kv, max_steps=1)
    _check(wl, steps=1, compare_caches=False)


def test_placement_invariance_bit_exact():
    """Same logical sequences, different physical placement: identical output bits."""
    wl1 = workloads.small_custom(seed=5, lengths=[100, 700, 33], num_q_heads=16, num_kv_heads=8,
                                 head_dim=128, block_size=16)
    wl2 = workloads.small_custom(seed=5, lengths=[100, 700, 33], num_q_heads=16, num_kv_heads=8,
                                 head_dim=128, block_size=16)
    wl2.free_order = np.ascontiguousarray(wl2.free_order[::-1])
    _, o1, _ = _gpu_run(wl1, 1)
    _, o2, _ = _gpu_run(wl2, 1)
    assert np.array_equal(o1[0].view(np.uint16), o2[0].view(np.uint16))


def test_shared_prefix_equals_private_copy_bit_exact():
    """A sequence reading a shared prefix gives the same bits as one holding a private copy."""
    shared = workloads.qwen3_prefix(batch=3, max_steps=1)
    _, o_sh, _ = _gpu_run(shared, 1)
    # private: every sequence allocates its own prefix with the same data
    priv = workloads.qwen3_prefix(batch=3, max_steps=1)
    r0 = priv.setup_rounds[0][0]
    priv.setup_rounds = [[r0] + [workloads.Op("allocate", s, 1024, key=0) for s in (1, 2)]] + \
        priv.setup_rounds[2:]
    priv.num_blocks = shared.num_blocks + 2 * 64
    priv.free_order = np.arange(priv.num_blocks, dtype=np.int32)
    _, o_pr, _ = _gpu_run(priv, 1)
    assert np.array_equal(o_sh[0].view(np.uint16), o_pr[0].view(np.uint16))


def test_zero_length_and_single_token():
    torch.manual_seed(0)
    B, hq, hkv, d, bs, nb = 3, 8, 4, 64, 16, 8
    kc = torch.randn(nb, hkv, bs, d, device=DEV).half()
    vc = torch.randn(nb, hkv, bs, d, device=DEV).half()
    q = torch.randn(B, hq, d, device=DEV).half()
    tables = torch.tensor([[3, -1], [5, -1], [0, 1]], dtype=torch.int32, device=DEV)
    ctx = torch.tensor([0, 1, 20], dtype=torch.int32, device=DEV)
    out = torch.full((B, hq, d), 7.0, dtype=torch.float16, device=DEV)
    ws = torch.empty(max(ops.workspace_bytes(B, hq, hkv, d, 2, bs, 64), 4), dtype=torch.uint8, device=DEV)
    ops.paged_attn_decode(out, q, kc, vc, tables, ctx, 0.125, partition_tokens=64, workspace=ws)
    torch.cuda.synchronize()
    assert (out[0] == 0).all()
    # one token: the output is V[0] of its KV head, exactly
    v0 = vc[5, :, 0, :].repeat_interleave(hq // hkv, dim=0)
    assert torch.equal(out[1], v0)
    ref = oattn.decode_attention(q.cpu().numpy(), kc.cpu().numpy(), vc.cpu().numpy(),
                                 tables.cpu().numpy().tolist(), ctx.cpu().tolist(), bs, 0.125)
    assert_close_to_oracle(out[2].cpu().numpy(), ref[2], "f16", "ragged")


def test_out_of_range_block_ids_are_skipped():
    """A table entry outside the pool is not followed: its tokens are left out."""
    B, hq, hkv, d, bs, nb = 2, 4, 4, 128, 16, 6
    torch.manual_seed(1)
    kc = torch.randn(nb, hkv, bs, d, device=DEV).half()
    vc = torch.randn(nb, hkv, bs, d, device=DEV).half()
    q = torch.randn(B, hq, d, device=DEV).half()
    tables = torch.tensor([[2, 999, 4], [1, -5, 3]], dtype=torch.int32, device=DEV)
    ctx = torch.tensor([48, 40], dtype=torch.int32, device=DEV)
    out = torch.empty(B, hq, d, dtype=torch.float16, device=DEV)
    ops.paged_attn_decode(out, q, kc, vc, tables, ctx, 0.1, partition_tokens=64)
    torch.cuda.synchronize()
    # reference: the same sequences without the skipped block
    kn, vn, qn = kc.cpu().numpy(), vc.cpu().numpy(), q.cpu().numpy()
    ref0 = oattn.decode_attention(qn[:1], kn, vn, [[2, 4]], [32], bs, 0.1)
    ref1 = oattn.decode_attention(qn[1:], kn, vn, [[1, 3]], [24], bs, 0.1)
    assert_close_to_oracle(out[0:1].cpu().numpy(), ref0, "f16", "skip0")
    assert_close_to_oracle(out[1:2].cpu().numpy(), ref1, "f16", "skip1")


def test_context_longer_than_table_is_clamped():
    B, hq, hkv, d, bs, nb = 1, 2, 2, 64, 16, 4
    torch.manual_seed(2)
    kc = torch.randn(nb, hkv, bs, d, device=DEV).half()
    vc = torch.randn(nb, hkv, bs, d, device=DEV).half()
    q = torch.randn(B, hq, d, device=DEV).half()
    tables = torch.tensor([[1, 2]], dtype=torch.int32, device=DEV)
    out = torch.empty(B, hq, d, dtype=torch.float16, device=DEV)
    ops.paged_attn_decode(out, q, kc, vc, tables, torch.tensor([1000], dtype=torch.int32, device=DEV),
                          0.125, partition_tokens=64)
    torch.cuda.synchronize()
    ref = oattn.decode_attention(q.cpu().numpy(), kc.cpu().numpy(), vc.cpu().numpy(), [[1, 2]], [32], bs, 0.125)
    assert_close_to_oracle(out.cpu().numpy(), ref, "f16", "clamp")


def test_repeat_calls_bit_identical():
    """The split depends only on the lengths and the worker count: two runs agree bit for bit."""
    wl = workloads.small_custom(seed=9, lengths=[5, 300, 1000, 17, 2049], num_q_heads=32, num_kv_heads=8,
                                head_dim=128, block_size=32)
    _, o1, _ = _gpu_run(wl, 1)
    _, o2, _ = _gpu_run(wl, 1)
    assert np.array_equal(o1[0].view(np.uint16), o2[0].view(np.uint16))


@pytest.mark.parametrize("shared", [False, True])
def test_pass1_timing_hook(shared):
    """The measurement hook (pkv_time_next_pass1): the armed pass-1 launch
    records both events, so they give a positive duration; the hook is used
    once and disarms; the output is bit-identical to an unarmed call on the
    same state. shared=True runs the grouped pass (a forked batch)."""
    if shared:
        wl = workloads.small_forks(seed=23, prompts=[200, 90], members=[4, 3], tails=[[1, 2, 3, 4], [0, 9, 30]],
                                   singles=[70, 5], num_q_heads=16, num_kv_heads=2, head_dim=128, block_size=16)
    else:
        wl = workloads.small_custom(seed=22, lengths=[5, 300, 1000, 17, 2049], num_q_heads=32, num_kv_heads=8,
                                    head_dim=128, block_size=32)
    eng = harness.make_engine(wl)
    harness.replay_setup(eng, wl, chunk_tokens=1 << 16)
    harness.run_steps(eng, wl, 1, shared_prefix=shared)
    _, _, q = harness.step_inputs(wl, 0, DEV)
    B = len(wl.batch)
    plain = torch.empty((B, wl.num_q_heads, wl.head_dim), dtype=torch.float16, device=DEV)
    timed = torch.empty_like(plain)
    again = torch.empty_like(plain)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    eng.attend(q, plain)
    ops.time_next_pass1(*ev)
    eng.attend(q, timed)
    eng.attend(q, again)  # disarmed again: must not touch the events
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1])
    log(f"timing hook ({'grouped' if shared else 'plain'} pass 1): {ms * 1e3:.1f} us")
    assert 0.0 < ms < 1000.0
    assert np.array_equal(plain.cpu().numpy().view(np.uint16), timed.cpu().numpy().view(np.uint16))
    assert np.array_equal(plain.cpu().numpy().view(np.uint16), again.cpu().numpy().view(np.uint16))
    with pytest.raises(ValueError):
        ops.time_next_pass1(ev[0], None)


@pytest.mark.parametrize("hq,hkv", [(2, 2), (8, 2)])
def test_batch_of_more_than_4096_sequences(hq, hkv):
    """4100 short sequences run as two launches (4096 + 4); every output is checked."""
    B, d, bs, maxb = 4100, 64, 16, 3
    g = np.random.default_rng(hq)
    nb = B * maxb
    kc = torch.from_numpy(g.standard_normal((nb, hkv, bs, d), dtype=np.float32).astype(np.float16)).to(DEV)
    vc = torch.from_numpy(g.standard_normal((nb, hkv, bs, d), dtype=np.float32).astype(np.float16)).to(DEV)
    q = torch.from_numpy(g.standard_normal((B, hq, d), dtype=np.float32).astype(np.float16)).to(DEV)
    tables = g.permutation(nb).astype(np.int32).reshape(B, maxb)
    ctx = g.integers(0, maxb * bs + 1, size=B).astype(np.int32)
    ctx[4096:] = [0, 1, 47, 48]
    out = torch.full((B, hq, d), 3.0, dtype=torch.float16, device=DEV)
    log(f"batch 4100 hq={hq} hkv={hkv}")
    ops.paged_attn_decode(out, q, kc, vc, torch.from_numpy(tables).to(DEV), torch.from_numpy(ctx).to(DEV),
                          0.125, partition_tokens=16)
    torch.cuda.synchronize()
    ref = oattn.decode_attention(q.cpu().numpy(), kc.cpu().numpy(), vc.cpu().numpy(), tables, ctx.tolist(),
                                 bs, 0.125)
    assert_close_to_oracle(out.cpu().numpy(), ref, "f16", "batch 4100")


def test_config3_prefix_cache_matches_scripted_sharing():
    """The shared-prefix workload with its sharing found by the block manager's prefix
    cache (every sequence allocated from its token ids) gives the same output bits as
    with the sharing written into the script; sampled outputs match the oracle."""
    scripted = workloads.qwen3_prefix(max_steps=1)
    cached = workloads.qwen3_prefix_cached(max_steps=1)
    log("config 3: scripted sharing")
    _, o1, _ = _gpu_run(scripted, 1)
    log("config 3: prefix-cache sharing")
    eng, o2, _ = _gpu_run(cached, 1)
    assert np.array_equal(o1[0].view(np.uint16), o2[0].view(np.uint16))
    assert eng.bm.stats()["prefix_hit_tokens"] == (len(cached.batch) - 1) * cached.meta["prefix_tokens"]
    o = runner.run(cached, steps=1, threads=ORACLE_THREADS)
    assert_close_to_oracle(o2[0], o.outputs[0], "f16", "config 3 cached")
    assert_caches_bit_exact(eng.k_cache, o.k_cache, "config 3 cached K cache")
    assert_caches_bit_exact(eng.v_cache, o.v_cache, "config 3 cached V cache")


_RSHAPES = [(hq, hkv, d, bs, kv) for (hq, hkv) in ((4, 4), (8, 4), (16, 4), (32, 4))
            for d in (64, 128) for bs in (16, 32, 64) for kv in ("f16", "fp8", "fp8_e5m2")]


@pytest.mark.parametrize("seed", range(RANDOM_DRAWS))
def test_random_decode_scripts(seed):
    """Seeded random batches of independent sequences (1-24 of them; lengths
    from 1 to 2500, a third of them next to a block or unit edge) decoded for
    three steps through the engine (write step with its metadata, pass 1 on
    the vector or matrix-core path, pass 2) at a random worker count: tables
    and lengths equal the oracle's, every output within tolerance, caches
    bit-exact."""
    g = np.random.default_rng(7000 + seed)
    hq, hkv, d, bs, kv = _RSHAPES[int(g.integers(0, len(_RSHAPES)))]
    n = int(g.integers(1, 25))
    lengths = []
    for _ in range(n):
        if g.random() < 0.33:
            edge = int(g.choice([bs, 16, 32, 64])) * int(g.integers(1, 12))
            lengths.append(max(1, edge + int(g.integers(-2, 3))))
        else:
            lengths.append(int(g.integers(1, 2501)))
    per_head = kv != "f16" and g.random() < 0.5
    part = int(g.choice([16, 80, 0]))
    log(f"random decode {seed}: {hq}/{hkv} d{d} bs{bs} {kv}{'+ph' if per_head else ''} lengths {lengths} "
        f"partition {part}")
    wl = workloads.small_custom(seed=8000 + seed, lengths=lengths, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                                block_size=bs, kv_dtype=kv, max_steps=3, per_head=per_head)
    _check(wl, steps=3, partition_tokens=part)
