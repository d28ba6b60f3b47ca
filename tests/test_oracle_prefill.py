"""Pins for the oracle's chunked (multi-token, causal) prefill attention.

* Library pin: PyTorch's scaled_dot_product_attention in float64 with
  is_causal=True on the whole prompt. For a whole-prompt chunk (n = L) its
  rows are the oracle's rows; for a chunk of the last n positions they are the
  last n rows of the whole prompt's causal attention (this fixes where the
  chunk sits: a chunk aligned to the start of the context fails it).
  Grouped-query heads through enable_gqa (query head h -> KV head h // group).
* Reductions: a one-row chunk is decode attention; the row at position 0
  returns V[0] exactly; splitting a prefill into consecutive chunks gives the
  same rows as one chunk.
* Causality: changing K/V after a row's position leaves the row unchanged;
  changing its own position's K/V changes it.
* Degenerate cases: an empty chunk, a chunk longer than its context (rows
  with nothing to attend are 0).
* Whole pipeline (prefix-cache allocation + scatter + gather + prefill)
  against SDPA on K/V assembled from the workload script's own meaning.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import attention, cache_ops, fp8, prefill, runner


def causal_sdpa64(Q, K, V, scale):
    """Q [L, Hq, D], K/V [L, Hkv, D] -> [L, Hq, D], torch SDPA is_causal in float64."""
    qt = torch.from_numpy(np.ascontiguousarray(np.transpose(Q, (1, 0, 2)), dtype=np.float64))[None]
    kt = torch.from_numpy(np.ascontiguousarray(np.transpose(K, (1, 0, 2)), dtype=np.float64))[None]
    vt = torch.from_numpy(np.ascontiguousarray(np.transpose(V, (1, 0, 2)), dtype=np.float64))[None]
    gqa = qt.shape[1] != kt.shape[1]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale,
                                                         enable_gqa=gqa)
    return np.transpose(o[0].numpy(), (1, 0, 2))


def _paged(seed, lengths, hkv, d, bs, kv_dtype="f16", inv_scale=1.0):
    """Sequences of random K/V scattered through a permuted pool."""
    g = np.random.default_rng(seed)
    nb = sum(-(-L // bs) for L in lengths) + 5
    perm = g.permutation(nb)
    kc = runner.empty_cache(nb, hkv, bs, d, kv_dtype)
    vc = runner.empty_cache(nb, hkv, bs, d, kv_dtype)
    tables, logical, pos = [], [], 0
    for L in lengths:
        nblk = -(-L // bs)
        t = perm[pos:pos + nblk].tolist()
        pos += nblk
        K = g.standard_normal((L, hkv, d)).astype(np.float16)
        V = g.standard_normal((L, hkv, d)).astype(np.float16)
        slots = [t[p // bs] * bs + p % bs for p in range(L)]
        cache_ops.scatter(kc, vc, K, V, slots, bs, kv_dtype, inv_scale, inv_scale)
        tables.append(t)
        logical.append((K, V))
    return kc, vc, tables, logical


def _queries(seed, rows, hq, d):
    return np.random.default_rng(seed).standard_normal((rows, hq, d)).astype(np.float16)


@pytest.mark.parametrize("hq,hkv,bs", [(4, 4, 4), (8, 2, 16), (6, 1, 8)])
def test_whole_prompt_matches_causal_sdpa(hq, hkv, bs):
    lengths = [1, 7, 16, 17, 45]
    d = 32
    kc, vc, tables, logical = _paged(21, lengths, hkv, d, bs)
    q = _queries(22, sum(lengths), hq, d)
    q_start = np.concatenate([[0], np.cumsum(lengths)])
    scale = 1.0 / np.sqrt(d)
    out = prefill.prefill_attention(q, q_start, kc, vc, tables, lengths, bs, scale)
    for s, (K, V) in enumerate(logical):
        r0, r1 = q_start[s], q_start[s + 1]
        ref = causal_sdpa64(q[r0:r1].astype(np.float64), K.astype(np.float64), V.astype(np.float64), scale)
        np.testing.assert_allclose(out[r0:r1], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4)])
def test_chunk_is_last_rows_of_whole_prompt(hq, hkv):
    """A chunk of the last n positions = the last n rows of causal attention over the prompt."""
    lengths, chunks = [40, 33, 64, 9], [5, 33, 17, 1]
    d, bs = 16, 8
    kc, vc, tables, logical = _paged(31, lengths, hkv, d, bs)
    scale = 0.2
    full_q = [_queries(40 + s, L, hq, d) for s, L in enumerate(lengths)]
    q = np.concatenate([fq[L - n:] for fq, L, n in zip(full_q, lengths, chunks)])
    q_start = np.concatenate([[0], np.cumsum(chunks)])
    out = prefill.prefill_attention(q, q_start, kc, vc, tables, lengths, bs, scale)
    for s, (K, V) in enumerate(logical):
        L, n = lengths[s], chunks[s]
        ref = causal_sdpa64(full_q[s].astype(np.float64), K.astype(np.float64), V.astype(np.float64), scale)
        np.testing.assert_allclose(out[q_start[s]:q_start[s + 1]], ref[L - n:], rtol=1e-12, atol=1e-12)


def test_one_row_chunk_is_decode_attention():
    lengths = [1, 30, 64, 65]
    hq, hkv, d, bs = 8, 2, 16, 16
    kc, vc, tables, _ = _paged(5, lengths, hkv, d, bs)
    q = _queries(6, len(lengths), hq, d)
    q_start = np.arange(len(lengths) + 1)
    a = prefill.prefill_attention(q, q_start, kc, vc, tables, lengths, bs, 0.25)
    b = attention.decode_attention(q, kc, vc, tables, lengths, bs, 0.25)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)


def test_position_zero_returns_v0_exactly():
    lengths = [12, 3]
    kc, vc, tables, logical = _paged(8, lengths, 2, 8, 4)
    q = _queries(9, sum(lengths), 4, 8)
    q_start = np.array([0, 12, 15])
    out = prefill.prefill_attention(q, q_start, kc, vc, tables, lengths, 4, 0.5)
    for s, r in ((0, 0), (1, 12)):
        V0 = logical[s][1][0].astype(np.float64)  # [Hkv, D]
        for h in range(4):
            assert np.array_equal(out[r, h], V0[h // 2])


def test_two_chunks_equal_one():
    """Prefilling positions [0, c) then [c, L) gives the rows of one whole-prompt chunk."""
    L, c = 50, 19
    kc, vc, tables, _ = _paged(12, [L], 4, 16, 8)
    q = _queries(13, L, 4, 16)
    whole = prefill.prefill_attention(q, [0, L], kc, vc, tables, [L], 8, 0.3)
    first = prefill.prefill_attention(q[:c], [0, c], kc, vc, tables, [c], 8, 0.3)
    second = prefill.prefill_attention(q[c:], [0, L - c], kc, vc, tables, [L], 8, 0.3)
    np.testing.assert_allclose(np.concatenate([first, second]), whole, rtol=1e-13, atol=1e-13)


def test_causality():
    L, n, bs = 30, 10, 8
    kc, vc, tables, _ = _paged(14, [L], 2, 16, bs)
    q = _queries(15, n, 2, 16)
    base = prefill.prefill_attention(q, [0, n], kc, vc, tables, [L], bs, 0.3)
    t = tables[0]
    for row in (0, 4, 9):
        p = L - n + row
        for pos, must_change in ((p + 1, False), (L - 1, False), (p, True)):
            if pos >= L or (pos > p) == must_change:
                continue
            kc2, vc2 = kc.copy(), vc.copy()
            kc2[t[pos // bs], :, pos % bs, :] += np.float16(1.5)
            vc2[t[pos // bs], :, pos % bs, :] -= np.float16(2.0)
            out = prefill.prefill_attention(q, [0, n], kc2, vc2, tables, [L], bs, 0.3)
            changed = not np.array_equal(out[row], base[row])
            assert changed == must_change, (row, pos)
            # rows before the changed position never change
            earlier = [r for r in range(n) if L - n + r < pos]
            assert np.array_equal(out[earlier], base[earlier])


def test_empty_and_overlong_chunks():
    kc, vc, tables, logical = _paged(16, [5, 3], 2, 8, 4)
    q = _queries(17, 6, 2, 8)
    # seq 0: empty chunk; seq 1: 6 rows over a 3-token context -> rows 0..2 have p < 0
    out = prefill.prefill_attention(q, [0, 0, 6], kc, vc, tables, [5, 3], 4, 0.4)
    assert out.shape == (6, 2, 8)
    assert np.array_equal(out[:3], np.zeros((3, 2, 8)))
    ref = causal_sdpa64(q[3:].astype(np.float64), logical[1][0].astype(np.float64),
                        logical[1][1].astype(np.float64), 0.4)
    np.testing.assert_allclose(out[3:], ref, rtol=1e-12, atol=1e-12)


def test_fp8_cache_matches_sdpa_on_dequantized_values():
    lengths, chunks = [33, 20], [33, 7]
    hkv, d, bs = 2, 16, 16
    scale = np.float32(3.0) / np.float32(448.0)
    inv = float(np.float32(1.0) / scale)
    kc, vc, tables, logical = _paged(18, lengths, hkv, d, bs, "fp8", inv)
    q = _queries(19, sum(chunks), 4, d)
    q_start = np.concatenate([[0], np.cumsum(chunks)])
    out = prefill.prefill_attention(q, q_start, kc, vc, tables, lengths, bs, 0.25, "fp8",
                                    float(scale), float(scale))
    for s, (K, V) in enumerate(logical):
        # dequantise through torch's own e4m3fn conversion (a library routine)
        kq = torch.from_numpy(fp8.quantize(K, inv)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        vq = torch.from_numpy(fp8.quantize(V, inv)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        n = chunks[s]
        full_q = np.zeros((lengths[s], 4, d))
        full_q[lengths[s] - n:] = q[q_start[s]:q_start[s + 1]]
        ref = causal_sdpa64(full_q, kq * float(scale), vq * float(scale), 0.25)
        np.testing.assert_allclose(out[q_start[s]:q_start[s + 1]], ref[lengths[s] - n:], rtol=1e-12, atol=1e-12)


def _logical_prompt_kv(wl, op):
    """K/V of a prompt from its script: the draws of its parts, in order."""
    return wl.prompt_kv(op, 0)


def test_pipeline_prefill_tiny_prefix_cache():
    """The tiny prefix-cache prefill: hits, chunk rows and outputs vs SDPA on the script's K/V."""
    wl = workloads.prefill_tiny()
    r = runner.run_prefill(wl)
    assert r.cached == {0: 0, 1: 32, 2: 0, 3: 32}
    assert r.chunks == [37, 68, 16, 218]
    ops = {o.seq: o for o in wl.setup_rounds[0]}
    for i, s in enumerate(wl.batch):
        K, V = _logical_prompt_kv(wl, ops[s])
        L, n = len(K), r.chunks[i]
        full_q = np.zeros((L, wl.num_q_heads, wl.head_dim))
        full_q[L - n:] = wl.prefill_queries(s, n)
        ref = causal_sdpa64(full_q, K.astype(np.float64), V.astype(np.float64), wl.sm_scale)
        np.testing.assert_allclose(r.output[r.q_start[i]:r.q_start[i + 1]], ref[L - n:], rtol=1e-12, atol=1e-12)


def test_pipeline_qwen3_prefill_small():
    """Five prompts of the Qwen3-shaped prefix-cache prefill: 4 of 5 hit the 64-block system prompt."""
    wl = workloads.qwen3_prefill(batch=5)
    r = runner.run_prefill(wl, seqs=[0, 3])
    assert [r.cached[s] for s in range(5)] == [0, 1024, 1024, 1024, 1024]
    L = wl.meta["lengths"]
    assert r.chunks == [L[0]] + [l - 1024 for l in L[1:]]
    ops = {o.seq: o for o in wl.setup_rounds[0]}
    for i in (0, 3):
        K, V = _logical_prompt_kv(wl, ops[i])
        n = r.chunks[i]
        full_q = np.zeros((len(K), wl.num_q_heads, wl.head_dim))
        full_q[len(K) - n:] = wl.prefill_queries(i, n)
        ref = causal_sdpa64(full_q, K.astype(np.float64), V.astype(np.float64), wl.sm_scale)
        np.testing.assert_allclose(r.output[r.q_start[i]:r.q_start[i + 1]], ref[len(K) - n:],
                                   rtol=1e-11, atol=1e-11)


def test_chunk_over_an_empty_context_is_zero():
    """A sequence with no tokens but a chunk of rows: every row sits at a
    position < 0, has nothing to attend and is 0; its neighbours are
    unaffected."""
    kc, vc, tables, logical = _paged(21, [0, 4], 2, 8, 4)
    q = _queries(22, 5, 2, 8)
    out = prefill.prefill_attention(q, [0, 3, 5], kc, vc, tables, [0, 4], 4, 0.5)
    assert np.array_equal(out[:3], np.zeros((3, 2, 8)))
    full_q = np.zeros((4, 2, 8))
    full_q[2:] = q[3:]
    ref = causal_sdpa64(full_q, logical[1][0].astype(np.float64), logical[1][1].astype(np.float64), 0.5)
    np.testing.assert_allclose(out[3:], ref[2:], rtol=1e-12, atol=1e-12)
