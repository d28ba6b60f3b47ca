"""Pins for the oracle's preemption (recompute and swap) and host pool.

* Hand-worked cases of preemption from the tail of the running set ("Where
  Did the VRAM Go (KV cache tutorial)", §7.1: the newest requests are
  preempted first, until enough blocks are free; their blocks are released,
  the others keep running), worked out by hand from the FIFO pool below.
* Data round trip: swap a group out (copy to host), let the freed device
  blocks be reused and overwritten, swap it back in: every sequence gathers
  exactly the K/V it had.
* A group's shared blocks are copied once; blocks shared with a sequence
  outside the group stay resident.
* Failing calls change nothing; a swapped-out sequence is not resident.
* Random operation sequences keep both pools conserved and every refcount
  equal to its references.
"""
import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import attention, cache_ops, runner
from oracle.allocator import ERR_EXISTS, ERR_INVALID, ERR_NO_SEQ, ERR_OOM, AllocError, BlockAllocatorModel
from tests.test_oracle_allocator import check_invariants


def _raises(code, fn, *a):
    try:
        fn(*a)
    except AllocError as e:
        assert e.code == code, (e.code, code)
    else:
        raise AssertionError("call should have failed")


def _running(nb=8, bs=4):
    """A (5 tokens: blocks 0,1), B (9: 2,3,4), C (8: 5,6) on an 8-block pool; block 7 free."""
    m = BlockAllocatorModel(nb, bs)
    m.allocate(0, 5)
    m.allocate(1, 9)
    m.allocate(2, 8)
    assert m.tables == {0: [0, 1], 1: [2, 3, 4], 2: [5, 6]} and m.free_list() == [7]
    return m


def test_preempt_tail_recompute_newest_first():
    m = _running()
    # enough already: nobody is preempted
    assert m.preempt_tail([0, 1, 2], 1) == ([], [])
    # 3 blocks: C (newest) gives 2 -> 3 available
    assert m.preempt_tail([0, 1, 2], 3) == ([2], [])
    assert m.free_list() == [7, 5, 6] and 2 not in m.tables
    # the preempted request comes back by prefill: a fresh allocation
    m.allocate(2, 8)
    assert m.block_table(2) == [7, 5]


def test_preempt_tail_walks_back_until_enough():
    m = _running()
    # 5 blocks: C gives 2 (3 available), B gives 3 (6 available)
    victims, pairs = m.preempt_tail([0, 1, 2], 5)
    assert victims == [2, 1] and pairs == []
    assert m.free_list() == [7, 5, 6, 2, 3, 4] and list(m.tables) == [0]


def test_preempt_tail_counts_only_released_blocks():
    m = BlockAllocatorModel(6, 4)
    m.allocate(0, 8)          # blocks 0, 1
    m.fork(0, 1)              # shares 0, 1
    m.allocate(2, 4)          # block 2
    # need 4: seq 2 releases block 2 (4 available: 3,4,5,2); seq 1 alone would release nothing
    assert m.preempt_tail([0, 1, 2], 4) == ([2], [])
    # need 6: seq 1 releases nothing (its blocks are still held by 0), seq 0 releases both
    assert m.preempt_tail([0, 1], 6) == ([1, 0], [])
    assert m.free_list() == [3, 4, 5, 2, 0, 1]


def test_preempt_tail_swap_mode():
    m = _running()
    m.set_host_blocks(4)
    victims, pairs = m.preempt_tail([0, 1, 2], 3, "swap")
    assert victims == [2] and pairs == [(5, 0), (6, 1)]
    assert m.host_tables == {2: [0, 1]} and m.host_counts == {2: 8}
    assert m.free_list() == [7, 5, 6] and m.host_free_list() == [2, 3]
    _raises(ERR_NO_SEQ, m.append, 2, 1)       # not resident
    _raises(ERR_EXISTS, m.allocate, 2, 1)     # id still taken
    # back in: host blocks 0, 1 -> device blocks 7, 5 (front of the free queue)
    assert m.swap_in([2]) == [(0, 7), (1, 5)]
    assert m.block_table(2) == [7, 5] and m.num_tokens(2) == 8
    assert m.host_free_list() == [2, 3, 0, 1]


def test_preempt_failures_change_nothing():
    m = _running()
    m.set_host_blocks(1)
    before = m.state()
    _raises(ERR_OOM, m.preempt_tail, [0, 1, 2], 9)           # even everyone is not enough
    _raises(ERR_OOM, m.preempt_tail, [0, 1, 2], 3, "swap")   # C needs 2 host blocks, 1 exists
    _raises(ERR_INVALID, m.preempt_tail, [0, 0], 3)
    _raises(ERR_NO_SEQ, m.preempt_tail, [0, 9], 3)
    _raises(ERR_INVALID, m.preempt_tail, [0], 3, "drop")
    assert m.state() == before


def test_group_swap_copies_shared_blocks_once():
    m = BlockAllocatorModel(16, 4)
    m.set_host_blocks(8)
    m.allocate(0, 10)                  # prompt: blocks 0, 1, 2 (last one partial)
    for b in (1, 2, 3):
        m.fork(0, b)                   # beams share all three
    m.append(1, 1)                     # copy-on-write of block 2 -> 3
    pairs = m.swap_out([0, 1, 2, 3])
    assert pairs == [(0, 0), (1, 1), (2, 2), (3, 3)]
    assert m.host_ref[:4] == [4, 4, 3, 1]
    assert m.host_tables == {0: [0, 1, 2], 1: [0, 1, 3], 2: [0, 1, 2], 3: [0, 1, 2]}
    assert sorted(m.free_list()) == list(range(16)) and m.tables == {}
    back = m.swap_in([3, 1])           # part of the group: its distinct host blocks only
    assert back == [(0, 4), (1, 5), (2, 6), (3, 7)]
    assert m.block_table(3) == [4, 5, 6] and m.block_table(1) == [4, 5, 7]
    assert m.host_ref[:4] == [2, 2, 2, 0] and m.host_free_list()[-1] == 3


def test_block_shared_outside_the_group_stays_resident():
    m = BlockAllocatorModel(8, 4)
    m.set_host_blocks(4)
    m.allocate(0, 8)
    m.share_prefix(0, 2, 1)
    m.append(1, 3)                     # its own block 2
    pairs = m.swap_out([1])
    assert pairs == [(0, 0), (1, 1), (2, 2)]
    assert m.ref[:3] == [1, 1, 0] and m.block_table(0) == [0, 1]
    assert m.free_list()[-1] == 2


def test_swap_failures_change_nothing_and_free_of_swapped():
    m = BlockAllocatorModel(4, 4)
    m.set_host_blocks(2)
    m.allocate(0, 12)                  # 3 blocks
    before = m.state()
    _raises(ERR_OOM, m.swap_out, [0])  # 3 host blocks needed
    _raises(ERR_INVALID, m.swap_out, [0, 0])
    _raises(ERR_NO_SEQ, m.swap_in, [0])
    assert m.state() == before
    m.free_seq(0)
    m.allocate(1, 4)
    m.swap_out([1])
    m.allocate(2, 16)                  # the whole device pool
    before = m.state()
    _raises(ERR_OOM, m.swap_in, [1])
    _raises(ERR_INVALID, m.set_host_blocks, 4)   # something is swapped out
    assert m.state() == before
    m.free_seq(1)                      # releases its host block
    assert m.host_free_list() == [1, 0] and m.host_tables == {}


def test_swap_round_trip_restores_every_sequence():
    """Swap out, let the released blocks be reused and overwritten, swap back in:
    the gathered K/V of every sequence is bit-identical (fp16 and fp8 caches)."""
    rng = np.random.default_rng(7)
    for kv_dtype in ("f16", "fp8"):
        nb, hkv, bs, d = 24, 2, 4, 8
        m = BlockAllocatorModel(nb, bs)
        m.set_host_blocks(16)
        kc = runner.empty_cache(nb, hkv, bs, d, kv_dtype)
        vc = runner.empty_cache(nb, hkv, bs, d, kv_dtype)
        kh = runner.empty_cache(16, hkv, bs, d, kv_dtype)
        vh = runner.empty_cache(16, hkv, bs, d, kv_dtype)

        def write(slots):
            K = rng.standard_normal((len(slots), hkv, d)).astype(np.float16)
            V = rng.standard_normal((len(slots), hkv, d)).astype(np.float16)
            cache_ops.scatter(kc, vc, K, V, slots, bs, kv_dtype, 2.0, 2.0)

        write(m.allocate(0, 13))
        m.fork(0, 1)
        r = m.append(1, 2)                # copy-on-write of the shared partial block
        assert r.cow_src >= 0
        cache_ops.block_copy(kc, vc, [(r.cow_src, r.cow_dst)])
        write(r.slots)
        write(m.allocate(2, 9))
        m.share_prefix(2, 2, 3)
        r = m.append(3, 5)                # the shared blocks are full: no copy
        assert r.cow_src < 0
        write(r.slots)
        seqs = [0, 1, 2, 3]
        gather = {s: (attention.gather_sequence(kc, m.block_table(s), m.num_tokens(s), bs, kv_dtype),
                      attention.gather_sequence(vc, m.block_table(s), m.num_tokens(s), bs, kv_dtype))
                  for s in seqs}
        out = m.swap_out([1, 3])
        cache_ops.block_swap(kc, vc, kh, vh, out)
        write(m.allocate(9, 4 * len(m.free_list())))   # reuse (and overwrite) every free block
        m.free_seq(9)
        back = m.swap_in([3, 1])
        cache_ops.block_swap(kh, vh, kc, vc, back)
        for s in seqs:
            K = attention.gather_sequence(kc, m.block_table(s), m.num_tokens(s), bs, kv_dtype)
            V = attention.gather_sequence(vc, m.block_table(s), m.num_tokens(s), bs, kv_dtype)
            assert not np.isnan(K).any() and not np.isnan(V).any()
            assert np.array_equal(K, gather[s][0]) and np.array_equal(V, gather[s][1]), (kv_dtype, s)


def check_swap_invariants(m: BlockAllocatorModel):
    check_invariants(m)
    href = [0] * m.num_host_blocks
    for s, t in m.host_tables.items():
        c = m.host_counts[s]
        assert len(t) == -(-c // m.bs)
        for h in t:
            href[h] += 1
    assert href == m.host_ref
    free = m.host_free_list()
    assert len(set(free)) == len(free)
    assert all(href[h] == 0 for h in free)
    assert set(free) | {h for h in range(m.num_host_blocks) if href[h]} == set(range(m.num_host_blocks))
    assert not set(m.tables) & set(m.host_tables)


swap_ops = st.tuples(
    st.sampled_from(["allocate", "append", "fork", "free", "swap_out", "swap_in", "preempt", "preempt_swap"]),
    st.lists(st.integers(0, 5), min_size=1, max_size=3), st.integers(0, 30))


@settings(max_examples=300, deadline=None)
@given(bs=st.sampled_from([1, 2, 4]), nb=st.integers(1, 20), nh=st.integers(0, 12),
       ops=st.lists(swap_ops, max_size=60))
def test_random_swap_ops_keep_invariants(bs, nb, nh, ops):
    m = BlockAllocatorModel(nb, bs)
    m.set_host_blocks(nh)
    for kind, ids, n in ops:
        before = m.state()
        try:
            if kind == "allocate":
                m.allocate(ids[0], n)
            elif kind == "append":
                m.append(ids[0], n % 6)
            elif kind == "fork":
                m.fork(ids[0], ids[-1])
            elif kind == "free":
                m.free_seq(ids[0])
            elif kind == "swap_out":
                pairs = m.swap_out(ids)
                assert len({d for d, _ in pairs}) == len(pairs)
            elif kind == "swap_in":
                m.swap_in(ids)
            else:
                running = sorted(m.tables)
                victims, _ = m.preempt_tail(running, n % (nb + 2), "swap" if kind == "preempt_swap" else "recompute")
                assert victims == list(reversed(running))[:len(victims)]
                assert m.available_blocks() >= n % (nb + 2)
        except AllocError:
            assert m.state() == before
        check_swap_invariants(m)


def test_preempt_workload_resumes_with_identical_outputs():
    """A Llama-2-7B-shaped batch of 16 with its newest 4 sequences preempted
    (swap, or recompute from the same K/V) and resumed decodes exactly like the
    plain batch: the oracle's outputs are equal to the last bit."""
    import workloads
    seqs = [0, 11, 12, 15]
    plain = runner.run(workloads.llama2_7b(max_steps=1, batch=16), steps=1, seqs=seqs)
    for mode in ("swap", "recompute"):
        wl = workloads.llama2_7b_preempt(mode, max_steps=1, batch=16, victims=4)
        r = runner.run(wl, steps=1, seqs=seqs)
        assert r.ctx_lens[0] == plain.ctx_lens[0]
        assert np.array_equal(r.outputs[0][seqs], plain.outputs[0][seqs]), mode
        # the resumed sequences live in other blocks than before
        assert any(r.tables[0][s] != plain.tables[0][s] for s in (12, 15))
