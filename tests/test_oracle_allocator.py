"""Pins for the oracle's block manager model.

Fixtures: the six-block refcount walkthrough ("vLLM Architecture and Memory
Use, ch. 3", §3.2), the four block-manager unit tests ("Inference Engine
Memory Optimisation", §3; one assert corrected, see the fixture), the RAG
pipeline simulation ("From OOM to Smooth Inference", §2.3). Invariants:
internal fragmentation per sequence in [0, block_size - 1] ("From OOM to
Smooth Inference", §2.1), refcounts equal to the number of table references,
pool conservation, no write into a shared block, failing calls change nothing.
"""
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle.allocator import (ERR_EXISTS, ERR_INVALID, ERR_NO_SEQ, ERR_OOM, AllocError,
                              BlockAllocatorModel)
from tests import alloc_driver


def make(nb, bs, order):
    return BlockAllocatorModel(nb, bs, order)


@pytest.mark.parametrize("case", alloc_driver.load("block_manager_unit_tests.json")["cases"],
                         ids=lambda c: c["name"])
def test_unit_cases(case):
    alloc_driver.run_unit_case(make, case, 16)


def test_refcount_walkthrough():
    alloc_driver.run_walkthrough(make)


def test_rag_simulation():
    alloc_driver.run_rag_simulation(make)


def test_constructor_validation():
    with pytest.raises(AllocError) as e:
        BlockAllocatorModel(0, 16)
    assert e.value.code == ERR_INVALID
    with pytest.raises(AllocError):
        BlockAllocatorModel(4, 0)
    with pytest.raises(AllocError):
        BlockAllocatorModel(4, 16, [0, 1, 1, 2])


def test_errors_change_nothing():
    m = BlockAllocatorModel(8, 4)
    m.allocate(1, 10)  # 3 blocks
    before = m.state()
    for call, code in [
        (lambda: m.allocate(1, 1), ERR_EXISTS),
        (lambda: m.allocate(2, 100), ERR_OOM),
        (lambda: m.append(9, 1), ERR_NO_SEQ),
        (lambda: m.append(1, 40), ERR_OOM),
        (lambda: m.free_seq(5), ERR_NO_SEQ),
        (lambda: m.fork(5, 6), ERR_NO_SEQ),
        (lambda: m.fork(1, 1), ERR_EXISTS),
        (lambda: m.share_prefix(1, 4, 7), ERR_INVALID),
        (lambda: m.share_prefix(1, 1, 1), ERR_EXISTS),
        (lambda: m.allocate(3, -1), ERR_INVALID),
    ]:
        with pytest.raises(AllocError) as e:
            call()
        assert e.value.code == code
        assert m.state() == before


def test_cow_oom_is_atomic():
    # the copy-on-write block and the growth blocks are checked together
    m = BlockAllocatorModel(3, 4)
    m.allocate(1, 6)  # 2 blocks, last one half full
    m.fork(1, 2)
    before = m.state()
    with pytest.raises(AllocError) as e:
        m.append(2, 3)  # needs 1 CoW block + 1 new block, 1 free
    assert e.value.code == ERR_OOM
    assert m.state() == before


def test_beam_cow_three_copies_last_in_place():
    # "From OOM to Smooth Inference", §6.1: forked beams copy only the last block
    m = BlockAllocatorModel(16, 4)
    m.allocate(0, 6)  # blocks 0, 1 (block 1 half full)
    for b in (1, 2, 3):
        m.fork(0, b)
    assert m.refcount(1) == 4
    pairs = []
    for b in (0, 1, 2, 3):
        r = m.append(b, 1)
        pairs.append((r.cow_src, r.cow_dst))
    assert pairs == [(1, 2), (1, 3), (1, 4), (-1, -1)]
    assert m.block_table(3) == [0, 1]
    assert [m.block_table(b) for b in (0, 1, 2)] == [[0, 2], [0, 3], [0, 4]]
    assert m.refcount(0) == 4 and m.refcount(1) == 1


def test_full_shared_block_is_not_copied():
    m = BlockAllocatorModel(8, 4)
    m.allocate(0, 8)  # two full blocks
    m.fork(0, 1)
    r = m.append(1, 1)
    assert (r.cow_src, r.cow_dst) == (-1, -1)
    assert m.block_table(1) == [0, 1, 2]
    assert r.slots == [2 * 4 + 0]


def test_append_more_than_a_block():
    m = BlockAllocatorModel(10, 4)
    m.allocate(0, 3)
    r = m.append(0, 9)  # 12 tokens -> 3 blocks
    assert m.block_table(0) == [0, 1, 2]
    assert r.slots == [3, 4, 5, 6, 7, 8, 9, 10, 11]


def test_share_prefix_counts():
    m = BlockAllocatorModel(10, 4)
    m.allocate(0, 10)  # blocks 0,1,2; 2 tokens in block 2
    m.share_prefix(0, 2, 1)
    assert m.num_tokens(1) == 8
    m.share_prefix(0, 3, 2)
    assert m.num_tokens(2) == 10
    r = m.append(2, 1)  # lands in shared, partial block 2 -> copy
    assert (r.cow_src, r.cow_dst) == (2, 3)
    r = m.append(1, 1)  # block 1 is full: new block, no copy
    assert (r.cow_src, r.cow_dst) == (-1, -1)


def test_zero_token_allocate():
    m = BlockAllocatorModel(4, 4)
    assert m.allocate(0, 0) == []
    assert m.block_table(0) == []
    r = m.append(0, 1)
    assert r.slots == [0] and m.block_table(0) == [0]


# ------------------------------------------------------------ invariants
def check_invariants(m: BlockAllocatorModel):
    refs = [0] * m.num_blocks
    for s, t in m.tables.items():
        c = m.counts[s]
        assert len(t) == -(-c // m.bs)
        frag = len(t) * m.bs - c
        assert 0 <= frag <= m.bs - 1
        for b in t:
            refs[b] += 1
    assert refs == m.ref
    free = m.free_list()
    evictable = m.evictable_list()
    assert len(set(free)) == len(free)
    assert len(set(evictable)) == len(evictable)
    for b in free + evictable:
        assert refs[b] == 0
    live = {b for b in range(m.num_blocks) if refs[b] > 0}
    assert not set(free) & set(evictable)
    assert set(free) | set(evictable) | live == set(range(m.num_blocks))
    # prefix cache: evictable blocks are cached, free ones are not; the chain of parents is closed
    for b in evictable:
        assert m.cache_entry(b) is not None
    for b in free:
        assert m.cache_entry(b) is None
    for b in range(m.num_blocks):
        e = m.cache_entry(b)
        if e is not None:
            assert e[0] == -1 or m.cache_entry(e[0]) is not None
            assert len(e[1]) == m.bs


op_strategy = st.tuples(
    st.sampled_from(["allocate", "append", "fork", "share", "free"]),
    st.integers(0, 5), st.integers(0, 5), st.integers(0, 40))


@settings(max_examples=300, deadline=None)
@given(bs=st.sampled_from([1, 2, 4, 16]), nb=st.integers(1, 24),
       ops=st.lists(op_strategy, max_size=60))
def test_random_ops_keep_invariants(bs, nb, ops):
    m = BlockAllocatorModel(nb, bs)
    for kind, a, b, n in ops:
        before = m.state()
        try:
            if kind == "allocate":
                m.allocate(a, n)
            elif kind == "append":
                r = m.append(a, n % 9)
                for slot in r.slots:  # never write into a shared block
                    assert m.refcount(slot // bs) == 1
            elif kind == "fork":
                m.fork(a, b)
            elif kind == "share":
                m.share_prefix(a, n % 4, b)
            else:
                m.free_seq(a)
        except AllocError:
            assert m.state() == before
        check_invariants(m)
