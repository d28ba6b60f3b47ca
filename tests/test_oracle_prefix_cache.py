"""Pins for the oracle's prefix cache ("Where Did the VRAM Go (KV cache
tutorial)", §4.2-4.4): a block's key is its token ids plus everything before
it, a new request maps hits into its table and prefills only the rest, shared
blocks carry reference counts, zero-count blocks wait for reuse, eviction is
least-recently-used, matching is exact at token level. The pins are closed
forms of that description (hits = leading full blocks that match exactly) and
invariants over random operation sequences, including a shadow of every slot's
content that checks a hit never maps a block whose content differs.
"""
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle.allocator import ERR_EXISTS, ERR_OOM, AllocError, BlockAllocatorModel
from tests.test_oracle_allocator import check_invariants


def prompt(n, base=1000):
    return list(range(base, base + n))


@pytest.mark.parametrize("bs,P", [(4, 10), (4, 12), (16, 100), (16, 1024), (16, 7)])
def test_identical_prompt_hits_every_full_block(bs, P):
    m = BlockAllocatorModel(64 + 2 * (P // bs + 1), bs)
    c0, s0 = m.allocate_prompt(0, prompt(P))
    assert c0 == 0 and len(s0) == P
    c1, s1 = m.allocate_prompt(1, prompt(P))
    assert c1 == (P // bs) * bs                     # the partial last block is never cached
    assert len(s1) == P - c1
    t0, t1 = m.block_table(0), m.block_table(1)
    assert t0[:P // bs] == t1[:P // bs]
    if P % bs:
        assert t0[-1] != t1[-1]
    for b in t0[:P // bs]:
        assert m.refcount(b) == 2                   # refcount = requests referencing the block
    st_ = m.stats()
    assert st_["prefix_hit_tokens"] == c1 and st_["prefix_query_tokens"] == 2 * P
    if P % bs == 0:
        assert st_["prefix_hit_tokens"] / st_["prefix_query_tokens"] == 0.5   # first 0 %, second 100 %


@pytest.mark.parametrize("k", [0, 1, 3, 4, 5, 8, 11, 12])
def test_prompts_diverging_at_token_k_hit_k_div_bs_blocks(k):
    bs, P = 4, 12
    m = BlockAllocatorModel(32, bs)
    a = prompt(P)
    b = list(a)
    if k < P:
        b[k] = -7
    m.allocate_prompt(0, a)
    c, _ = m.allocate_prompt(1, b)
    assert c == (k // bs) * bs if k < P else P


def test_same_block_tokens_after_a_different_prefix_miss():
    # block 1 holds the same four tokens in both prompts, but what precedes it differs
    bs = 4
    m = BlockAllocatorModel(16, bs)
    m.allocate_prompt(0, [1, 2, 3, 4, 9, 9, 9, 9])
    c, _ = m.allocate_prompt(1, [5, 6, 7, 8, 9, 9, 9, 9])
    assert c == 0
    assert m.block_table(0)[1] != m.block_table(1)[1]


def test_freed_prompt_stays_cached_until_evicted():
    bs = 4
    m = BlockAllocatorModel(6, bs)                  # ids 0..5
    m.allocate_prompt(0, prompt(10))                # blocks 0,1 (full, cached) and 2 (partial)
    m.free_seq(0)
    assert m.free_list() == [3, 4, 5, 2]            # the partial block returns to the free queue
    assert m.evictable_list() == [1, 0]             # deepest first
    assert m.available_blocks() == 6
    c, slots = m.allocate_prompt(1, prompt(10))
    assert c == 8 and m.block_table(1) == [0, 1, 3]  # revived from the cache, fresh tail from the queue
    assert m.evictable_list() == []
    assert slots == [12, 13]


def test_lru_eviction_order_children_first():
    bs = 2
    m = BlockAllocatorModel(6, bs)
    m.allocate_prompt(0, [1, 1, 2, 2])              # A: blocks 0, 1
    m.allocate_prompt(1, [3, 3, 4, 4])              # B: blocks 2, 3
    m.free_seq(0)                                   # evictable [1, 0]
    m.free_seq(1)                                   # evictable [1, 0, 3, 2]
    assert m.evictable_list() == [1, 0, 3, 2]
    m.allocate(2, 6)                                # 3 blocks: 4, 5 from the queue, then evict 1
    assert m.block_table(2) == [4, 5, 1]
    assert m.cache_entry(1) is None and m.cache_entry(0) == (-1, [1, 1])
    c, _ = m.allocate_prompt(3, [1, 1, 2, 2])       # A's first block still hits, its second was evicted
    assert c == 2 and m.block_table(3)[0] == 0
    assert m.evictable_list() == [2]                # block 3 (B's second) was evicted for A's new tail


def test_oom_leaves_state_and_revived_blocks_are_not_capacity():
    bs = 2
    m = BlockAllocatorModel(4, bs)
    m.allocate_prompt(0, [1, 1, 2, 2, 3, 3])        # blocks 0, 1, 2 cached
    m.free_seq(0)                                   # evictable [2, 1, 0], free [3]
    before = m.state()
    # hits blocks 0 and 1 (reviving them), needs 3 fresh: only block 3 and evictable 2 remain
    with pytest.raises(AllocError) as e:
        m.allocate_prompt(1, [1, 1, 2, 2, 5, 5, 6, 6, 7])
    assert e.value.code == ERR_OOM
    assert m.state() == before
    with pytest.raises(AllocError) as e:
        m.allocate_prompt(0, [1, 1])
        m.allocate_prompt(0, [1, 1])
    assert e.value.code == ERR_EXISTS


def test_many_requests_share_one_prefix():
    # 256 requests with one 1024-token prefix and private suffixes: the prefix is stored once
    bs, pre = 16, 1024
    m = BlockAllocatorModel(64 + 256 * 4, bs)
    for s in range(256):
        c, _ = m.allocate_prompt(s, prompt(pre) + prompt(17 + s % 30, base=10 ** 6 * (s + 1)))
        assert c == (0 if s == 0 else pre)
    t0 = m.block_table(0)[:64]
    for b in t0:
        assert m.refcount(b) == 256
    assert all(m.block_table(s)[:64] == t0 for s in range(256))


# --------------------------------------------------------------- random sequences
TOKENS = st.lists(st.integers(0, 2), min_size=0, max_size=14)   # small alphabet: many shared prefixes
op_strategy = st.tuples(st.sampled_from(["prompt", "prompt", "append", "fork", "free", "allocate"]),
                        st.integers(0, 5), st.integers(0, 5), TOKENS)


@settings(max_examples=300, deadline=None)
@given(bs=st.sampled_from([1, 2, 3, 4]), nb=st.integers(1, 20), ops=st.lists(op_strategy, max_size=50))
def test_random_prompt_ops_keep_invariants_and_content(bs, nb, ops):
    m = BlockAllocatorModel(nb, bs)
    content = {}        # slot -> token written there
    prompts = {}        # seq -> its prompt, for sequences made by allocate_prompt
    marker = [10 ** 6]  # unique tokens for appended positions

    def fresh_token():
        marker[0] += 1
        return marker[0]

    for kind, a, b, toks in ops:
        before = m.state()
        try:
            if kind == "prompt":
                c, slots = m.allocate_prompt(a, toks)
                for t, sl in zip(toks[c:], slots):
                    content[sl] = t
                prompts[a] = list(toks)
            elif kind == "allocate":
                slots = m.allocate(a, len(toks))
                for sl in slots:
                    content[sl] = fresh_token()
            elif kind == "append":
                r = m.append(a, 1 + b % 3)
                if r.cow_src >= 0:
                    for o in range(bs):
                        if r.cow_src * bs + o in content:
                            content[r.cow_dst * bs + o] = content[r.cow_src * bs + o]
                for sl in r.slots:
                    assert m.refcount(sl // bs) == 1
                    content[sl] = fresh_token()
            elif kind == "fork":
                m.fork(a, b)
                if a in prompts:
                    prompts[b] = prompts[a]
            else:
                m.free_seq(a)
                prompts.pop(a, None)
        except AllocError:
            assert m.state() == before
        check_invariants(m)
        # every live prompt reads exactly its own tokens through its table
        for s, toks_s in prompts.items():
            if s not in m.tables:
                continue
            n = min(len(toks_s), m.num_tokens(s))
            got = [content.get(sl) for sl in m.slots(s, 0, n)]
            assert got == toks_s[:n]
        # a cached block holds its key's tokens and, through its parents, the whole prefix
        for blk in range(m.num_blocks):
            e = m.cache_entry(blk)
            if e is not None:
                assert [content.get(blk * bs + o) for o in range(bs)] == e[1]
        # the evictable list holds a block's cached children before the block itself
        ev = m.evictable_list()
        pos = {x: i for i, x in enumerate(ev)}
        for blk in ev:
            for child in range(m.num_blocks):
                e = m.cache_entry(child)
                if e is not None and e[0] == blk:
                    assert child in pos and pos[child] < pos[blk]


def test_cached_workload_gives_the_scripted_outputs_exactly():
    """Sharing found by the prefix cache and sharing written into the script
    give the same float64 attention outputs (same K/V per logical position),
    while the cached run writes the system prompt once."""
    import numpy as np

    import workloads
    from oracle import runner
    scripted = runner.run(workloads.qwen3_prefix(batch=4, max_steps=1), steps=1)
    cached_wl = workloads.qwen3_prefix_cached(batch=4, max_steps=1)
    cached = runner.run(cached_wl, steps=1, keep_rounds=True)
    assert np.array_equal(scripted.outputs[0], cached.outputs[0])
    hits = [c for _, c, _ in cached.rounds[0].prompts]
    assert hits == [0, 1024, 1024, 1024]
    t = cached.tables[0]
    assert all(t[s][:64] == t[0][:64] for s in range(4))
    assert cached.alloc.stats()["prefix_hit_tokens"] == 3 * 1024
