"""CPU oracle for the paged-KV decode path. TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct reference written from the
pages on paged KV caches (PagedAttention). Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The product library (``paged_kv_cache_60_amd``) never imports it,
and this package never imports the product library: the two share no code.
The seeded input generators in ``workloads/`` are the only thing both sides use.

Modules
-------
allocator   block manager model: FIFO free pool, block tables, refcounts,
            per-sequence token counts, fork / share-prefix / copy-on-write.
fp8         OCP e4m3fn encode (round-to-nearest-even, saturating) and decode,
            written from the format definition.
cache_ops   slot scatter into the paged cache and whole-block copy.
attention   gather-by-block-table then fp64 softmax attention for one decode
            token per sequence.
prefill     chunked (multi-token, causal) attention over the same paged
            cache: the positions a prompt did not find in the prefix cache.
kvsize      closed forms for KV bytes, pool sizing and reservation waste.
runner      drives a workload scenario through the functions above.

Every function cites the passage of the pages it follows as
"<page title>, <section>". Where the pages are silent the reading taken is
stated in the docstring.

Parity status: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` against printed values, closed forms, library
routines or brute force.
"""
