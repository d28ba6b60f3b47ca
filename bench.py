"""Benchmark of the paged KV decode step on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--config 2] [--flush]

One step = the whole hot path for one batch: host block-manager bookkeeping
(append one token per sequence), one host-to-device copy of the step's
metadata, copy-on-write block copies (if any), paged_kv_write of the new
tokens, paged_attn_decode (pass 1 over equal shares of the KV, pass 2 combining
split segments). Inputs are resident
in HBM before the timed region; the setup (prompt writes) is untimed.

Default workload: Llama-2-7B-shaped single layer, batch 64, 32/32 heads,
head_dim 128, block size 16, fp16 KV, context lengths uniform in [128, 2048].

Printed: one JSON line. `value` is the whole-step throughput in GB/s of
algorithmic bytes (K/V read by attention, queries, block tables, context
lengths, output, plus the bytes paged_kv_write and paged_block_copy move) over
the wall time of the timed steps. K/V blocks that several sequences share
count once (at the most rows any sequence reads from them): that is the HBM
lower bound; `value_logical_gbs` counts every sequence's reads. Without shared
blocks the two are equal. `roofline` is for the dominant kernel,
attention pass 1: its algorithmic bytes per launch over its average launch
duration, measured with HIP events on every EVENT_EVERY-th timed launch. The
events are attached to the pass-1 launch itself (the library's
pkv_time_next_pass1 hook launches it with hipExtLaunchKernel), so they time
the kernel's execution alone, on the stream it runs on. Under the profiler
the launch that carries them starts and ends a few microseconds apart from
its neighbours in the stream; hence only every EVENT_EVERY-th launch.
`cpu_baseline` is the CPU oracle timed on a sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved HBM GB/s (% of peak) + KV tokens read/sec"
PEAK_GBS = 8000.0  # MI355X HBM3E
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
EVENT_EVERY = 5  # timed steps per pass-1 event pair


KERNEL_SOURCES = ("attn_decode.hip", "attn_gqa_mfma.hpp", "attn_group_mfma.hpp", "device_common.hpp")
PREFILL_SOURCES = ("attn_prefill.hip", "device_common.hpp")


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    """sha256[:16] over the sources the attention kernels are built from."""
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "paged_kv_cache_60_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def attention_bytes(ctx, hq, hkv, d, bs, elem):
    """Algorithmic bytes of one decode-attention call: (pass 1, total), counting
    every sequence's K/V reads (logical bytes)."""
    ctx = np.asarray(ctx, dtype=np.int64)
    B = len(ctx)
    kv = int((ctx * hkv * d * 2 * elem).sum())
    tables = int(((ctx + bs - 1) // bs).sum()) * 4
    q_in = B * hq * d * 2
    out = B * hq * d * 2
    p1 = kv + q_in + tables + 4 * B
    return p1, p1 + out


def unique_kv_bytes(tables, ctx, hkv, d, bs, elem):
    """K/V bytes of one call counting each physical block once, at the largest
    number of its rows any sequence reads: the HBM lower bound when sequences
    share blocks (a common prefix, the prompt of a beam group)."""
    ctx = np.asarray(ctx, dtype=np.int64)
    nblk = (ctx + bs - 1) // bs
    idx = np.arange(tables.shape[1], dtype=np.int64)
    live = idx[None, :] < nblk[:, None]
    used = np.clip(ctx[:, None] - idx[None, :] * bs, 0, bs)
    phys = tables[live].astype(np.int64)
    rows = np.zeros(int(phys.max()) + 1 if phys.size else 1, dtype=np.int64)
    np.maximum.at(rows, phys, used[live])
    return int(rows.sum()) * hkv * d * 2 * elem


def write_bytes(T, hkv, d, elem):
    return T * hkv * d * (2 + elem) * 2 + 8 * T


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(wl, target_s=15.0):
    """Oracle timing on the host: gather + fp64 attention for whole sequences of
    the workload, sequence by sequence until ~target_s of work is done."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as oattn
    from oracle import cache_ops
    from oracle.allocator import BlockAllocatorModel
    from oracle.runner import empty_cache

    alloc = BlockAllocatorModel(wl.num_blocks, wl.block_size, wl.free_order)
    kc = empty_cache(wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim, wl.kv_dtype)
    vc = empty_cache(wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim, wl.kv_dtype)
    order = list(wl.batch)
    # setup + one decode step, on the host model, writing every sequence's tokens
    for ops in wl.setup_rounds + [wl.step_ops(0)]:
        for op in ops:
            if op.kind == "allocate":
                slots = alloc.allocate(op.seq, op.n)
            elif op.kind == "append":
                r = alloc.append(op.seq, op.n)
                slots = r.slots
                if r.cow_src >= 0:
                    cache_ops.block_copy(kc, vc, [(r.cow_src, r.cow_dst)])
            elif op.kind == "share_prefix":
                alloc.share_prefix(op.src, op.n, op.seq)
                continue
            elif op.kind == "fork":
                alloc.fork(op.src, op.seq)
                continue
            if op.n:
                K, V = wl.op_kv(op)
                cache_ops.scatter(kc, vc, K, V, slots, wl.block_size, wl.kv_dtype,
                                  wl.k_inv_scale, wl.v_inv_scale)
    q = wl.queries(0)
    tables = [alloc.block_table(s) for s in order]
    lens = [alloc.num_tokens(s) for s in order]
    done, tokens, elapsed = [], 0, 0.0
    with threadpool_limits(limits=1):
        # whole sequences, the batch over and over, until ~target_s of work
        while elapsed < target_s and len(done) < 64 * len(order):
            i = len(done) % len(order)
            t0 = time.perf_counter()
            oattn.decode_attention(q, kc, vc, tables, lens, wl.block_size, wl.sm_scale, wl.kv_dtype,
                                   wl.k_scale, wl.v_scale, seqs=[i])
            elapsed += time.perf_counter() - t0
            done.append(i)
            tokens += lens[i]
    elem = 1 if wl.kv_dtype != "f16" else 2
    _, nbytes = attention_bytes([lens[i] for i in done], wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                wl.block_size, elem)
    return {
        "value": round(nbytes / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"gather + fp64 attention of {len(done)} sequences (the {len(order)} of one decode step, "
                  f"in order, repeated; {tokens} KV tokens, all {wl.num_q_heads} query heads), "
                  f"{elapsed:.1f} s on one host core",
        "kv_tokens_per_s": round(tokens / elapsed, 1),
    }


def load_counters(config_name, sources=KERNEL_SOURCES):
    """HBM bytes per launch of the workload's dominant kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source;
    else None."""
    try:
        with open(PROFILE_COUNTERS) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(config_name)
    if not entry or entry.get("kernel_source_sha256_16") != kernel_source_hash(sources):
        return None
    return entry.get("hbm_bytes_per_launch")


PREFILL_METRIC = "paged prefill attention: achieved TFLOP/s (% of MFMA fp16 dense peak) + query tokens/sec"
PEAK_TFLOPS_F16 = 2500.0  # MI355X dense fp16 matrix peak
PREFILL_WORKLOADS = {"qwen3": "qwen3_prefill", "llama2": "llama2_7b_chunked"}


def prefill_flops(ctx, chunks, hq, d):
    """Algorithmic flops of one chunked-prefill call: q.k and p.v (2 flops per
    multiply-add each) over the positions every query row sees, causal."""
    total = 0
    for L, n in zip(ctx, chunks):
        pos = np.arange(int(L) - int(n), int(L), dtype=np.int64)
        total += int(np.maximum(pos + 1, 0).sum())
    return 4 * hq * d * total


def prefill_cpu_baseline(wl, target_s=15.0):
    """Oracle prefill (gather + fp64 causal attention) on whole sequences of the
    workload, one at a time until ~target_s of work is done, on one host core."""
    from threadpoolctl import threadpool_limits

    from oracle import runner

    o = runner.run_prefill(wl, seqs=[])  # setup only: the allocator and the caches
    done, flops, elapsed = [], 0, 0.0
    from oracle.prefill import prefill_attention
    with threadpool_limits(limits=1):
        # whole sequences' chunks, the batch over and over, until ~target_s of work
        while elapsed < target_s and len(done) < 16 * len(wl.batch):
            i = len(done) % len(wl.batch)
            n = o.chunks[i]
            q = wl.prefill_queries(wl.batch[i], n)
            t0 = time.perf_counter()
            prefill_attention(q, [0, n], o.k_cache, o.v_cache, [o.tables[i]], [o.ctx_lens[i]], wl.block_size,
                              wl.sm_scale, wl.kv_dtype, wl.k_scale, wl.v_scale)
            elapsed += time.perf_counter() - t0
            done.append(i)
            flops += prefill_flops([o.ctx_lens[i]], [n], wl.num_q_heads, wl.head_dim)
    rows = sum(o.chunks[i] for i in done)
    return {
        "value": round(flops / elapsed / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"gather + fp64 causal attention of {len(done)} sequences' chunks (the {len(wl.batch)} of one "
                  f"prefill pass, in order, repeated as needed; {rows} query rows), {elapsed:.1f} s on one host core",
        "query_tokens_per_s": round(rows / elapsed, 1),
    }


def bench_prefill(args):
    """One step = paged_kv_write of every chunk's K/V + paged_attn_prefill over the batch."""
    import torch

    import workloads
    from paged_kv_cache_60_amd import _lib, harness, ops
    _lib.load()

    wl = getattr(workloads, PREFILL_WORKLOADS[args.prefill])()
    log(f"bench: {wl.name}: setup")
    eng = harness.make_engine(wl, poison=False)
    cached = harness.replay_setup(eng, wl, chunk_tokens=1 << 16)
    q, q_start, chunks = harness.prefill_inputs(wl, cached)
    tables, ctx = eng.prepare_prefill(wl.batch, wl.max_blocks_per_seq)
    ctx_h = ctx.cpu().numpy()
    # the chunks' K/V rows and slots, staged in HBM (re-written each step: same values, same slots)
    ks, vs, sl = [], [], []
    ops_by_seq = {o.seq: o for r in wl.setup_rounds for o in r}
    for s, n in zip(wl.batch, chunks):
        op = ops_by_seq[s]
        L = int(ctx_h[wl.batch.index(s)])
        if op.kind == "prompt":
            K, V = wl.prompt_kv(op, L - n)
        else:
            K, V = wl.op_kv(op)
            K, V = K[L - n:], V[L - n:]
        ks.append(K)
        vs.append(V)
        sl.append(np.asarray(eng.bm.slots(s, L - n, n), dtype=np.int64))
    k_new = torch.from_numpy(np.concatenate(ks)).cuda()
    v_new = torch.from_numpy(np.concatenate(vs)).cuda()
    slots = torch.from_numpy(np.concatenate(sl)).cuda()
    del ks, vs
    out = torch.empty_like(q)
    torch.cuda.synchronize()

    def step(ev=None):
        ops.paged_kv_write(k_new, v_new, eng.k_cache, eng.v_cache, slots, wl.kv_dtype, wl.k_inv_scale,
                           wl.v_inv_scale)
        if ev is not None:
            ev[0].record()
        eng.prefill(tables, ctx, q, q_start, out)
        if ev is not None:
            ev[1].record()

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    log(f"bench: timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_ms = [a.elapsed_time(b) for a, b in evs]
    hq, hkv, d = wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    flops = prefill_flops(ctx_h, chunks, hq, d)
    rows = int(sum(chunks))
    attn_s = float(np.mean(attn_ms)) / 1e3
    achieved = flops / attn_s / 1e12
    value = flops * args.steps / wall / 1e12
    result = {
        "metric": PREFILL_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if wl.kv_dtype == "f16" else ("fp8e4m3" if wl.kv_dtype == "fp8" else "fp8e5m2") + "-kv/f16",
        "data": "synthetic",
        "config": {**wl.summary(), "query_rows": rows, "prefix_cache_hit_tokens": int(sum(cached.values())),
                   "timing": "wall clock per step (write + prefill); roofline from events around the prefill"},
        "pct_of_peak": round(100.0 * value / PEAK_TFLOPS_F16, 2),
        "query_tokens_per_s": round(rows * args.steps / wall, 1),
        "prefill_us": round(attn_s * 1e6, 2),
        "prefill_us_p10_p50_p90": [round(float(x) * 1e3, 2) for x in np.percentile(attn_ms, [10, 50, 90])],
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_TFLOPS_F16,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_TFLOPS_F16, 4),
            "traffic": load_counters(wl.name, PREFILL_SOURCES),
            "kernel": "attn_prefill_kernel",
            "flops_per_launch": flops,
        },
    }
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        result["cpu_baseline"] = prefill_cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)


SWAP_METRIC = "preemption by swapping: paged_block_swap bus GB/s (device <-> pinned host), per direction"
PCIE_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction


def bench_swap(args):
    """Time paged_block_swap on the preemption workload: the 16 newest sequences
    of the Llama-2-7B batch (their whole K/V) copied to the pinned host pool
    (out) and back (in); each timed step is one out and one in."""
    import torch

    import workloads
    from paged_kv_cache_60_amd import _lib, harness, ops
    _lib.load()

    wl = workloads.llama2_7b_preempt("swap")
    log(f"bench: {wl.name}: setup")
    eng = harness.make_engine(wl, poison=False)
    harness.replay_setup(eng, wl, chunk_tokens=1 << 16)
    tail = wl.meta["preempted"]
    dev = []
    for s_ in tail:
        dev += eng.bm.block_table(s_)
    n = len(dev)
    assert n == wl.num_host_blocks
    out_pairs = torch.tensor([[b, h] for h, b in enumerate(dev)], dtype=torch.int32, device="cuda")
    in_pairs = torch.tensor([[h, b] for h, b in enumerate(dev)], dtype=torch.int32, device="cuda")
    nbytes = 2 * n * eng.block_bytes  # K and V
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        ops.paged_block_swap(eng.k_cache, eng.v_cache, eng.k_host, eng.v_host, out_pairs, "out")
        ops.paged_block_swap(eng.k_cache, eng.v_cache, eng.k_host, eng.v_host, in_pairs, "in")
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in ev:
        e[0].record()
        ops.paged_block_swap(eng.k_cache, eng.v_cache, eng.k_host, eng.v_host, out_pairs, "out")
        e[1].record()
        ops.paged_block_swap(eng.k_cache, eng.v_cache, eng.k_host, eng.v_host, in_pairs, "in")
        e[2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_out = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) / 1e3
    t_in = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) / 1e3
    value = 2 * nbytes * args.steps / wall / 1e9
    best = max(nbytes / t_out, nbytes / t_in) / 1e9
    result = {
        "metric": SWAP_METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": wl.name, "swapped_sequences": len(tail), "blocks": n,
                   "bytes_per_direction": nbytes, "block_bytes": eng.block_bytes,
                   "timing": "wall clock of out + in per step; per direction from events"},
        "swap_out_gbs": round(nbytes / t_out / 1e9, 2),
        "swap_in_gbs": round(nbytes / t_in / 1e9, 2),
        "swap_out_us": round(t_out * 1e6, 1),
        "swap_in_us": round(t_in * 1e6, 1),
        "roofline": {
            "bound": "pcie",
            "achieved": round(best, 2),
            "peak": PCIE_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(best / PCIE_PEAK_GBS, 4),
            "traffic": None,
            "kernel": "block_swap_kernel",
        },
    }
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle block swap)")
        result["cpu_baseline"] = swap_cpu_baseline(eng.block_bytes, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def swap_cpu_baseline(block_bytes, target_s=15.0, n=256):
    """Oracle block swap (cache_ops.block_swap, whole blocks between two host
    arrays standing for the device and host pools) of n blocks, out and in,
    repeated until ~target_s."""
    from oracle import cache_ops
    elems = block_bytes // 2
    g = np.random.default_rng(61)
    dev_k = g.standard_normal((n, elems), dtype=np.float32).astype(np.float16)
    dev_v = g.standard_normal((n, elems), dtype=np.float32).astype(np.float16)
    host_k, host_v = np.zeros_like(dev_k), np.zeros_like(dev_v)
    out_pairs = [(b, n - 1 - b) for b in range(n)]
    in_pairs = [(h, b) for b, h in out_pairs]
    rounds, elapsed = 0, 0.0
    while elapsed < target_s and rounds < 10000:
        t0 = time.perf_counter()
        cache_ops.block_swap(dev_k, dev_v, host_k, host_v, out_pairs)
        cache_ops.block_swap(host_k, host_v, dev_k, dev_v, in_pairs)
        elapsed += time.perf_counter() - t0
        rounds += 1
    nbytes = 2 * 2 * n * block_bytes  # K and V, out and in
    return {
        "value": round(nbytes * rounds / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"cache_ops.block_swap of {n} blocks of {block_bytes} bytes (K and V), out and in, "
                  f"{rounds} rounds, {elapsed:.1f} s on one host core (host arrays on both sides)",
    }


SCATTER_METRIC = "paged_kv_write / paged_block_copy: achieved HBM GB/s (bytes read + written)"
SCATTER_SOURCES = ("kv_write.hip", "block_copy.hip", "device_common.hpp")


def bench_scatter(args):
    """paged_kv_write and paged_block_copy at sizes where HBM, not latency, is
    the bound: a prefill-sized scatter of 65 536 tokens into shuffled slots of a
    Llama-2-7B-shaped layer (fp16 copy) and of the beam workload's layer (e4m3
    encode, one scale per tensor), and 2048 copy-on-write pairs of
    Llama-2-7B-shaped blocks. Each is timed by events around every launch
    (median of --steps). value = the fp16 scatter's GB/s."""
    import torch

    from paged_kv_cache_60_amd import ops
    g = torch.Generator(device="cpu").manual_seed(60)
    gd = torch.Generator(device="cuda").manual_seed(60)

    def scatter_case(hkv, d, bs, kv, T):
        nb = (T * 11 // 10 + bs - 1) // bs
        slots = torch.randperm(nb * bs, generator=g)[:T].to(torch.int64).cuda()
        k = torch.randn((T, hkv, d), generator=gd, dtype=torch.float16, device="cuda")
        v = torch.randn((T, hkv, d), generator=gd, dtype=torch.float16, device="cuda")
        cdt = torch.float16 if kv == "f16" else torch.uint8
        kc = torch.zeros((nb, hkv, bs, d), dtype=cdt, device="cuda")
        vc = torch.zeros_like(kc)
        e = 2 if kv == "f16" else 1
        nbytes = 2 * T * hkv * d * 2 + 2 * T * hkv * d * e + T * 8
        inv = 1.0 if kv == "f16" else 448.0 / 4.5
        run = lambda: ops.paged_kv_write(k, v, kc, vc, slots, kv, inv, inv)  # noqa: E731
        return run, nbytes, {"tokens": T, "kv_heads": hkv, "head_dim": d, "block_size": bs, "kv_dtype": kv}

    def copy_case(hkv, d, bs, n):
        nb = 2 * n + 16
        perm = torch.randperm(nb, generator=g)
        pairs = torch.stack([perm[:n], perm[n:2 * n]], 1).to(torch.int32).contiguous().cuda()
        kc = torch.randn((nb, hkv, bs, d), generator=gd, dtype=torch.float16, device="cuda")
        vc = torch.randn((nb, hkv, bs, d), generator=gd, dtype=torch.float16, device="cuda")
        nbytes = 2 * 2 * n * hkv * bs * d * 2 + n * 8
        run = lambda: ops.paged_block_copy(kc, vc, pairs)  # noqa: E731
        return run, nbytes, {"pairs": n, "kv_heads": hkv, "head_dim": d, "block_size": bs, "kv_dtype": "f16"}

    cases = {"write_f16_llama2_7b": scatter_case(32, 128, 16, "f16", 65536),
             "write_e4m3_beam": scatter_case(8, 128, 64, "fp8", 65536),
             "copy_f16_llama2_7b": copy_case(32, 128, 16, 2048)}
    res = {}
    for name, (run, nbytes, shape) in cases.items():
        log(f"bench: scatter {name}")
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        ts = []
        for _ in range(args.steps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            run()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / 1e3)
        t = float(np.median(ts))
        res[name] = {**shape, "bytes": nbytes, "us": round(t * 1e6, 2), "gbs": round(nbytes / t / 1e9, 2),
                     "us_p10_p50_p90": [round(float(x) * 1e6, 2) for x in np.percentile(ts, [10, 50, 90])]}
    main_case = res["write_f16_llama2_7b"]
    result = {
        "metric": SCATTER_METRIC,
        "value": main_case["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_case["us"] / 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "scatter_llama2_7b_65536_tokens", **{k: v for k, v in main_case.items()
                                                                     if k in ("tokens", "kv_heads", "head_dim",
                                                                              "block_size", "kv_dtype")},
                   "timing": "events around every launch, median"},
        "cases": res,
        "roofline": {
            "bound": "hbm",
            "achieved": main_case["gbs"],
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(main_case["gbs"] / PEAK_GBS, 4),
            "traffic": load_counters("scatter_llama2_7b_65536_tokens", SCATTER_SOURCES),
            "kernel": "kv_write_kernel",
        },
    }
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle scatter)")
        result["cpu_baseline"] = scatter_cpu_baseline(args.cpu_seconds)
    print(json.dumps(result), flush=True)


def scatter_cpu_baseline(target_s=15.0, T=4096):
    """Oracle scatter (cache_ops.scatter, token by token) of T tokens of the
    Llama-2-7B layer shape into shuffled slots, repeated until ~target_s."""
    from threadpoolctl import threadpool_limits

    from oracle import cache_ops
    hkv, d, bs = 32, 128, 16
    g = np.random.default_rng(60)
    nb = (T * 11 // 10 + bs - 1) // bs
    slots = g.permutation(nb * bs)[:T].astype(np.int64)
    k = g.standard_normal((T, hkv, d), dtype=np.float32).astype(np.float16)
    v = g.standard_normal((T, hkv, d), dtype=np.float32).astype(np.float16)
    kc = np.zeros((nb, hkv, bs, d), dtype=np.float16)
    vc = np.zeros_like(kc)
    nbytes = 2 * T * hkv * d * 2 * 2 + T * 8
    passes, elapsed = 0, 0.0
    with threadpool_limits(limits=1):
        while elapsed < target_s and passes < 1000:
            t0 = time.perf_counter()
            cache_ops.scatter(kc, vc, k, v, slots, bs)
            elapsed += time.perf_counter() - t0
            passes += 1
    return {
        "value": round(nbytes * passes / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"cache_ops.scatter of {T} fp16 tokens (32 KV heads, head_dim 128, shuffled slots), "
                  f"{passes} passes, {elapsed:.1f} s on one host core",
        "tokens_per_s": round(T * passes / elapsed, 1),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload 1-5 (2 = Llama-2-7B batch 64)")
    ap.add_argument("--partition", type=int, default=0,
                    help="tokens per attention worker (0 = the library default worker count)")
    ap.add_argument("--flush", action="store_true", help="evict L2/MALL between steps (time by events)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--kv", choices=["fp8", "fp8_e5m2"], default=None,
                    help="fp8 format of the beam workload (--config 5): e4m3 (default) or e5m2")
    ap.add_argument("--per-head", action="store_true",
                    help="one fp8 scale per KV head for the beam workload (--config 5)")
    ap.add_argument("--prefill", choices=sorted(PREFILL_WORKLOADS),
                    help="time chunked prefill instead of decode (qwen3: prefix-cache prefill, batch 256; "
                         "llama2: last-512-token chunks, batch 64)")
    ap.add_argument("--swap", action="store_true",
                    help="time paged_block_swap (preemption by swapping, 16 sequences of the Llama-2-7B batch)")
    ap.add_argument("--scatter", action="store_true",
                    help="time paged_kv_write (fp16 and e4m3, 65 536 tokens) and paged_block_copy (2048 pairs)")
    ap.add_argument("--shared", dest="shared", action="store_true", default=None,
                    help="attend with paged_attn_decode_shared: runs of the batch that share leading blocks "
                         "(beams of one prompt, a common prefix) read them once (default: when the block "
                         "manager finds such runs)")
    ap.add_argument("--no-shared", dest="shared", action="store_false",
                    help="attend with paged_attn_decode even where sequences share blocks")
    ap.add_argument("--calibrate", action="store_true",
                    help="first run one plain 256 MiB device copy (known bytes, for counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode path "
              f"runs on a single GPU", file=sys.stderr)
        sys.exit(2)
    import torch

    import workloads
    from paged_kv_cache_60_amd import _lib, harness
    from paged_kv_cache_60_amd import ops
    _lib.load()  # fail loudly if the HIP library is missing

    if args.calibrate:
        # a plain copy of known size: the counter runs scale FETCH_SIZE / WRITE_SIZE by what
        # they read for this dispatch
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    if args.prefill:
        bench_prefill(args)
        return
    if args.swap:
        bench_swap(args)
        return
    if args.scatter:
        bench_scatter(args)
        return

    total_steps = args.warmup + args.steps
    fp8_kw = {}
    if args.kv or args.per_head:
        if args.config != 5:
            print("--kv / --per-head apply to the fp8 beam workload (--config 5)", file=sys.stderr)
            sys.exit(2)
        fp8_kw = {"kv_dtype": args.kv or "fp8", "per_head": args.per_head}
    wl = workloads.make(args.config, max_steps=total_steps + 1, **fp8_kw)
    log(f"bench: {wl.name}: setup")
    dev = torch.device("cuda")
    eng = harness.make_engine(wl, poison=False)
    harness.replay_setup(eng, wl, chunk_tokens=1 << 16)
    eng.prepare_steps(wl.batch, wl.max_blocks_per_seq, args.partition, shared_prefix=args.shared)
    workers = ops.decode_workers(len(wl.batch), wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size,
                                 wl.max_blocks_per_seq, wl.kv_dtype, args.partition)
    group = wl.num_q_heads // wl.num_kv_heads
    kernel = "attn_partition_mfma_kernel" if group >= 4 else "attn_partition_kernel"
    shared = eng.groups is not None
    if shared:
        # the grouped pass 1 runs one worker (wave) per SIMD for an fp16 cache, two for fp8
        workers = (1 if wl.kv_dtype == "f16" else 2) * 4 * torch.cuda.get_device_properties(0).multi_processor_count
        # one grouped pass 1 over every sequence: each group's shared blocks once, then the members' tails
        kernel = "attn_group_mfma_kernel"
        log(f"bench: {eng.groups.shape[1]} shared-prefix groups")

    # stage every step's inputs in HBM before timing
    B = len(wl.batch)
    inputs = [harness.step_inputs(wl, s) for s in range(total_steps)]
    out = torch.empty((B, wl.num_q_heads, wl.head_dim), dtype=torch.float16, device=dev)
    flush_buf = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device=dev) if args.flush else None
    elem = 1 if wl.kv_dtype != "f16" else 2
    torch.cuda.synchronize()

    def one_step(s, ev=None):
        slot, n_cow, n_upd = eng.host_step()
        k, v, q = inputs[s]
        if ev is not None:
            ops.time_next_pass1(ev[0], ev[1])  # this step's pass-1 launch records the pair
        eng.device_step(slot, n_cow, n_upd, k, v, q, out)
        return n_cow

    log(f"bench: warmup {args.warmup}")
    for s in range(args.warmup):
        one_step(s)
        if flush_buf is not None:
            flush_buf.zero_()
    torch.cuda.synchronize()

    cow_total = 0
    ev_steps = [i for i in range(args.steps) if i % EVENT_EVERY == EVENT_EVERY - 1] or [args.steps - 1]
    ev_pairs = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for i in ev_steps}
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    for a_, b_ in ev_pairs.values():  # create the events' handles before the timed region
        a_.record()
        b_.record()
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        s = args.warmup + i
        if flush_buf is not None:
            step_ev[i][0].record()
        cow_total += one_step(s, ev_pairs.get(i))
        if flush_buf is not None:
            step_ev[i][1].record()
            flush_buf.zero_()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # context lengths of the timed steps: the final lengths minus the steps after each
    tab_final, ctx_final = eng.host_tables()
    ctx_steps = [ctx_final - (args.steps - 1 - i) for i in range(args.steps)]
    p1_ms = [a.elapsed_time(b) for a, b in ev_pairs.values()]
    step_ms = [a.elapsed_time(b) for a, b in step_ev] if flush_buf is not None else [wall / args.steps * 1e3]
    hq, hkv, d, bs = wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size

    def step_bytes(c, unique):
        """(pass-1 bytes, whole-step bytes) of a step with context lengths c."""
        p1, tot = attention_bytes(c, hq, hkv, d, bs, elem)
        if unique:
            delta = int((np.asarray(c, dtype=np.int64) * hkv * d * 2 * elem).sum()) - \
                unique_kv_bytes(tab_final, c, hkv, d, bs, elem)
            p1, tot = p1 - delta, tot - delta
        return p1, tot + write_bytes(B, hkv, d, elem)

    uniq = [step_bytes(c, True) for c in ctx_steps]
    logi = [step_bytes(c, False) for c in ctx_steps]
    cow_bytes = cow_total * eng.block_bytes * 4  # read + write, K and V
    tot_bytes = sum(t for _, t in uniq) + cow_bytes
    tot_bytes_logical = sum(t for _, t in logi) + cow_bytes
    p1_bytes = [uniq[i][0] for i in ev_pairs]
    p1_bytes_logical = [logi[i][0] for i in ev_pairs]
    kv_tokens = sum(int(c.sum()) for c in ctx_steps)

    if args.flush:
        elapsed = sum(step_ms) / 1e3  # GPU time of the steps, flushes excluded
    else:
        elapsed = wall
    ms_per_step = elapsed / args.steps * 1e3
    value = tot_bytes / elapsed / 1e9
    p1_avg_s = sum(p1_ms) / len(p1_ms) / 1e3
    achieved = (sum(p1_bytes) / len(p1_bytes)) / p1_avg_s / 1e9
    achieved_logical = (sum(p1_bytes_logical) / len(p1_bytes_logical)) / p1_avg_s / 1e9
    traffic = load_counters(wl.name + ("_shared" if shared else ""))

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if wl.kv_dtype == "f16" else ("fp8e4m3" if wl.kv_dtype == "fp8" else "fp8e5m2") + "-kv/f16",
        "data": "synthetic",
        "config": {
            **wl.summary(),
            "mean_ctx_len": round(float(np.mean([c.mean() for c in ctx_steps])), 1),
            "partition_tokens": args.partition,
            "attention_workers": workers,
            "shared_prefix_groups": int(eng.groups.shape[1]) if shared else 0,
            "disjoint_blocks": eng.disjoint is not None,
            "timing": "gpu events per step, L2/MALL flushed between steps" if args.flush else "wall clock",
        },
        "pct_of_peak": round(100.0 * value / PEAK_GBS, 2),
        "value_logical_gbs": round(tot_bytes_logical / elapsed / 1e9, 2),
        "kv_tokens_per_s": round(kv_tokens / elapsed, 1),
        "attention_pass1_us": round(p1_avg_s * 1e6, 2),
        "attention_pass1_us_p10_p50_p90": [round(float(x) * 1e3, 2) for x in np.percentile(p1_ms, [10, 50, 90])],
        "attention_pass1_launches_timed": len(p1_ms),
        "step_gpu_us": round(float(np.mean(step_ms)) * 1e3, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": kernel,
            "achieved_logical": round(achieved_logical, 2),
            # algorithmic bytes per launch (unique K/V), over the event-timed launches and over
            # every timed step (the average a kernel trace of the run compares with)
            "bytes_per_launch": int(np.mean(p1_bytes)),
            "bytes_per_launch_all_steps": int(np.mean([u[0] for u in uniq])),
        },
    }
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(workloads.make(args.config, max_steps=1, **fp8_kw), args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
