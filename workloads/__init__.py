"""Seeded synthetic workloads for the paged-KV decode path.

This module is the only code that both the CPU oracle (``oracle/``) and the
HIP library's tests and benchmark use. It holds shapes, random draws and the
scripts of block-manager operations, and nothing of the method's arithmetic:
no slot computation, no cache writes, no fp8 encoding, no attention.

Each workload is shaped like a model that the pages on paged KV caches use as
an example. Random draws come from NumPy's PCG64, one independent stream per
purpose, keyed by ``SeedSequence([seed, stream, index...])``, so any piece
(one operation's K/V rows, one step's queries) can be regenerated alone:

    stream 0  sequence lengths
    stream 1  initial free-block order (a permutation of the pool)
    stream 2  queries, one draw per decode step
    stream 3  K then V rows of one token-creating operation
    stream 4  prompt token ids
    stream 5  prefill query rows, one draw per sequence

K/V/Q values are float32 N(0, 1) draws rounded to float16.

A workload is a script: setup rounds, then decode steps. A round is a list of
operations applied to the block manager in order; the tokens that the round
creates are then written (after any copy-on-write block copies the round
produced). Each decode step appends one token to every sequence of the batch
and then runs attention for the batch. A prefill run instead attends, after
the setup, with one query row per position of each sequence's chunk: the
positions a prompt wrote past its cached blocks, or the last ``meta["chunk"][s]``
positions of a sequence built by plain allocation.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

STREAM_LENGTHS = 0
STREAM_PERM = 1
STREAM_Q = 2
STREAM_KV = 3
STREAM_TOKENS = 4
STREAM_PREFILL_Q = 5


def rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *key])))


@dataclass(frozen=True)
class Op:
    """One block-manager call.

    kind: "allocate" (seq, n tokens), "append" (seq, n tokens),
          "share_prefix" (src -> seq, n blocks), "fork" (src -> seq),
          "prompt" (seq, n = len(tokens): a new sequence through the prefix
          cache; only the tokens after the cached ones are written).
    key:  index of the op's K/V draw in stream 3 (allocate / append).
    tokens: a prompt's token ids.
    parts:  a prompt's K/V rows, in order, as (key in stream 3, rows) draws.
    Preemption ops ("Where Did the VRAM Go (KV cache tutorial)", §7.1-7.2):
          "swap_out" / "swap_in" (group = the sequences, in order),
          "preempt" (group = the running list, n = blocks needed,
          mode = "recompute" or "swap"), "free" (seq).
    """
    kind: str
    seq: int
    n: int = 0
    src: int = -1
    key: int = -1
    tokens: tuple = ()
    parts: tuple = ()
    group: tuple = ()
    mode: str = ""

    @property
    def creates_tokens(self) -> bool:
        return self.kind in ("allocate", "append") and self.n > 0


@dataclass
class Workload:
    name: str
    seed: int
    description: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    kv_dtype: str  # "f16", "fp8" (e4m3fn) or "fp8_e5m2"
    num_blocks: int
    free_order: np.ndarray  # int32 permutation of the pool
    batch: list  # sequence ids, in batch order
    setup_rounds: list  # list[list[Op]]
    max_steps: int  # decode steps the pool is sized for
    max_blocks_per_seq: int  # block-table width that fits max_steps steps
    k_scale: float = 1.0  # fp8 dequantisation scales (float32 values)
    v_scale: float = 1.0
    k_inv_scale: float = 1.0  # fp8 quantisation multipliers (float32 values)
    v_inv_scale: float = 1.0
    meta: dict = field(default_factory=dict)
    num_host_blocks: int = 0  # host pool for swapped-out sequences

    # ------------------------------------------------------------ derived
    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def step_ops(self, step: int) -> list:
        """Decode step `step` (0-based): append one token to every batch sequence."""
        if step >= self.max_steps:
            raise ValueError(f"workload sized for {self.max_steps} decode steps")
        base = 1_000_000 + step * len(self.batch)
        return [Op("append", s, 1, key=base + i) for i, s in enumerate(self.batch)]

    def queries(self, step: int) -> np.ndarray:
        g = rng(self.seed, STREAM_Q, step)
        B = len(self.batch)
        return g.standard_normal((B, self.num_q_heads, self.head_dim), dtype=np.float32).astype(np.float16)

    def prefill_queries(self, seq: int, n: int) -> np.ndarray:
        """Query rows [n, Hq, D] float16 of sequence `seq`'s prefill chunk."""
        g = rng(self.seed, STREAM_PREFILL_Q, seq)
        return g.standard_normal((n, self.num_q_heads, self.head_dim), dtype=np.float32).astype(np.float16)

    def chunk_lengths(self, cached: dict) -> list:
        """Query rows per batch sequence for a prefill run after the setup.

        cached: {seq: tokens found in the prefix cache} for prompt sequences,
        as the block manager reported them; such a sequence's chunk is the
        rest of its prompt. Other sequences take meta["chunk"][batch index]."""
        prompt_len = {o.seq: o.n for r in self.setup_rounds for o in r if o.kind == "prompt"}
        chunk = self.meta.get("chunk")
        out = []
        for i, s in enumerate(self.batch):
            if s in prompt_len:
                out.append(prompt_len[s] - int(cached[s]))
            elif chunk is not None:
                out.append(int(chunk[i]))
            else:
                raise ValueError(f"sequence {s} has no prefill chunk")
        return out

    def _draw(self, key: int, n: int):
        g = rng(self.seed, STREAM_KV, key)
        shape = (n, self.num_kv_heads, self.head_dim)
        k = g.standard_normal(shape, dtype=np.float32).astype(np.float16)
        v = g.standard_normal(shape, dtype=np.float32).astype(np.float16)
        return k, v

    def op_kv(self, op: Op):
        """(K, V) float16 [n, Hkv, D] for a token-creating op (a prompt: all its rows)."""
        if op.kind == "prompt":
            return self.prompt_kv(op, 0)
        return self._draw(op.key, op.n)

    def prompt_kv(self, op: Op, start: int):
        """(K, V) of a prompt's rows start..n-1 (the ones not found in the cache);
        draws that lie wholly before `start` are skipped."""
        hkv, d = self.num_kv_heads, self.head_dim
        ks, vs, pos = [], [], 0
        for key, rows in op.parts:
            if rows > 0 and pos + rows > start:
                k, v = self._draw(key, rows)
                lo = max(0, start - pos)
                ks.append(k[lo:])
                vs.append(v[lo:])
            pos += rows
        if not ks:
            z = np.zeros((0, hkv, d), dtype=np.float16)
            return z, z.copy()
        return np.concatenate(ks), np.concatenate(vs)

    def round_kv(self, ops, threads: int = 8):
        """Concatenated (K, V) of a round's token-creating ops, in op order."""
        ops = [o for o in ops if o.creates_tokens]
        hkv, d = self.num_kv_heads, self.head_dim
        if not ops:
            z = np.zeros((0, hkv, d), dtype=np.float16)
            return z, z.copy()
        total = sum(o.n for o in ops)
        K = np.empty((total, hkv, d), dtype=np.float16)
        V = np.empty((total, hkv, d), dtype=np.float16)
        offs = np.cumsum([0] + [o.n for o in ops])

        def fill(i):
            k, v = self.op_kv(ops[i])
            K[offs[i]:offs[i + 1]] = k
            V[offs[i]:offs[i + 1]] = v

        if threads > 1 and len(ops) > 1:
            with ThreadPoolExecutor(max_workers=threads) as ex:
                list(ex.map(fill, range(len(ops))))
        else:
            for i in range(len(ops)):
                fill(i)
        return K, V

    def summary(self) -> dict:
        out = {
            "workload": self.name,
            "batch": len(self.batch),
            "q_heads": self.num_q_heads,
            "kv_heads": self.num_kv_heads,
            "head_dim": self.head_dim,
            "block_size": self.block_size,
            "kv_dtype": self.kv_dtype,
            "num_blocks": self.num_blocks,
        }
        L = self.meta.get("lengths")
        if L:
            out.update(ctx_len_min=int(min(L)), ctx_len_max=int(max(L)),
                       ctx_len_mean=round(float(np.mean(L)), 1))
        out.update({k: v for k, v in self.meta.items() if not isinstance(v, (list, tuple))})
        return out


# ---------------------------------------------------------------- builders
def _ceil_div(a, b):
    return -(-a // b)


def _perm(seed, n):
    return rng(seed, STREAM_PERM).permutation(n).astype(np.int32)


FP8_MAX = {"fp8": 448.0, "fp8_e5m2": 57344.0}  # largest finite e4m3 / e5m2 value


def _fp8_scales(wl: Workload, steps: int, per_head: bool = False):
    """Scale = max|x| / (the format's largest value) over every K (resp. V)
    value the workload generates for its setup and first `steps` decode steps,
    in float32, for the whole tensor or for each KV head; the multiplier is
    float32(1) / scale."""
    hkv = wl.num_kv_heads
    kmax = np.zeros(hkv, dtype=np.float32)
    vmax = np.zeros(hkv, dtype=np.float32)
    ops = [o for r in wl.setup_rounds for o in r]
    for s in range(steps):
        ops += wl.step_ops(s)
    for o in ops:
        if o.creates_tokens or o.kind == "prompt":
            k, v = wl.op_kv(o)
            if len(k):
                kmax = np.maximum(kmax, np.abs(k.astype(np.float32)).max(axis=(0, 2)))
                vmax = np.maximum(vmax, np.abs(v.astype(np.float32)).max(axis=(0, 2)))
    fmax = np.float32(FP8_MAX[wl.kv_dtype])
    if per_head:
        ks, vs = kmax / fmax, vmax / fmax
        wl.k_scale, wl.v_scale = ks, vs
        wl.k_inv_scale, wl.v_inv_scale = np.float32(1.0) / ks, np.float32(1.0) / vs
    else:
        ks = np.float32(kmax.max()) / fmax
        vs = np.float32(vmax.max()) / fmax
        wl.k_scale, wl.v_scale = float(ks), float(vs)
        wl.k_inv_scale = float(np.float32(1.0) / ks)
        wl.v_inv_scale = float(np.float32(1.0) / vs)


def tiny(max_steps: int = 2) -> Workload:
    """4 sequences of lengths 37, 100, 16, 250 (attended at the first step);
    8 query heads = 8 KV heads, head_dim 64, block size 16, a 64-block pool in a
    seeded random order. Each sequence holds L-1 tokens before the first
    decode step, so step 0 writes position L-1 and attends L tokens, and step 1
    writes position L (the length-16 sequence crosses into a second block)."""
    seed = 1
    lengths = [37, 100, 16, 250]
    nb = 64
    setup = [[Op("allocate", s, L - 1, key=s) for s, L in enumerate(lengths)]]
    return Workload(
        name="tiny_paged_decode", seed=seed,
        description="4 seqs L={37,100,16,250}, 8/8 heads, D=64, bs=16, 64-block pool",
        num_q_heads=8, num_kv_heads=8, head_dim=64, block_size=16, kv_dtype="f16",
        num_blocks=nb, free_order=_perm(seed, nb), batch=list(range(4)),
        setup_rounds=setup, max_steps=max_steps,
        max_blocks_per_seq=_ceil_div(max(lengths) - 1 + max_steps, 16),
        meta={"lengths": lengths},
    )


def llama2_7b(max_steps: int = 128, batch: int = 64) -> Workload:
    """Llama-2-7B-shaped single layer: 32 query heads = 32 KV heads, head_dim
    128, block size 16, batch 64, attended lengths uniform on [128, 2048];
    pool = 1.1 x the blocks the batch needs through max_steps decode steps,
    in a seeded random order."""
    seed = 2
    bs = 16
    L = rng(seed, STREAM_LENGTHS).integers(128, 2048, size=batch, endpoint=True).tolist()
    need = sum(_ceil_div(l + max_steps, bs) for l in L)
    nb = math.ceil(1.1 * need)
    setup = [[Op("allocate", s, l - 1, key=s) for s, l in enumerate(L)]]
    return Workload(
        name="llama2_7b_decode_b64", seed=seed,
        description="Llama-2-7B-shaped layer: 32/32 heads, D=128, bs=16, batch 64, L~U[128,2048]",
        num_q_heads=32, num_kv_heads=32, head_dim=128, block_size=bs, kv_dtype="f16",
        num_blocks=nb, free_order=_perm(seed, nb), batch=list(range(batch)),
        setup_rounds=setup, max_steps=max_steps,
        max_blocks_per_seq=_ceil_div(max(L) - 1 + max_steps, bs),
        meta={"lengths": L},
    )


def qwen3_prefix(max_steps: int = 32, batch: int = 256) -> Workload:
    """Qwen3-0.6B-shaped grouped-query layer: 16 query heads over 8 KV heads,
    head_dim 128, block size 16, batch 256. Sequence 0 holds a 1024-token
    system-prompt prefix (64 blocks); sequences 1..255 share it through
    share_prefix (refcount 256); every sequence then appends a suffix of
    uniform length in [16, 3072] tokens (the last suffix token is written by
    the first decode step)."""
    seed = 3
    bs = 16
    prefix = 1024
    pblocks = prefix // bs
    suffix = rng(seed, STREAM_LENGTHS).integers(16, 3072, size=batch, endpoint=True).tolist()
    need = pblocks + sum(_ceil_div(s + max_steps, bs) for s in suffix)
    nb = math.ceil(1.1 * need)
    r0 = [Op("allocate", 0, prefix, key=0)]
    r1 = [Op("share_prefix", s, pblocks, src=0) for s in range(1, batch)]
    r2 = [Op("append", s, suffix[s] - 1, key=1 + s) for s in range(batch) if suffix[s] > 1]
    lengths = [prefix + s for s in suffix]
    return Workload(
        name="qwen3_0p6b_gqa_prefix_b256", seed=seed,
        description="Qwen3-0.6B-shaped GQA 16/8 heads, D=128, bs=16, batch 256, "
                    "shared 1024-token prefix + suffix~U[16,3072]",
        num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=bs, kv_dtype="f16",
        num_blocks=nb, free_order=_perm(seed, nb), batch=list(range(batch)),
        setup_rounds=[r0, r1, r2], max_steps=max_steps,
        max_blocks_per_seq=_ceil_div(max(lengths) - 1 + max_steps, bs),
        meta={"lengths": lengths, "prefix_tokens": prefix},
    )


def qwen3_prefix_cached(max_steps: int = 32, batch: int = 256) -> Workload:
    """The Qwen3-0.6B shared-prefix workload with its sharing found by the
    prefix cache instead of scripted: every sequence arrives as one prompt of
    token ids (the same 1024-token system prompt, then its own suffix) and is
    allocated through the block manager's prefix cache ("Where Did the VRAM Go
    (KV cache tutorial)", §4.2). K/V rows of each logical position are the same
    draws as in the scripted workload, so attention outputs must be identical."""
    base = qwen3_prefix(max_steps=max_steps, batch=batch)
    prefix = base.meta["prefix_tokens"]
    lengths = base.meta["lengths"]
    g = rng(base.seed, STREAM_TOKENS, 0)
    sys_prompt = g.integers(0, 50_000, size=prefix).tolist()
    ops = []
    for s in range(batch):
        suffix = lengths[s] - prefix - 1          # the last token is written by the first decode step
        toks = sys_prompt + rng(base.seed, STREAM_TOKENS, 1 + s).integers(0, 50_000, size=suffix).tolist()
        ops.append(Op("prompt", s, len(toks), tokens=tuple(toks), parts=((0, prefix), (1 + s, suffix))))
    base.name = "qwen3_0p6b_gqa_prefix_cached_b256"
    base.description = base.description + ", sharing found by the prefix cache"
    base.setup_rounds = [ops]
    return base


def prefill_tiny() -> Workload:
    """Prefill through the prefix cache at the tiny decode shape: 8 query
    heads = 8 KV heads, head_dim 64, block size 16, a 64-block pool in a seeded
    order. Four prompts of 37, 100, 16 and 250 tokens; prompts 0, 1 and 3 open
    with the same 32-token system prompt (two full blocks), so prompt 0 misses
    and prompts 1 and 3 find both blocks; prompt 2 is 16 tokens of its own.
    Each prompt's chunk is what it did not find: 37, 68, 16 and 218 rows."""
    seed = 6
    lengths = [37, 100, 16, 250]
    common = 32
    sys_prompt = rng(seed, STREAM_TOKENS, 0).integers(0, 50_000, size=common).tolist()
    ops = []
    for s, L in enumerate(lengths):
        if L >= common and s != 2:
            own = rng(seed, STREAM_TOKENS, 1 + s).integers(0, 50_000, size=L - common).tolist()
            toks, parts = sys_prompt + own, ((0, common), (1 + s, L - common))
        else:
            toks, parts = rng(seed, STREAM_TOKENS, 1 + s).integers(0, 50_000, size=L).tolist(), ((1 + s, L),)
        ops.append(Op("prompt", s, L, tokens=tuple(toks), parts=parts))
    nb = 64
    return Workload(
        name="tiny_prefill_prefix_cache", seed=seed,
        description="4 prompts L={37,100,16,250} (3 share a 32-token system prompt), 8/8 heads, D=64, "
                    "bs=16, 64-block pool",
        num_q_heads=8, num_kv_heads=8, head_dim=64, block_size=16, kv_dtype="f16",
        num_blocks=nb, free_order=_perm(seed, nb), batch=list(range(4)),
        setup_rounds=[ops], max_steps=0, max_blocks_per_seq=_ceil_div(max(lengths), 16),
        meta={"lengths": lengths},
    )


def qwen3_prefill(batch: int = 256) -> Workload:
    """Prefill of the Qwen3-0.6B-shaped shared-prefix workload through the
    prefix cache: 16 query heads over 8 KV heads, head_dim 128, block size
    16; every prompt is the same 1024-token system prompt plus its own suffix
    (uniform [16, 3072] tokens, less the one a decode step would add). Prompt
    0 misses and prefills all of its tokens; the other 255 find the 64 system
    prompt blocks and prefill only their suffix ("Where Did the VRAM Go (KV
    cache tutorial)", §4.2, §5)."""
    wl = qwen3_prefix_cached(max_steps=0, batch=batch)
    wl.name = "qwen3_0p6b_gqa_prefill_prefix_cache_b256" if batch == 256 else f"qwen3_prefill_b{batch}"
    wl.description = ("Qwen3-0.6B-shaped GQA 16/8 heads, D=128, bs=16: prefill of 256 prompts = shared "
                      "1024-token system prompt (cached after the first) + suffix~U[16,3072]")
    wl.meta = dict(wl.meta, lengths=[L - 1 for L in wl.meta["lengths"]])
    return wl


def llama2_7b_chunked(batch: int = 64, chunk: int = 512) -> Workload:
    """Chunked prefill at the Llama-2-7B decode shape: 32 query heads = 32
    KV heads, head_dim 128, block size 16, batch 64 with context lengths
    uniform on [128, 2048] (the same draws as the decode workload); each
    sequence's last min(L, 512) positions are one prefill chunk that attends
    the earlier positions and itself. Chunk boundaries fall inside blocks."""
    base = llama2_7b(max_steps=1, batch=batch)
    L = base.meta["lengths"]
    setup = [[Op("allocate", s, l, key=s) for s, l in enumerate(L)]]
    base.name = f"llama2_7b_chunked_prefill_b{batch}_c{chunk}"
    base.description = f"Llama-2-7B-shaped layer, batch {batch}, L~U[128,2048], last {chunk}-token chunk prefilled"
    base.setup_rounds = setup
    base.max_steps = 0
    base.max_blocks_per_seq = _ceil_div(max(L), 16)
    base.meta = dict(base.meta, chunk=[min(l, chunk) for l in L])
    return base


def llama2_7b_preempt(mode: str = "swap", max_steps: int = 2, batch: int = 64, victims: int = 16) -> Workload:
    """The Llama-2-7B batch-64 decode workload with preemption ("Where Did the
    VRAM Go (KV cache tutorial)", §7.1-7.2; "From OOM to Smooth Inference", §5).
    After the batch is prefilled, a burst of `victims` new requests needs the
    blocks of the newest `victims` running sequences: they are preempted from
    the tail of the running set (mode "swap": copied to a host pool; mode
    "recompute": dropped). The burst's requests are written, run and finish;
    the preempted sequences then come back (swapped in, or allocated and
    prefilled again from the same K/V draws), and the whole batch decodes.
    Its K/V are then exactly those of the plain workload, so the decode
    outputs must be too."""
    base = llama2_7b(max_steps=max_steps, batch=batch)
    L = base.meta["lengths"]
    bs = base.block_size
    nb = base.num_blocks
    held = [_ceil_div(l - 1, bs) for l in L]
    tail = list(range(batch - victims, batch))
    need = nb - sum(held) + sum(held[s] for s in tail)  # every block the tail holds, plus the free ones
    burst = [batch + i for i in range(victims)]
    r0 = [Op("allocate", s, L[s] - 1, key=s) for s in range(batch)]
    r1 = [Op("preempt", -1, need, group=tuple(range(batch)), mode=mode)]
    r2 = [Op("allocate", b, held[t] * bs, key=10_000 + b) for b, t in zip(burst, tail)]
    r3 = [Op("free", b) for b in burst]
    if mode == "swap":
        r4 = [Op("swap_in", -1, group=tuple(tail))]
    else:
        r4 = [Op("allocate", s, L[s] - 1, key=s) for s in tail]
    base.name = f"llama2_7b_decode_b{batch}_preempt_{mode}"
    base.description = (f"Llama-2-7B-shaped decode, batch {batch}: the newest {victims} sequences preempted "
                        f"({mode}) for a burst of {victims} requests, then resumed")
    base.setup_rounds = [r0, r1, r2, r3, r4]
    base.num_host_blocks = sum(held[s] for s in tail) if mode == "swap" else 0
    base.meta = dict(base.meta, preempted=tail, mode=mode)
    return base


def opt13b_rag(max_steps: int = 32, batch: int = 128) -> Workload:
    """OPT-13B-shaped RAG decode: 40 query heads = 40 KV heads, head_dim 128,
    block size 32, batch 128, attended lengths round(N(3000, 400)) clipped to
    [1024, 4096]; each decode step writes one token per sequence through its
    slot and appends a block when the last one is full."""
    seed = 4
    bs = 32
    g = rng(seed, STREAM_LENGTHS)
    L = np.clip(np.rint(g.normal(3000.0, 400.0, size=batch)), 1024, 4096).astype(int).tolist()
    need = sum(_ceil_div(l + max_steps, bs) for l in L)
    nb = math.ceil(1.1 * need)
    setup = [[Op("allocate", s, l - 1, key=s) for s, l in enumerate(L)]]
    return Workload(
        name="opt13b_rag_decode_b128", seed=seed,
        description="OPT-13B-shaped layer: 40/40 heads, D=128, bs=32, batch 128, L~N(3000,400) in [1024,4096]",
        num_q_heads=40, num_kv_heads=40, head_dim=128, block_size=bs, kv_dtype="f16",
        num_blocks=nb, free_order=_perm(seed, nb), batch=list(range(batch)),
        setup_rounds=setup, max_steps=max_steps,
        max_blocks_per_seq=_ceil_div(max(L) - 1 + max_steps, bs),
        meta={"lengths": L},
    )


def beam_fp8(max_steps: int = 8, prompts: int = 32, beams: int = 4, tail_max: int = 128,
             kv_dtype: str = "fp8", per_head: bool = False) -> Workload:
    """Beam / parallel-sampling decode with an fp8 e4m3 KV cache: 64 query
    heads over 8 KV heads, head_dim 128, block size 64. 32 prompts of uniform
    length in [512, 2048] are allocated (beam 0 of each prompt holds it) and
    written in one call; each is forked to 3 more beams (refcount 4). Every beam
    then grows a private tail of uniform length in [1, 128] tokens, one token
    per beam per round in sequence order, so the first three beams to write
    into a partially filled shared prompt block copy it and the last one
    writes in place; the last tail token is written by the first decode step.
    K and V each use one float32 scale max|x|/448 over the data generated.
    tail_max = 1 makes every tail a single token, so all copy-on-write happens
    inside the first decode step. kv_dtype "fp8_e5m2" stores e5m2 instead
    (scale max|x|/57344); per_head gives every KV head its own scale ("Where
    Did the VRAM Go (KV cache tutorial)", §6.2-6.3)."""
    seed = 5
    bs = 64
    g = rng(seed, STREAM_LENGTHS)
    P = g.integers(512, 2048, size=prompts, endpoint=True).tolist()
    T = g.integers(1, tail_max, size=(prompts, beams), endpoint=True).tolist()
    seq = lambda i, b: i * beams + b  # noqa: E731
    r0 = [Op("allocate", seq(i, 0), P[i], key=i) for i in range(prompts)]
    r1 = [Op("fork", seq(i, b), src=seq(i, 0)) for i in range(prompts) for b in range(1, beams)]
    rounds = [r0, r1]
    key = prompts
    max_tail = max(max(t) for t in T)
    for r in range(max_tail - 1):
        ops = []
        for i in range(prompts):
            for b in range(beams):
                if T[i][b] - 1 > r:
                    ops.append(Op("append", seq(i, b), 1, key=key))
                    key += 1
        if ops:
            rounds.append(ops)
    need = 0
    for i in range(prompts):
        full = P[i] // bs
        need += full + sum(_ceil_div(P[i] + T[i][b] + max_steps, bs) - full for b in range(beams))
    nb = math.ceil(1.1 * need)
    lengths = [P[i] + T[i][b] for i in range(prompts) for b in range(beams)]
    fmt = "e4m3" if kv_dtype == "fp8" else "e5m2"
    gran = "per-head" if per_head else "per-tensor"
    suffix = ("" if kv_dtype == "fp8" else "_e5m2") + ("_perhead" if per_head else "")
    wl = Workload(
        name="beam4_fp8_gqa64x8" + suffix, seed=seed,
        description=f"32 prompts x beam 4, fp8 {fmt} KV ({gran} scale), 64/8 heads, D=128, bs=64, "
                    "prompt~U[512,2048], tails~U[1,128] with copy-on-write",
        num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=bs, kv_dtype=kv_dtype,
        num_blocks=nb, free_order=_perm(seed, nb), batch=list(range(prompts * beams)),
        setup_rounds=rounds, max_steps=max_steps,
        max_blocks_per_seq=_ceil_div(max(lengths) - 1 + max_steps, bs),
        meta={"lengths": lengths, "prompts": P, "tails": T},
    )
    _fp8_scales(wl, max_steps, per_head)
    return wl


CONFIGS = {
    1: tiny,
    2: llama2_7b,
    3: qwen3_prefix,
    4: opt13b_rag,
    5: beam_fp8,
}


def make(config: int, **kw) -> Workload:
    return CONFIGS[config](**kw)


def small_prefill(seed: int, lengths, chunks, num_q_heads, num_kv_heads, head_dim, block_size,
                  kv_dtype="f16", slack=1.25, per_head=False) -> Workload:
    """Independent sequences of the given context lengths, each holding all
    its tokens, whose last chunks[s] positions are prefilled (edge cases:
    chunks of one row, whole-sequence chunks, chunk edges inside blocks)."""
    L = list(lengths)
    need = sum(_ceil_div(l, block_size) for l in L)
    nb = max(1, math.ceil(slack * need))
    setup = [[Op("allocate", s, l, key=s) for s, l in enumerate(L)]]
    wl = Workload(
        name=f"prefill_{seed}", seed=seed, description="prefill edge-case workload",
        num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        block_size=block_size, kv_dtype=kv_dtype, num_blocks=nb, free_order=_perm(seed, nb),
        batch=list(range(len(L))), setup_rounds=setup, max_steps=0,
        max_blocks_per_seq=max(1, _ceil_div(max(L + [1]), block_size)),
        meta={"lengths": L, "chunk": list(chunks)},
    )
    if kv_dtype != "f16":
        _fp8_scales(wl, 0, per_head)
    return wl


def small_forks(seed: int, prompts, members, tails, singles, num_q_heads, num_kv_heads, head_dim,
                block_size, kv_dtype="f16", max_steps=1, per_head=False) -> Workload:
    """Prompts forked into several members that then grow private tails
    (appended one token per member per round, so the first members to write
    into a shared partial block copy it), with independent sequences between
    the groups in the batch: prompt i has members[i] sequences, tails[i] their
    tail lengths, and singles[i] independent sequences follow its group."""
    bs = block_size
    ops0, ops1, batch, lengths = [], [], [], []
    nxt, key = 0, 0
    groups = []
    for i, P in enumerate(prompts):
        ids = list(range(nxt, nxt + members[i]))
        nxt += members[i]
        ops0.append(Op("allocate", ids[0], P, key=key))
        key += 1
        ops1 += [Op("fork", c, src=ids[0]) for c in ids[1:]]
        groups.append(ids)
        batch += ids
        lengths += [P + t + 1 for t in tails[i]]
        for _ in range(singles[i]):
            L = 16 * (i + 1) + 7 * len(batch) + 1
            ops0.append(Op("allocate", nxt, L, key=key))
            key += 1
            batch.append(nxt)
            lengths.append(L + 1)
            nxt += 1
    rounds = [ops0, ops1]
    for r in range(max(max(t) for t in tails)):
        ops = []
        for i, ids in enumerate(groups):
            for m, s_ in enumerate(ids):
                if tails[i][m] > r:
                    ops.append(Op("append", s_, 1, key=key))
                    key += 1
        if ops:
            rounds.append(ops)
    need = sum(_ceil_div(L + max_steps, bs) for L in lengths)
    nb = max(1, math.ceil(1.25 * need))
    wl = Workload(
        name=f"forks_{seed}", seed=seed, description="forked prompts with private tails",
        num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=bs,
        kv_dtype=kv_dtype, num_blocks=nb, free_order=_perm(seed, nb), batch=batch, setup_rounds=rounds,
        max_steps=max_steps, max_blocks_per_seq=_ceil_div(max(lengths) - 1 + max_steps, bs),
        meta={"lengths": lengths},
    )
    if kv_dtype != "f16":
        _fp8_scales(wl, max_steps, per_head)
    return wl


def small_custom(seed: int, lengths, num_q_heads, num_kv_heads, head_dim, block_size,
                 kv_dtype="f16", num_blocks=None, max_steps=1, slack=1.25, per_head=False) -> Workload:
    """A plain workload of independent sequences for edge-case tests."""
    L = list(lengths)
    need = sum(_ceil_div(max(l, 0) + max_steps, block_size) for l in L)
    nb = num_blocks if num_blocks is not None else max(1, math.ceil(slack * need))
    setup = [[Op("allocate", s, max(l - 1, 0), key=s) for s, l in enumerate(L)]]
    wl = Workload(
        name=f"custom_{seed}", seed=seed, description="edge-case workload",
        num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        block_size=block_size, kv_dtype=kv_dtype, num_blocks=nb, free_order=_perm(seed, nb),
        batch=list(range(len(L))), setup_rounds=setup, max_steps=max_steps,
        max_blocks_per_seq=max(1, _ceil_div(max(L + [1]) - 1 + max_steps, block_size)),
        meta={"lengths": L},
    )
    if kv_dtype != "f16":
        _fp8_scales(wl, max_steps, per_head)
    return wl
