/*
 * pagedkv.h -- C ABI of libpagedkv.so: paged KV cache decode path for
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages on paged KV caches / PagedAttention):
 *   [OOM]    "From OOM to Smooth Inference (RAG memory management)"
 *   [ENGINE] "Inference Engine Memory Optimisation (KV Cache to Continuous Batching)"
 *   [VRAM]   "Where Did the VRAM Go (KV cache tutorial)"
 *   [VLLM]   "vLLM Architecture and Memory Use, ch. 3"
 *
 * Conventions shared by every call
 *   - KV cache layout, for K and for V alike: [num_blocks][num_kv_heads]
 *     [block_size][head_dim], contiguous, element type fp16, OCP fp8 e4m3fn or
 *     OCP fp8 e5m2 (one byte; [VRAM] §6.2). An fp8 cache has its scales one
 *     per tensor (the float arguments) or one per KV head (the *_scaled
 *     calls, [VRAM] §6.3: the granularity can go down to one per head). Physical block b, KV head h, offset o starts at element
 *     ((b * num_kv_heads + h) * block_size + o) * head_dim.
 *   - A slot is block * block_size + offset ([OOM] §2.1: logical block i of
 *     a sequence lives in physical block table[i]).
 *   - Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *   - Device pointers are owned by the caller and must stay valid until the
 *     work queued on `stream` has finished. `stream` is a hipStream_t passed
 *     as void* (NULL = the null stream). Kernels allocate nothing and return
 *     as soon as the work is queued.
 *   - Alignment: the kernels move K/V rows, queries, outputs, host-pool
 *     blocks and workspaces with 16-byte vector accesses, so every such
 *     pointer (k_new, v_new, k_cache, v_cache, k_host, v_host, q, out,
 *     workspace) must be 16-byte aligned; index and scale arrays must be
 *     aligned to their element size (8 bytes for int64 slot mappings, 4 for
 *     int32 tables, lengths, pairs, updates and groups, and float scales).
 *     A misaligned pointer makes the call PKV_ERR_INVALID before anything is
 *     queued. (hipMalloc and torch allocations are 256-byte aligned; a view
 *     that starts inside an allocation may not be.)
 *   - Every call returns a pkv_status. Argument errors are detected on the
 *     host before anything is queued and leave all state unchanged.
 *   - Out-of-range indices that only the device can see (a slot, a block
 *     id in a table or a copy pair) are skipped rather than followed, so a
 *     bad index never reads or writes outside the buffers given.
 *   - head_dim is 64 or 128; block_size is 16, 32 or 64 (bs is a multiple of
 *     16); num_q_heads is num_kv_heads times 1, 2, 4 or 8.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID = -1, /* bad argument or shape; nothing done            */
  PKV_ERR_OOM = -2,     /* block pool exhausted; nothing done            */
  PKV_ERR_NO_SEQ = -3,  /* unknown sequence id; nothing done             */
  PKV_ERR_EXISTS = -4,  /* sequence id already live; nothing done        */
  PKV_ERR_HIP = -5      /* the HIP runtime refused a launch              */
} pkv_status;

typedef enum { PKV_KV_F16 = 0, PKV_KV_FP8_E4M3 = 1, PKV_KV_FP8_E5M2 = 2 } pkv_kv_dtype;

typedef enum { PKV_SWAP_OUT = 0, PKV_SWAP_IN = 1 } pkv_swap_dir;

typedef enum { PKV_PREEMPT_RECOMPUTE = 0, PKV_PREEMPT_SWAP = 1 } pkv_preempt_mode;

/* Human-readable name of a status code (static string). */
const char* pkv_status_str(int status);

/* ======================================================================
 * Device kernels
 * ==================================================================== */

/*
 * paged_kv_write -- scatter new K/V rows into their paged slots.
 * [OOM] §2.3 (allocation and append map each new token to a slot of a
 * physical block); [VRAM] §6.1-6.2 (fp8 storage with a scale).
 *
 *   k_new, v_new   device, fp16 [num_tokens][num_kv_heads][head_dim]
 *   k_cache/v_cache device, cache layout above, dtype kv_dtype
 *   slot_mapping   device, int64 [num_tokens]; -1 = skip this token.
 *                  Slots outside [0, num_blocks*block_size) are skipped.
 *   kv_dtype       PKV_KV_F16: the fp16 bits are copied unchanged.
 *                  PKV_KV_FP8_E4M3: byte = e4m3(float32(x) * inv_scale),
 *                  rounded to nearest even, saturated to +-448.
 *                  PKV_KV_FP8_E5M2: byte = e5m2(float32(x) * inv_scale),
 *                  rounded to nearest even, saturated to +-57344.
 *   k/v_inv_scale  fp8 only: multiplier applied before encoding (1/scale).
 * Two valid tokens must not share a slot (the later write would race).
 */
int paged_kv_write(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                   const int64_t* slot_mapping, int num_tokens, int num_blocks,
                   int num_kv_heads, int head_dim, int block_size, int kv_dtype,
                   float k_inv_scale, float v_inv_scale, void* stream);

/* paged_kv_write with one multiplier per KV head: k_inv_scales and
 * v_inv_scales are device float arrays of num_kv_heads entries (head h's rows
 * are encoded as fp8(float32(x) * inv_scales[h])); they may be NULL for an
 * fp16 cache, INVALID otherwise. [VRAM] §6.3. */
int paged_kv_write_scaled(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                          const int64_t* slot_mapping, int num_tokens, int num_blocks,
                          int num_kv_heads, int head_dim, int block_size, int kv_dtype,
                          const float* k_inv_scales, const float* v_inv_scales, void* stream);

/*
 * paged_kv_write_step -- paged_kv_write and paged_step_metadata in one
 * launch, for a decode step: writes the new tokens exactly as paged_kv_write
 * and, in the same kernel, copies ctx_src[n_ctx] -> ctx_dst and writes each
 * block-table update (row, logical index, block) into
 * block_tables[row * max_blocks + index] (updates outside [0, num_rows) x
 * [0, max_blocks) are skipped). slot_mapping, ctx_src and updates may be
 * pinned host memory read directly by the kernel. When all three are pinned
 * host memory (or empty), num_tokens, n_ctx and n_updates are each at most
 * 128, num_blocks * block_size fits in 31 bits and the stream is not being
 * captured, the call reads them itself and passes their values in the
 * launch's arguments, which saves the kernel a round trip over the bus; they
 * must then hold the step's values when the call is made. In every case they
 * must not change until the kernel has run. Work that reads ctx_dst or
 * block_tables must be queued after this call.
 */
int paged_kv_write_step(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                        const int64_t* slot_mapping, int num_tokens, int num_blocks,
                        int num_kv_heads, int head_dim, int block_size, int kv_dtype,
                        float k_inv_scale, float v_inv_scale, const int32_t* ctx_src,
                        int32_t* ctx_dst, int n_ctx, const int32_t* updates, int n_updates,
                        int32_t* block_tables, int num_rows, int max_blocks, void* stream);

/* paged_kv_write_step with per-KV-head multipliers (device arrays, as in
 * paged_kv_write_scaled). */
int paged_kv_write_step_scaled(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                               const int64_t* slot_mapping, int num_tokens, int num_blocks,
                               int num_kv_heads, int head_dim, int block_size, int kv_dtype,
                               const float* k_inv_scales, const float* v_inv_scales, const int32_t* ctx_src,
                               int32_t* ctx_dst, int n_ctx, const int32_t* updates, int n_updates,
                               int32_t* block_tables, int num_rows, int max_blocks, void* stream);

/*
 * paged_block_copy -- whole-block copy for copy-on-write.
 * [VLLM] §3.3 (a write into a shared block first copies it to a new block);
 * [OOM] §6.1 (forked beams copy only their last block).
 *
 *   pairs        int32 [num_pairs][2] = (src block, dst block), device memory
 *                or pinned host memory; ids outside [0, num_blocks) are skipped.
 *   block_bytes  bytes of one block of one cache
 *                (= num_kv_heads * block_size * head_dim * element size);
 *                must be a multiple of 16. K and V are both copied.
 * No dst may equal another pair's src or dst (copy-on-write destinations
 * are fresh blocks, so this always holds for the block manager's pairs).
 */
int paged_block_copy(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs,
                     int num_blocks, size_t block_bytes, void* stream);

/*
 * paged_block_swap -- whole-block copies between the device caches and a host
 * pool of the same layout, for preemption by swapping: a preempted request's
 * blocks are copied to CPU memory and back ([VRAM] §7.1-7.2; [OOM] §5 swap
 * versus recompute; [VLLM] §3.4 swap space). Pairs come from
 * pkv_bm_swap_out / pkv_bm_swap_in / pkv_bm_preempt_tail.
 *
 *   k_cache/v_cache device caches [num_blocks][Hkv][bs][D]
 *   k_host/v_host   pinned host memory (hipHostMalloc) of the same layout,
 *                   [num_host_blocks][Hkv][bs][D], read or written by the
 *                   kernel directly over the bus
 *   pairs           int32 [num_pairs][2], device or pinned host memory:
 *                   PKV_SWAP_OUT: (device block, host block), host <- device;
 *                   PKV_SWAP_IN:  (host block, device block), device <- host.
 *                   A pair with an id out of range is skipped.
 *   block_bytes     bytes of one block of one cache, a multiple of 16.
 * No destination may appear twice. Copies are ordered on `stream` like any
 * kernel: queue a swap-out before anything that writes the released device
 * blocks, and a swap-in before anything that reads the sequences.
 */
int paged_block_swap(void* k_cache, void* v_cache, void* k_host, void* v_host, const int32_t* pairs,
                     int num_pairs, int num_blocks, int num_host_blocks, size_t block_bytes, int direction,
                     void* stream);

/*
 * paged_attn_decode -- one query token per sequence attends over its paged
 * K/V: out[s][h] = sum_t softmax_t(sm_scale * q[s][h].K_t) V_t over the
 * ctx_lens[s] tokens reached through block_tables[s] ([OOM] §2.1-2.3,
 * [ENGINE] §2.2).
 * Split-sequence, stream-K style: the (sequence, KV head) segments are laid
 * end to end in units of 16 tokens (32 for 4 or 8 query heads per KV head)
 * and cut into equal contiguous shares, one per worker (a wave). Pass 1: each
 * worker runs an online softmax over its share; a segment it holds whole is
 * written to `out`, a segment split between workers leaves (max, sum,
 * output) partials (the output fp32 and unnormalised for 1 or 2 query heads
 * per KV head, fp16 and divided by the sum for 4 or 8). Pass 2 combines the partials of split
 * segments and writes zeros for sequences with ctx_len 0.
 *
 *   out            device, fp16 [num_seqs][num_q_heads][head_dim]
 *   q              device, fp16 [num_seqs][num_q_heads][head_dim]
 *   block_tables   device, int32 [num_seqs][max_blocks_per_seq]; entries past
 *                  ceil(ctx_len/block_size) are ignored (they may be read,
 *                  as every entry of the row must be readable, but their
 *                  values never matter); entries outside [0, num_blocks) are
 *                  never followed (their tokens are skipped).
 *   ctx_lens       device, int32 [num_seqs], tokens to attend (includes the
 *                  token written this step). Clamped to
 *                  [0, max_blocks_per_seq*block_size]; 0 gives a zero output.
 *   sm_scale       softmax scale (1/sqrt(head_dim) usually); any real value:
 *                  a negative scale is softmax of the negated logits, 0 the
 *                  plain average of V over the context (so is an fp8 K
 *                  multiplier of 0, e.g. for a head of zeros).
 *   k_scale/v_scale fp8 only: dequantisation multipliers (K = byte * k_scale);
 *                  kv_dtype PKV_KV_FP8_E4M3 or PKV_KV_FP8_E5M2 (both widened
 *                  to fp16 exactly before the arithmetic).
 *   partition_tokens 0 = one worker per SIMD of the device (fp16 KV with one
 *                  query head per KV head) or two (other shapes), within
 *                  what the device can hold at once, rounded down to a
 *                  multiple of num_kv_heads where that drops under 1/16 of
 *                  them and keeps whole workgroups of 4; else a multiple of 16:
 *                  each worker takes about this many tokens of the longest
 *                  possible batch (at most 8192 workers either way).
 *   workspace      device, >= paged_attn_decode_workspace_bytes(...) bytes
 *                  (partials and the unit prefix; contents on entry are
 *                  ignored). Calls that share a workspace must not overlap.
 * Shapes: head_dim 64 or 128; block_size 16, 32 or 64; num_q_heads a multiple
 * of num_kv_heads with 1, 2, 4 or 8 query heads per KV head. Batches of more
 * than 4096 sequences run as consecutive launches.
 * Results are deterministic: they depend only on the inputs, the shape and the
 * worker count, not on block placement.
 * Returns PKV_ERR_INVALID for a bad shape, null pointer or short workspace
 * (nothing is queued), PKV_ERR_HIP if a launch fails.
 */
size_t paged_attn_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                         int head_dim, int max_blocks_per_seq, int block_size,
                                         int partition_tokens);

int paged_attn_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int max_blocks_per_seq,
                      const int32_t* ctx_lens, int num_seqs, int num_q_heads,
                      int num_kv_heads, int head_dim, int block_size, int num_blocks,
                      float sm_scale, int kv_dtype, float k_scale, float v_scale,
                      int partition_tokens, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Same as paged_attn_decode, restricted to pass 1 (passes = 1), pass 2
 * (passes = 2) or both (passes = 3). Queuing pass 1 then pass 2 with the
 * same arguments is identical to paged_attn_decode for batches of up to 4096
 * sequences; it exists so that each pass can be timed on its own. */
int paged_attn_decode_passes(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, int max_blocks_per_seq,
                             const int32_t* ctx_lens, int num_seqs, int num_q_heads,
                             int num_kv_heads, int head_dim, int block_size, int num_blocks,
                             float sm_scale, int kv_dtype, float k_scale, float v_scale,
                             int partition_tokens, void* workspace, size_t workspace_bytes,
                             int passes, void* stream);

/* paged_attn_decode_passes with one dequantisation scale per KV head:
 * k_scales and v_scales are device float arrays of num_kv_heads entries (K of
 * head h = byte * k_scales[h]); they may be NULL for an fp16 cache, INVALID
 * otherwise. [VRAM] §6.3 (scales per attention head). */
int paged_attn_decode_scaled(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, int max_blocks_per_seq,
                             const int32_t* ctx_lens, int num_seqs, int num_q_heads,
                             int num_kv_heads, int head_dim, int block_size, int num_blocks,
                             float sm_scale, int kv_dtype, const float* k_scales, const float* v_scales,
                             int partition_tokens, void* workspace, size_t workspace_bytes,
                             int passes, void* stream);

/*
 * paged_attn_decode_noalloc -- paged_attn_decode without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * arguments, kernels and results as paged_attn_decode with the same
 * partition_tokens (bit for bit: the same workers and the same sums); the
 * pass-1 partials and unit prefix live instead in a device array of
 * PKV_DECODE_NOALLOC_SCRATCH_BYTES that the library holds on each device
 * for the life of the process, laid out for the workers actually launched:
 * W * 2 * G * (head_dim + 2) * 4 bytes plus (min(num_seqs, 4096) + 1) * 4,
 * each part rounded up to 256 (W = paged_attn_decode_workers(...)). With
 * partition_tokens = 0 every supported shape fits on a 256-CU MI355X (at
 * most 2048 workers: 17 MB for 8 query heads per KV head and head_dim 128);
 * a shape or
 * partition_tokens whose partials do not fit returns PKV_ERR_INVALID before
 * anything is queued. The call allocates nothing: its first use on a device
 * only looks up that device's copy of the array (PKV_ERR_HIP if the lookup
 * fails). Every call on a device shares its array, so calls that overlap on
 * one device (two streams, or two host threads) race and give wrong results;
 * queue them on one stream or serialise them. Nothing in the array needs to
 * start at zero.
 */
#define PKV_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

int paged_attn_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* ctx_lens, int num_seqs, int num_q_heads,
                              int num_kv_heads, int head_dim, int block_size, int num_blocks,
                              float sm_scale, int kv_dtype, float k_scale, float v_scale,
                              int partition_tokens, void* stream);

/*
 * pkv_time_next_pass1 -- measurement hook, for benchmarks and profilers. The
 * next pass-1 launch that the calling thread makes (through
 * paged_attn_decode, _passes, _scaled, _noalloc or paged_attn_decode_shared)
 * is launched with hipExtLaunchKernel and records start_event and stop_event
 * (hipEvent_t, created by the caller with timing enabled) as the start and
 * the stop of that kernel's own execution, so that
 * hipEventElapsedTime(start_event, stop_event) is the kernel's duration
 * alone, without the idle time that separate event records add to the
 * stream. The hook then disarms; both null disarms it as well. Exactly one
 * null: PKV_ERR_INVALID. It changes no result. A call that fails before its
 * pass-1 launch leaves the hook armed.
 */
int pkv_time_next_pass1(void* start_event, void* stop_event);

/* The number of workers (waves) pass 1 uses for this shape on the current
 * device (for one launch of up to 4096 sequences), or a negative status for an
 * invalid shape or a failed device query. */
int paged_attn_decode_workers(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                              int block_size, int max_blocks_per_seq, int kv_dtype,
                              int partition_tokens);

/*
 * paged_attn_decode_shared -- paged_attn_decode for a batch in which runs of
 * consecutive sequences share their leading blocks: beams or parallel samples
 * forked from one prompt ([VLLM] §3.2) or requests mapped onto the same
 * prefix-cache blocks ([VRAM] §4.2-4.4). The output is the same attention as
 * paged_attn_decode's; only the order of the sums differs.
 * Group g is the sequences first[g] .. first[g] + size[g] - 1 of the batch.
 * Its shared tokens are the first prefix[g], rounded down to a multiple of
 * 16. One pass 1 launch covers the whole batch on the matrix cores: a group is
 * cut into parts of up to 32 query columns (members x query heads of a KV
 * head); a part reads the shared tokens once for all its columns, through the
 * table of its first member (and no more of them than that member's ctx_len,
 * rounded down to 16), then each member's remaining tokens through that
 * member's own table; a sequence in no group is a part of its own. A merge pass combines the parts
 * that were split between workers (exact up to rounding: the softmax of a
 * concatenation is the weighted merge of the softmaxes of its parts).
 *   group_first, group_size, group_prefix  device, int32 [num_groups]
 *                  (pkv_bm_prefix_groups computes them). Precondition: groups
 *                  ascending and disjoint, and every member maps its first
 *                  prefix[g] tokens (as far as its ctx_len reaches) to the
 *                  same physical blocks as the group's first sequence. A member with fewer tokens than that
 *                  attends only to its own ctx_len of them. Entries that break
 *                  the precondition give wrong results but never an access
 *                  outside the buffers (members past the batch are dropped).
 *                  With num_groups = 0 the caller declares that no block is
 *                  held by two sequences of the batch: the call is
 *                  paged_attn_decode (the same shares and sums, the same
 *                  bits), with its waves ordered for disjoint blocks -- each
 *                  XCD reads all KV heads of a range of tiles, not a few heads
 *                  of every tile, when one XCD's heads of a block would be
 *                  under 32 KiB (faster for disjoint blocks; slower where
 *                  sequences do share blocks, which head-major order serves
 *                  through one L2, so the declaration is the caller's).
 *   k_scale, v_scale, k_scales, v_scales  fp8 only: per-tensor multipliers, or
 *                  one per KV head when k_scales and v_scales (device float
 *                  [num_kv_heads]) are both non-NULL.
 *   passes         bits 0 or 1: pass 1; bit 2: the merge. 7 = the whole call
 *                  (each pass can be queued on its own to be timed).
 *   workspace      device, >= paged_attn_decode_shared_workspace_bytes(...).
 * Other arguments, shapes and errors as paged_attn_decode; num_seqs at most
 * 4096, num_groups in [0, num_seqs].
 */
size_t paged_attn_decode_shared_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                                int head_dim);

int paged_attn_decode_shared(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, int max_blocks_per_seq,
                             const int32_t* ctx_lens, int num_seqs, int num_q_heads,
                             int num_kv_heads, int head_dim, int block_size, int num_blocks,
                             float sm_scale, int kv_dtype, float k_scale, float v_scale,
                             const float* k_scales, const float* v_scales, const int32_t* group_first,
                             const int32_t* group_size, const int32_t* group_prefix, int num_groups,
                             int partition_tokens, void* workspace, size_t workspace_bytes,
                             int passes, void* stream);

/*
 * paged_attn_prefill -- chunked (multi-token, causal) attention over the paged
 * K/V. A request that found its leading blocks in the prefix cache prefills
 * only the positions that missed ([VRAM] §4.2, §5); a prompt split into chunks
 * prefills chunk by chunk. Sequence s holds L = ctx_lens[s] tokens (including
 * the chunk, whose K/V must be in the cache already, e.g. by paged_kv_write);
 * its n = q_start[s+1] - q_start[s] query rows are the last n positions of
 * that context, and row i (position p = L - n + i) attends positions 0..p:
 *   out[r][h] = sum_{t<=p} softmax_t(sm_scale * q[r][h].K_t) V_t.
 * A row with p < 0 (a chunk longer than its context) is written as zeros.
 *
 *   out, q         device, fp16 [total_q][num_q_heads][head_dim]; rows of
 *                  sequence s at q_start[s] .. q_start[s+1]-1
 *   block_tables   device, int32 [num_seqs][max_blocks_per_seq], as in
 *                  paged_attn_decode (entries past ceil(L/bs) ignored,
 *                  ids outside [0, num_blocks) never followed: their tokens
 *                  are skipped)
 *   ctx_lens       device, int32 [num_seqs]; clamped to
 *                  [0, max_blocks_per_seq * block_size]
 *   q_start        device, int32 [num_seqs + 1], non-decreasing from 0 to
 *                  total_q; a sequence whose rows fall outside [0, total_q)
 *                  is skipped (its rows are not written)
 *   sm_scale, kv_dtype, k_scale, v_scale: as in paged_attn_decode.
 * No workspace: one workgroup computes 128 (query token, query head) pairs of
 * one KV head over every position they see, on the matrix cores. Batches of
 * more than 4096 sequences run as consecutive launches. Shapes as in
 * paged_attn_decode. Returns PKV_ERR_INVALID for a bad shape or null pointer
 * (nothing is queued), PKV_ERR_HIP if a launch fails.
 */
int paged_attn_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, int max_blocks_per_seq, const int32_t* ctx_lens,
                       const int32_t* q_start, int num_seqs, int total_q, int num_q_heads,
                       int num_kv_heads, int head_dim, int block_size, int num_blocks,
                       float sm_scale, int kv_dtype, float k_scale, float v_scale, void* stream);

/* paged_attn_prefill with one dequantisation scale per KV head (device
 * arrays, as in paged_attn_decode_scaled). */
int paged_attn_prefill_scaled(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, int max_blocks_per_seq, const int32_t* ctx_lens,
                              const int32_t* q_start, int num_seqs, int total_q, int num_q_heads,
                              int num_kv_heads, int head_dim, int block_size, int num_blocks,
                              float sm_scale, int kv_dtype, const float* k_scales, const float* v_scales,
                              void* stream);

/*
 * paged_step_metadata -- bring a decode step's metadata to the device.
 * Copies slot_mapping (int64, n_seqs), ctx_lens (int32, n_seqs) and the
 * copy-on-write pairs (int32, 2*n_cow) from src buffers into dst buffers and
 * writes each block-table update (row, logical index, block) -- as produced by
 * pkv_bm_decode_step -- into block_tables[row * max_blocks + index]
 * (updates outside [0, num_rows) x [0, max_blocks) are skipped). One small
 * kernel: the src pointers may be pinned host memory (hipHostMalloc), read
 * directly by the kernel, so no separate DMA copy is queued.
 */
int paged_step_metadata(const int64_t* slots_src, int64_t* slots_dst, const int32_t* ctx_src,
                        int32_t* ctx_dst, int n_seqs, const int32_t* cow_src, int32_t* cow_dst,
                        int n_cow, const int32_t* updates, int n_updates, int32_t* block_tables,
                        int num_rows, int max_blocks, void* stream);

/* ======================================================================
 * Host block manager
 * A FIFO pool of physical blocks, per-sequence block tables and token
 * counts, per-block reference counts ([OOM] §2.3; [ENGINE] §3;
 * [VLLM] §3.2-3.3), and a prefix cache of full blocks ([VRAM] §4.2-4.4).
 * Host memory only; not thread-safe per handle. Output arrays are copies
 * into caller buffers. A failing call changes no state.
 *
 * Prefix cache. A full block written through pkv_bm_allocate_prompt is keyed
 * by (parent block, its block_size token ids): the parent is the previous
 * block of the same prompt (-1 for the first), and its own key carries its
 * parent, so a key stands for the block's tokens and everything before them
 * and a match is exact (hashes only speed up the lookup). A cached block
 * whose refcount reaches 0 keeps its key on an evictable list until it is
 * reused by a hit or evicted. Fresh blocks come from the free queue first,
 * then from the oldest evictable block (its key is dropped). Sequences made
 * by the other calls are never cached; without pkv_bm_allocate_prompt the
 * manager behaves exactly as a plain FIFO pool.
 * ==================================================================== */

typedef struct pkv_bm pkv_bm;

typedef struct {
  int32_t total_blocks;
  int32_t free_blocks;    /* in the free queue                               */
  int32_t used_blocks;    /* referenced by live sequences: total - free - evictable */
  int32_t live_seqs;
  int64_t filled_slots;   /* token slots holding data, shared blocks once    */
  double utilization;     /* used / total ([ENGINE] §3 utilisation)          */
  double slot_utilization;/* filled_slots / (used * block_size), 0 if unused */
  int32_t evictable_blocks;    /* cached, refcount 0                         */
  int32_t cached_blocks;       /* holding a prefix-cache key                 */
  int64_t prefix_query_tokens; /* tokens passed to pkv_bm_allocate_prompt    */
  int64_t prefix_hit_tokens;   /* of those, found in the cache               */
  int32_t host_blocks;         /* host pool size (pkv_bm_set_host_blocks)    */
  int32_t host_free_blocks;    /* in the host pool's free queue              */
  int32_t swapped_seqs;        /* sequences swapped out to the host pool     */
} pkv_bm_stats_t;

/* New manager over blocks 0..num_blocks-1. free_order (host, may be NULL =
 * ascending) is the initial FIFO order and must be a permutation. */
int pkv_bm_create(int num_blocks, int block_size, const int32_t* free_order, pkv_bm** out);
void pkv_bm_destroy(pkv_bm* bm);

/* New sequence holding num_tokens (>= 0) tokens: pops ceil(n/bs) blocks from
 * the front of the pool. slots_out (host, may be NULL) receives the n slots.
 * EXISTS if seq is live, OOM if the pool is short. [ENGINE] §3, [OOM] §2.3. */
int pkv_bm_allocate(pkv_bm* bm, int64_t seq, int num_tokens, int64_t* slots_out);

/* New sequence for a prompt of n_tokens token ids (host), reusing cached
 * blocks ([VRAM] §4.2: a request maps the blocks it finds into its table and
 * prefills only the rest). The longest run of leading full blocks whose keys
 * are cached is mapped (refcount +1, evictable ones revived); the first miss
 * ends the match; the remaining blocks are fresh and every fresh full block
 * is registered under its parent. The partial last block is never cached.
 * *n_cached = tokens covered by the mapped blocks (a multiple of block_size);
 * slots_out (host, room for n_tokens entries) receives the slots of tokens
 * n_cached .. n_tokens-1, the ones whose K/V the caller must write.
 * EXISTS if seq is live; OOM (nothing changed) if the free queue plus the
 * evictable blocks not revived by this call are too few. */
int pkv_bm_allocate_prompt(pkv_bm* bm, int64_t seq, const int32_t* tokens, int n_tokens,
                           int* n_cached, int64_t* slots_out);

/* Append n_tokens (>= 0) to seq. If the first new position falls inside the
 * current last block and that block is shared (refcount > 1), a fresh block
 * replaces it in the table (copy-on-write, [VLLM] §3.3) and cow_src / cow_dst
 * receive the pair to copy (else -1/-1). New blocks are popped for the rest.
 * slots_out (may be NULL) receives the n slots. */
int pkv_bm_append(pkv_bm* bm, int64_t seq, int n_tokens, int64_t* slots_out,
                  int32_t* cow_src, int32_t* cow_dst);

/* Append one token to each of n_seqs sequences, in order (a decode step).
 * slot_mapping_out[n_seqs] gets each token's slot; cow_pairs_out[2*n_seqs]
 * gets the copy-on-write pairs in order, *n_cow their count. All or nothing:
 * on OOM/NO_SEQ no sequence is changed. Duplicate ids are INVALID. */
int pkv_bm_append_batch(pkv_bm* bm, const int64_t* seqs, int n_seqs, int64_t* slot_mapping_out,
                        int32_t* cow_pairs_out, int* n_cow);

/* A decode step's bookkeeping in one call: pkv_bm_append_batch, plus what a
 * device-resident copy of the batch's block tables needs to stay current.
 * updates_out[3*k .. 3*k+2] = (batch row, logical block index, physical
 * block) for every table entry the step added or replaced by copy-on-write
 * (at most one per sequence), *n_updates their count; ctx_lens_out[n_seqs]
 * gets the new token counts. Capacity of updates_out: 3*n_seqs. max_blocks
 * is the column count of the device tables: a sequence whose new token
 * would need a table entry at index >= max_blocks makes the call INVALID
 * before any state changes (max_blocks < 1 is INVALID too). */
int pkv_bm_decode_step(pkv_bm* bm, const int64_t* seqs, int n_seqs, int64_t* slot_mapping_out,
                       int32_t* cow_pairs_out, int* n_cow, int32_t* updates_out, int* n_updates,
                       int32_t* ctx_lens_out, int max_blocks);

/* child shares every block of parent (refcount +1 each) and its token
 * count: beams / parallel samples ([VLLM] §3.2). */
int pkv_bm_fork(pkv_bm* bm, int64_t parent, int64_t child);

/* dst's table is src's first n_blocks blocks (refcount +1 each); dst's token
 * count is min(n_blocks*bs, src's count). INVALID if n_blocks exceeds src's
 * table. [ENGINE] §3 share_prefix. */
int pkv_bm_share_prefix(pkv_bm* bm, int64_t src, int n_blocks, int64_t dst);

/* Release seq: refcount -1 on each block in table order; uncached blocks
 * reaching 0 go to the back of the pool, cached ones to the back of the
 * evictable list, deepest block first (so eviction, oldest first, always
 * takes a block's cached descendants before the block). [OOM] §2.3,
 * [ENGINE] §3, [VLLM] §3.2, [VRAM] §4.3-4.4. */
int pkv_bm_free(pkv_bm* bm, int64_t seq);

/* ----------------------------------------------------------------------
 * Preemption and swapping ([VRAM] §7.1-7.2: when no new KV block can be had,
 * running requests are preempted from the tail of the running set, newest
 * first; recompute drops their cache and prefills them again later, swap
 * copies their blocks to CPU memory and back; [OOM] §5; [VLLM] §3.4).
 * A swapped-out sequence is not resident: calls that need its blocks on the
 * device return NO_SEQ, its id stays taken (EXISTS) and pkv_bm_free releases
 * its host blocks. Prefix-cache keys do not travel with swapped data.
 * ---------------------------------------------------------------------- */

/* Host pool of num_host_blocks blocks, ids 0..n-1 in a FIFO queue. INVALID
 * while any sequence is swapped out. */
int pkv_bm_set_host_blocks(pkv_bm* bm, int num_host_blocks);

/* Swap a group of resident sequences out. Every distinct device block of the
 * group, in order of first appearance (sequences in the order given, tables
 * in order), takes one host block from the front of the host queue, and
 * pairs_out[2*i], pairs_out[2*i+1] = (device block, host block) for
 * paged_block_swap(PKV_SWAP_OUT); a block the group's sequences share is
 * copied once. Each sequence then releases its device blocks as pkv_bm_free
 * does (a block still held by a sequence outside the group stays resident).
 * cap = room for pairs in pairs_out (pairs, not ints). OOM (nothing changed)
 * if the host queue is too short; NO_SEQ if a sequence is not resident;
 * INVALID for a duplicate id or a short cap. */
int pkv_bm_swap_out(pkv_bm* bm, const int64_t* seqs, int n_seqs, int32_t* pairs_out, int cap, int* n_pairs);

/* Swap a group of swapped-out sequences back in: every distinct host block,
 * in order of first appearance, takes a fresh device block (the free queue,
 * then the oldest evictable cached block) and pairs_out gets (host block,
 * device block) for paged_block_swap(PKV_SWAP_IN); host blocks whose count
 * reaches 0 go to the back of the host queue. OOM (nothing changed) if too
 * few device blocks are available. */
int pkv_bm_swap_in(pkv_bm* bm, const int64_t* seqs, int n_seqs, int32_t* pairs_out, int cap, int* n_pairs);

/* Preempt from the tail of running[0..n_running) (index n_running-1 first)
 * until the blocks a new allocation can take (free + evictable) reach
 * blocks_needed, counting only the device blocks each victim would actually
 * release. victims_out (room for n_running ids) gets the victims in order,
 * *n_victims their count. PKV_PREEMPT_RECOMPUTE frees them (their requests
 * are prefilled again later); PKV_PREEMPT_SWAP swaps them out as one group
 * (pairs_out / cap / *n_pairs as in pkv_bm_swap_out). No victim if enough
 * blocks are available already. OOM (nothing changed) if every listed
 * sequence together does not release enough, or the host pool is too small;
 * on any error the outputs are unspecified and the state unchanged. */
int pkv_bm_preempt_tail(pkv_bm* bm, const int64_t* running, int n_running, int blocks_needed, int mode,
                        int64_t* victims_out, int* n_victims, int32_t* pairs_out, int cap, int* n_pairs);

/* A swapped-out sequence's host block table and token count. NO_SEQ if the
 * sequence is not swapped out. */
int pkv_bm_swapped_table(const pkv_bm* bm, int64_t seq, int32_t* out, int cap, int* n);
int pkv_bm_swapped_tokens(const pkv_bm* bm, int64_t seq, int* n);
/* The host pool's free queue (front first) and a host block's refcount. */
int pkv_bm_host_free_list(const pkv_bm* bm, int32_t* out, int cap, int* n);
int pkv_bm_host_refcount(const pkv_bm* bm, int32_t host_block, int* rc);

/* Queries. Arrays are host buffers of `cap` entries; *n gets the count. */
int pkv_bm_slots(const pkv_bm* bm, int64_t seq, int start, int n, int64_t* out);
int pkv_bm_block_table(const pkv_bm* bm, int64_t seq, int32_t* out, int cap, int* n);
int pkv_bm_num_tokens(const pkv_bm* bm, int64_t seq, int* n);
int pkv_bm_refcount(const pkv_bm* bm, int32_t block, int* rc);
int pkv_bm_free_list(const pkv_bm* bm, int32_t* out, int cap, int* n); /* FIFO order */
/* Evictable cached blocks, oldest (next to evict) first. */
int pkv_bm_evictable_list(const pkv_bm* bm, int32_t* out, int cap, int* n);
/* *cached = 1 and (*parent, tokens_out[block_size]) = the block's key if it is
 * cached, else *cached = 0. tokens_out (host) needs block_size entries. */
int pkv_bm_cache_entry(const pkv_bm* bm, int32_t block, int* cached, int32_t* parent,
                       int32_t* tokens_out);
int pkv_bm_num_free(const pkv_bm* bm);
int pkv_bm_stats(const pkv_bm* bm, pkv_bm_stats_t* out);

/* Decode-batch export: tables_out[n_seqs][max_blocks] (-1 padded) and
 * ctx_lens_out[n_seqs] for the listed sequences. INVALID if a table is
 * wider than max_blocks. */
int pkv_bm_export(const pkv_bm* bm, const int64_t* seqs, int n_seqs, int32_t* tables_out,
                  int max_blocks, int32_t* ctx_lens_out);

/* The groups paged_attn_decode_shared reads once: walking seqs in order, a
 * group is a maximal run of consecutive entries (at most max_members) whose
 * first table entry is one block every member holds in full (token count >=
 * block_size); its prefix is block_size times the number of leading table
 * positions at which every member holds the same block, in full. Runs of one
 * entry are not groups. Writes (first batch index, members, prefix tokens) of
 * each group in batch order and their number to *num_groups. Shared blocks
 * are never written (copy-on-write, [VLLM] §3.3), and an append only adds or
 * replaces blocks past the full ones, so the groups stay valid through decode
 * steps until a sequence of the batch is freed, forked or swapped.
 * NO_SEQ for a sequence that is not resident; INVALID if cap is too small. */
int pkv_bm_prefix_groups(const pkv_bm* bm, const int64_t* seqs, int n_seqs, int max_members,
                         int32_t* group_first, int32_t* group_size, int32_t* group_prefix, int cap,
                         int* num_groups);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
