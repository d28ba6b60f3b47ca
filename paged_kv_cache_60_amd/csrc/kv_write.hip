// paged_kv_write: scatter each new token's K and V rows into its paged slot.
//
// The slot of a token comes from the host block manager; slot = block *
// block_size + offset ("From OOM to Smooth Inference (RAG memory
// management)", §2.1 and §2.3). With an fp8 cache each value is stored as
// fp8(float32(x) * inv_scale) ("Where Did the VRAM Go (KV cache tutorial)",
// §6.1-6.3): e4m3 rounded to nearest even and saturated to +-448, or e5m2
// (one more exponent bit, one less mantissa bit) saturated to +-57344; the
// multiplier is one per tensor or one per KV head.
//
// One thread moves 8 consecutive elements of one (token, head) row: a 16-byte
// load of fp16 and a 16-byte (fp16) or 8-byte (fp8) store, so a wave covers
// whole rows with coalesced accesses on both sides.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/pagedkv.h"
#include "device_common.hpp"

namespace pkv {
namespace {

// Four fp8 bytes (value j in byte j) for four floats: round to nearest even,
// saturate (an infinite input too), keep the sign of zero, NaN -> 0x7F.
// gfx950's packed conversion (two floats per instruction, OCP e4m3fn or e5m2)
// rounds to nearest even but does not saturate -- past the largest finite
// value it gives NaN (e4m3) or infinity (e5m2) -- so the inputs are clamped to
// +-max first (a value between max and the next half step rounds to max
// either way), and its NaN code is replaced by 0x7F. Equal to the plain
// bit-pattern definition of both formats on every fp16 input at several
// scales (checked on the device against that definition and the oracle).
template <int FMT>
__device__ __forceinline__ uint32_t fp8x4_encode(float a, float b, float c, float d) {
  constexpr float kMax = FMT == kE4M3 ? 448.0f : 57344.0f;
  auto sat = [](float x) { return fminf(fmaxf(x, -kMax), kMax); };
  uint32_t w;
  if constexpr (FMT == kE4M3) {
    w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
    w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), (int)w, true);
  } else {
    w = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(sat(a), sat(b), 0, false);
    w = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(sat(c), sat(d), (int)w, true);
  }
  const uint32_t nan = (a != a ? 0x000000FFu : 0u) | (b != b ? 0x0000FF00u : 0u) | (c != c ? 0x00FF0000u : 0u) |
                       (d != d ? 0xFF000000u : 0u);
  return (w & ~nan) | (0x7F7F7F7Fu & nan);
}

// Step metadata applied by the write kernel of a decode step (see
// paged_kv_write_step): context lengths and changed block-table entries.
struct StepMeta {
  const int32_t* ctx_src;
  int32_t* ctx_dst;
  int n_ctx;
  const int32_t* updates;  // [n_updates][3] = (row, logical index, block)
  int n_updates;
  int32_t* tables;
  int rows;
  int max_blocks;
};

// A small decode step's slots, context lengths and table updates, copied
// from pinned host memory into the launch's own arguments: the kernel then
// reads them from the argument segment instead of across the bus. Slots
// outside [0, num_slots) are stored as -1 (skipped either way).
constexpr int kInlineRows = 128;
struct StepInline {
  int32_t slots[kInlineRows];
  int32_t ctx[kInlineRows];
  int32_t upd[3 * kInlineRows];
};
struct NoInline {};

// k_inv_h / v_inv_h: one multiplier per KV head (device memory), or null to
// use k_inv / v_inv for every head.
// One grid row (blockIdx.y) per KV head; along x, the threads take the
// head's 16-byte chunks (8 elements) token by token: chunk c of token t is
// i = t * cpr + c with cpr = head_dim / 8 a power of two, so the index math is
// shifts and masks (block_size is a power of two too). With META, grid row 0
// also copies item i of the context lengths and applies item i of the table
// updates. With META every load of an iteration (the slot, the K and V
// chunks, the metadata items; the slots and metadata may sit in host memory)
// is issued before the first store, so an iteration costs one round trip, not
// a chain of them. With INL = StepInline the slots and metadata come from
// `inl` (at most kInlineRows of each) and the pointers to them are unused.
template <int FMT, bool META, class INL = NoInline>
__global__ void __launch_bounds__(256)
kv_write_kernel(const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new,
                uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                const int64_t* __restrict__ slots, int64_t num_tokens, int cpr_log2, int num_kv_heads,
                int64_t num_slots, int bs_log2, float k_inv, float v_inv,
                const float* __restrict__ k_inv_h, const float* __restrict__ v_inv_h, StepMeta meta,
                INL inl) {
  constexpr bool kInline = std::is_same<INL, StepInline>::value;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int h = blockIdx.y;
  const int cpr = 1 << cpr_log2;
  const int64_t n = num_tokens << cpr_log2;  // this head's chunks
  const bool meta_row = META && h == 0;
  const int64_t n_meta = meta_row ? (meta.n_ctx > meta.n_updates ? meta.n_ctx : meta.n_updates) : 0;
  const int64_t n_all = n > n_meta ? n : n_meta;
  float kinv = k_inv, vinv = v_inv;
  if (FMT != kF16 && k_inv_h) {
    kinv = k_inv_h[h];
    vinv = v_inv_h[h];
  }
  for (int64_t i = gtid; i < n_all; i += stride) {
    // loads
    const bool do_ctx = meta_row && i < meta.n_ctx;
    const bool do_upd = meta_row && i < meta.n_updates;
    int ctx = 0, row = -1, idx = -1, blk = 0;
    if constexpr (kInline) {
      if (do_ctx) ctx = inl.ctx[i];
      if (do_upd) {
        row = inl.upd[3 * i];
        idx = inl.upd[3 * i + 1];
        blk = inl.upd[3 * i + 2];
      }
    } else {
      if (do_ctx) ctx = meta.ctx_src[i];
      if (do_upd) {
        row = meta.updates[3 * i];
        idx = meta.updates[3 * i + 1];
        blk = meta.updates[3 * i + 2];
      }
    }
    const bool chunk = i < n;
    const int64_t t = i >> cpr_log2;
    const int ch = (int)i & (cpr - 1);
    const int64_t src = (t * num_kv_heads + h) * cpr + ch;  // chunk index in k_new / v_new
    int64_t slot = -1;
    u32x4 kv = u32x4{0u, 0u, 0u, 0u}, vv = u32x4{0u, 0u, 0u, 0u};
    if (chunk) {
      if constexpr (kInline)
        slot = inl.slots[t];
      else
        slot = slots[t];
      kv = k_new[src];
      vv = v_new[src];
      // In a decode step (META: a few tokens, one round trip decides the
      // time) the three loads are kept ahead of the slot test below: the test
      // reads the slot only through this statement, which needs the K/V data
      // (else the compiler moves the K/V loads behind the test, or the test
      // between them, and waits for the slot first). A large scatter is
      // throughput-bound, and there the statement, which also stops the
      // compiler from overlapping consecutive iterations, measured slower.
      if constexpr (META) asm volatile("" : "+v"(slot) : "v"(kv), "v"(vv));
    }
    // stores
    if (do_ctx) meta.ctx_dst[i] = ctx;
    if (do_upd && row >= 0 && row < meta.rows && idx >= 0 && idx < meta.max_blocks)
      meta.tables[(int64_t)row * meta.max_blocks + idx] = blk;
    if (!chunk || slot < 0 || slot >= num_slots) continue;
    const int64_t blk_id = slot >> bs_log2;
    const int off = (int)slot & ((1 << bs_log2) - 1);
    // element index of the destination chunk
    const int64_t dst = ((((blk_id * num_kv_heads + h) << bs_log2) + off) << (cpr_log2 + 3)) + (int64_t)ch * 8;
    if constexpr (FMT == kF16) {
      *reinterpret_cast<u32x4*>(k_cache + dst * 2) = kv;
      *reinterpret_cast<u32x4*>(v_cache + dst * 2) = vv;
    } else {
      u32x2 ko, vo;
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        // fp16 pairs 2w, 2w + 1: values 4w .. 4w + 3, scaled in fp32
        const uint32_t k0 = kv[2 * w], k1 = kv[2 * w + 1];
        const uint32_t v0 = vv[2 * w], v1 = vv[2 * w + 1];
        ko[w] = fp8x4_encode<FMT>(__fmul_rn(h_lo(k0), kinv), __fmul_rn(h_hi(k0), kinv), __fmul_rn(h_lo(k1), kinv),
                                  __fmul_rn(h_hi(k1), kinv));
        vo[w] = fp8x4_encode<FMT>(__fmul_rn(h_lo(v0), vinv), __fmul_rn(h_hi(v0), vinv), __fmul_rn(h_lo(v1), vinv),
                                  __fmul_rn(h_hi(v1), vinv));
      }
      *reinterpret_cast<u32x2*>(k_cache + dst) = ko;
      *reinterpret_cast<u32x2*>(v_cache + dst) = vo;
    }
  }
}

}  // namespace
}  // namespace pkv

namespace pkv {
namespace {

// Whether p is pinned host memory, so that the host can read it here. A
// pointer the runtime does not know leaves an error, which is cleared.
bool pinned_host(const void* p) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return at.type == hipMemoryTypeHost;
}

// Whether work queued on s is being captured into a graph (or the query
// fails, which is taken as yes).
bool capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) {
    (void)hipGetLastError();
    return true;
  }
  return st != hipStreamCaptureStatusNone;
}

int launch_kv_write(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                    const int64_t* slot_mapping, int num_tokens, int num_blocks, int num_kv_heads,
                    int head_dim, int block_size, int kv_dtype, float k_inv_scale, float v_inv_scale,
                    const float* k_inv_h, const float* v_inv_h, const StepMeta* meta, void* stream) {
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0) return PKV_ERR_INVALID;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_INVALID;
  if (block_size != 16 && block_size != 32 && block_size != 64) return PKV_ERR_INVALID;
  if (kv_dtype != PKV_KV_F16 && kv_dtype != PKV_KV_FP8_E4M3 && kv_dtype != PKV_KV_FP8_E5M2)
    return PKV_ERR_INVALID;
  const int64_t meta_work = meta ? (meta->n_ctx > meta->n_updates ? meta->n_ctx : meta->n_updates) : 0;
  if (num_tokens == 0 && meta_work == 0) return PKV_OK;
  if (num_tokens > 0 && (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping)) return PKV_ERR_INVALID;
  if (!vec_aligned(k_new) || !vec_aligned(v_new) || !vec_aligned(k_cache) || !vec_aligned(v_cache) ||
      !aligned_to(slot_mapping, 8) || !aligned_to(k_inv_h, 4) || !aligned_to(v_inv_h, 4))
    return PKV_ERR_INVALID;
  if (meta && (!aligned_to(meta->ctx_src, 4) || !aligned_to(meta->ctx_dst, 4) || !aligned_to(meta->updates, 4) ||
               !aligned_to(meta->tables, 4)))
    return PKV_ERR_INVALID;
  if (num_kv_heads > 65535) return PKV_ERR_INVALID;  // one grid row per head
  const int cpr_log2 = head_dim == 64 ? 3 : 4;      // log2(head_dim / 8)
  const int bs_log2 = block_size == 16 ? 4 : (block_size == 32 ? 5 : 6);
  const int64_t per_head = (int64_t)num_tokens << cpr_log2;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  const int threads = 256;
  const int64_t work = per_head > meta_work ? per_head : meta_work;
  int64_t blocks = (work + threads - 1) / threads;
  const int64_t cap = 65536 / num_kv_heads > 0 ? 65536 / num_kv_heads : 1;  // ~64k workgroups in all
  if (blocks > cap) blocks = cap;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const auto* kn = static_cast<const u32x4*>(k_new);
  const auto* vn = static_cast<const u32x4*>(v_new);
  auto* kc = static_cast<uint8_t*>(k_cache);
  auto* vc = static_cast<uint8_t*>(v_cache);
  const StepMeta m = meta ? *meta : StepMeta{nullptr, nullptr, 0, nullptr, 0, nullptr, 0, 0};
  const bool fp8 = kv_dtype != PKV_KV_F16;
  const float ki = fp8 ? k_inv_scale : 1.0f;
  const float vi = fp8 ? v_inv_scale : 1.0f;
  const dim3 grid((unsigned)blocks, (unsigned)num_kv_heads);
  // a decode step small enough to travel in the launch's arguments, with
  // its slots and metadata in pinned host memory, on a stream that is not
  // being captured (a captured launch keeps reading the host memory at each
  // replay)
  if (meta && num_tokens <= kInlineRows && m.n_ctx <= kInlineRows && m.n_updates <= kInlineRows &&
      num_slots <= 0x7FFFFFFF && !capturing(s) && (num_tokens == 0 || pinned_host(slot_mapping)) &&
      (m.n_ctx == 0 || pinned_host(m.ctx_src)) && (m.n_updates == 0 || pinned_host(m.updates))) {
    StepInline in;
    for (int t = 0; t < num_tokens; ++t) {
      const int64_t sl = slot_mapping[t];
      in.slots[t] = sl >= 0 && sl < num_slots ? (int32_t)sl : -1;
    }
    for (int i = 0; i < m.n_ctx; ++i) in.ctx[i] = m.ctx_src[i];
    for (int i = 0; i < 3 * m.n_updates; ++i) in.upd[i] = m.updates[i];
    decltype(&kv_write_kernel<kF16, true, StepInline>) ik;
    if (kv_dtype == PKV_KV_F16)
      ik = kv_write_kernel<kF16, true, StepInline>;
    else if (kv_dtype == PKV_KV_FP8_E4M3)
      ik = kv_write_kernel<kE4M3, true, StepInline>;
    else
      ik = kv_write_kernel<kE5M2, true, StepInline>;
    hipLaunchKernelGGL(ik, grid, dim3(threads), 0, s, kn, vn, kc, vc, slot_mapping, (int64_t)num_tokens,
                       cpr_log2, num_kv_heads, num_slots, bs_log2, ki, vi, fp8 ? k_inv_h : nullptr,
                       fp8 ? v_inv_h : nullptr, m, in);
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
  }
  decltype(&kv_write_kernel<kF16, false>) kern;
  if (kv_dtype == PKV_KV_F16)
    kern = meta ? kv_write_kernel<kF16, true> : kv_write_kernel<kF16, false>;
  else if (kv_dtype == PKV_KV_FP8_E4M3)
    kern = meta ? kv_write_kernel<kE4M3, true> : kv_write_kernel<kE4M3, false>;
  else
    kern = meta ? kv_write_kernel<kE5M2, true> : kv_write_kernel<kE5M2, false>;
  hipLaunchKernelGGL(kern, grid, dim3(threads), 0, s, kn, vn, kc, vc, slot_mapping, (int64_t)num_tokens,
                     cpr_log2, num_kv_heads, num_slots, bs_log2, ki, vi, fp8 ? k_inv_h : nullptr,
                     fp8 ? v_inv_h : nullptr, m, NoInline{});
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace
}  // namespace pkv

extern "C" int paged_kv_write(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              const int64_t* slot_mapping, int num_tokens, int num_blocks,
                              int num_kv_heads, int head_dim, int block_size, int kv_dtype,
                              float k_inv_scale, float v_inv_scale, void* stream) {
  return pkv::launch_kv_write(k_new, v_new, k_cache, v_cache, slot_mapping, num_tokens, num_blocks,
                              num_kv_heads, head_dim, block_size, kv_dtype, k_inv_scale, v_inv_scale,
                              nullptr, nullptr, nullptr, stream);
}

extern "C" int paged_kv_write_scaled(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                     const int64_t* slot_mapping, int num_tokens, int num_blocks,
                                     int num_kv_heads, int head_dim, int block_size, int kv_dtype,
                                     const float* k_inv_scales, const float* v_inv_scales, void* stream) {
  if (kv_dtype != PKV_KV_F16 && num_tokens > 0 && (!k_inv_scales || !v_inv_scales)) return PKV_ERR_INVALID;
  return pkv::launch_kv_write(k_new, v_new, k_cache, v_cache, slot_mapping, num_tokens, num_blocks,
                              num_kv_heads, head_dim, block_size, kv_dtype, 1.0f, 1.0f, k_inv_scales,
                              v_inv_scales, nullptr, stream);
}

extern "C" int paged_kv_write_step(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                   const int64_t* slot_mapping, int num_tokens, int num_blocks,
                                   int num_kv_heads, int head_dim, int block_size, int kv_dtype,
                                   float k_inv_scale, float v_inv_scale, const int32_t* ctx_src,
                                   int32_t* ctx_dst, int n_ctx, const int32_t* updates, int n_updates,
                                   int32_t* block_tables, int num_rows, int max_blocks, void* stream) {
  if (n_ctx < 0 || n_updates < 0 || num_rows < 0 || max_blocks < 0) return PKV_ERR_INVALID;
  if (n_ctx > 0 && (!ctx_src || !ctx_dst)) return PKV_ERR_INVALID;
  if (n_updates > 0 && (!updates || !block_tables)) return PKV_ERR_INVALID;
  const pkv::StepMeta m{ctx_src, ctx_dst, n_ctx, updates, n_updates, block_tables, num_rows, max_blocks};
  return pkv::launch_kv_write(k_new, v_new, k_cache, v_cache, slot_mapping, num_tokens, num_blocks,
                              num_kv_heads, head_dim, block_size, kv_dtype, k_inv_scale, v_inv_scale,
                              nullptr, nullptr, &m, stream);
}

extern "C" int paged_kv_write_step_scaled(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                          const int64_t* slot_mapping, int num_tokens, int num_blocks,
                                          int num_kv_heads, int head_dim, int block_size, int kv_dtype,
                                          const float* k_inv_scales, const float* v_inv_scales,
                                          const int32_t* ctx_src, int32_t* ctx_dst, int n_ctx,
                                          const int32_t* updates, int n_updates, int32_t* block_tables,
                                          int num_rows, int max_blocks, void* stream) {
  if (n_ctx < 0 || n_updates < 0 || num_rows < 0 || max_blocks < 0) return PKV_ERR_INVALID;
  if (n_ctx > 0 && (!ctx_src || !ctx_dst)) return PKV_ERR_INVALID;
  if (n_updates > 0 && (!updates || !block_tables)) return PKV_ERR_INVALID;
  if (kv_dtype != PKV_KV_F16 && num_tokens > 0 && (!k_inv_scales || !v_inv_scales)) return PKV_ERR_INVALID;
  const pkv::StepMeta m{ctx_src, ctx_dst, n_ctx, updates, n_updates, block_tables, num_rows, max_blocks};
  return pkv::launch_kv_write(k_new, v_new, k_cache, v_cache, slot_mapping, num_tokens, num_blocks,
                              num_kv_heads, head_dim, block_size, kv_dtype, 1.0f, 1.0f, k_inv_scales,
                              v_inv_scales, &m, stream);
}
