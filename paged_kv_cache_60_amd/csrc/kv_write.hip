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

#include "../../include/pagedkv.h"
#include "device_common.hpp"

namespace pkv {
namespace {

// e4m3fn byte for a float: round to nearest even, saturate to +-448, keep the
// sign of zero, NaN -> 0x7F. All steps are exact except the final rint, which
// is the rounding itself.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __builtin_fabsf(f);
  if (!(a == a)) return 0x7Fu;
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) {  // below 2^-6: subnormal grid of 2^-9
    const float q = __builtin_rintf(a * 512.0f);  // 0..8; 8 is the smallest normal, code 0x08
    return sign | (uint32_t)q;
  }
  int e = (int)((__builtin_bit_cast(uint32_t, a) >> 23) & 0xFF) - 127;  // -6..8
  float q = __builtin_rintf(__builtin_ldexpf(a, 3 - e));                 // 8..16
  if (q == 16.0f) {
    q = 8.0f;
    e += 1;
  }
  return sign | ((uint32_t)(e + 7) << 3) | ((uint32_t)q - 8u);
}

// e5m2 byte for a float: round to nearest even, saturate to +-57344 (an
// infinite input too), keep the sign of zero, NaN -> 0x7F. Exponent bias 15,
// 2 mantissa bits, subnormals on a grid of 2^-16 below 2^-14.
__device__ __forceinline__ uint32_t e5m2_rne_sat(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __builtin_fabsf(f);
  if (!(a == a)) return 0x7Fu;
  if (a >= 57344.0f) return sign | 0x7Bu;
  if (a < 6.103515625e-05f) {  // below 2^-14
    const float q = __builtin_rintf(a * 65536.0f);  // 0..4; 4 is the smallest normal, code 0x04
    return sign | (uint32_t)q;
  }
  int e = (int)((__builtin_bit_cast(uint32_t, a) >> 23) & 0xFF) - 127;  // -14..15
  float q = __builtin_rintf(__builtin_ldexpf(a, 2 - e));                 // 4..8
  if (q == 8.0f) {
    q = 4.0f;
    e += 1;
  }
  return sign | ((uint32_t)(e + 15) << 2) | ((uint32_t)q - 4u);
}

template <int FMT>
__device__ __forceinline__ uint32_t fp8_encode(float f) {
  if constexpr (FMT == kE4M3)
    return e4m3_rne_sat(f);
  else
    return e5m2_rne_sat(f);
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

// k_inv_h / v_inv_h: one multiplier per KV head (device memory), or null to
// use k_inv / v_inv for every head.
template <int FMT, bool META>
__global__ void __launch_bounds__(256)
kv_write_kernel(const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new,
                uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                const int64_t* __restrict__ slots, int64_t total_chunks, int chunks_per_token,
                int chunks_per_row, int64_t num_slots, int bs, int64_t row_stride_blk,
                int head_dim, float k_inv, float v_inv, const float* __restrict__ k_inv_h,
                const float* __restrict__ v_inv_h, StepMeta meta) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if constexpr (META) {
    for (int64_t i = gtid; i < meta.n_ctx; i += stride) meta.ctx_dst[i] = meta.ctx_src[i];
    for (int64_t k = gtid; k < meta.n_updates; k += stride) {
      const int row = meta.updates[3 * k];
      const int idx = meta.updates[3 * k + 1];
      if (row >= 0 && row < meta.rows && idx >= 0 && idx < meta.max_blocks)
        meta.tables[(int64_t)row * meta.max_blocks + idx] = meta.updates[3 * k + 2];
    }
  }
  for (int64_t i = gtid; i < total_chunks; i += stride) {
    const int64_t t = i / chunks_per_token;
    const int within = (int)(i - t * chunks_per_token);
    const int h = within / chunks_per_row;
    const int ch = within - h * chunks_per_row;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t blk = slot / bs;
    const int off = (int)(slot - blk * bs);
    // element index of the destination chunk
    const int64_t dst = (blk * row_stride_blk + (int64_t)h * bs + off) * head_dim + (int64_t)ch * 8;
    const u32x4 kv = k_new[i];
    const u32x4 vv = v_new[i];
    if constexpr (FMT == kF16) {
      *reinterpret_cast<u32x4*>(k_cache + dst * 2) = kv;
      *reinterpret_cast<u32x4*>(v_cache + dst * 2) = vv;
    } else {
      const float kinv = k_inv_h ? k_inv_h[h] : k_inv;
      const float vinv = v_inv_h ? v_inv_h[h] : v_inv;
      u32x2 ko, vo;
      for (int w = 0; w < 2; ++w) {
        uint32_t kb = 0, vb = 0;
        for (int j = 0; j < 4; ++j) {
          const uint32_t kw = kv[w * 2 + j / 2];
          const uint32_t vw = vv[w * 2 + j / 2];
          const float kf = (j & 1) ? h_hi(kw) : h_lo(kw);
          const float vf = (j & 1) ? h_hi(vw) : h_lo(vw);
          kb |= fp8_encode<FMT>(__fmul_rn(kf, kinv)) << (8 * j);
          vb |= fp8_encode<FMT>(__fmul_rn(vf, vinv)) << (8 * j);
        }
        ko[w] = kb;
        vo[w] = vb;
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
  const int chunks_per_row = head_dim / 8;
  const int chunks_per_token = chunks_per_row * num_kv_heads;
  const int64_t total = (int64_t)num_tokens * chunks_per_token;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  const int64_t row_stride_blk = (int64_t)num_kv_heads * block_size;
  const int threads = 256;
  const int64_t work = total > meta_work ? total : meta_work;
  int64_t blocks = (work + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const auto* kn = static_cast<const u32x4*>(k_new);
  const auto* vn = static_cast<const u32x4*>(v_new);
  auto* kc = static_cast<uint8_t*>(k_cache);
  auto* vc = static_cast<uint8_t*>(v_cache);
  const StepMeta m = meta ? *meta : StepMeta{nullptr, nullptr, 0, nullptr, 0, nullptr, 0, 0};
  const bool fp8 = kv_dtype != PKV_KV_F16;
  const float ki = fp8 ? k_inv_scale : 1.0f;
  const float vi = fp8 ? v_inv_scale : 1.0f;
  decltype(&kv_write_kernel<kF16, false>) kern;
  if (kv_dtype == PKV_KV_F16)
    kern = meta ? kv_write_kernel<kF16, true> : kv_write_kernel<kF16, false>;
  else if (kv_dtype == PKV_KV_FP8_E4M3)
    kern = meta ? kv_write_kernel<kE4M3, true> : kv_write_kernel<kE4M3, false>;
  else
    kern = meta ? kv_write_kernel<kE5M2, true> : kv_write_kernel<kE5M2, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(threads), 0, s, kn, vn, kc, vc, slot_mapping,
                     total, chunks_per_token, chunks_per_row, num_slots, block_size, row_stride_blk,
                     head_dim, ki, vi, fp8 ? k_inv_h : nullptr, fp8 ? v_inv_h : nullptr, m);
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
