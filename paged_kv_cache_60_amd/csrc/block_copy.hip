// paged_block_copy: whole-block copies for copy-on-write.
//
// A write into a block that several sequences share first duplicates the
// block into a fresh one ("vLLM Architecture and Memory Use, ch. 3", §3.3);
// forked beams duplicate only their last, partially filled block ("From OOM
// to Smooth Inference (RAG memory management)", §6.1). The pairs come from the
// host block manager; K and V are copied alike.
//
// One workgroup per (pair, cache); 256 threads move 16 bytes each per step,
// i.e. 4 KiB per step, fully coalesced on both sides.
//
// paged_block_swap: the same whole-block copies between the device caches
// and a pinned host pool, for preemption by swapping ("Where Did the VRAM Go
// (KV cache tutorial)", §7.1-7.2; "From OOM to Smooth Inference", §5). The
// kernel reads or writes the host pool directly over the bus; each thread
// keeps four 16-byte transfers in flight, so a launch of many pairs covers
// the bus latency without one DMA request per block.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pagedkv.h"
#include "device_common.hpp"

namespace pkv {
namespace {

__global__ void __launch_bounds__(256)
block_copy_kernel(u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache,
                  const int32_t* __restrict__ pairs, int num_blocks, int64_t vecs_per_block) {
  const int p = blockIdx.x;
  u32x4* cache = blockIdx.y == 0 ? k_cache : v_cache;
  const int32_t src = pairs[2 * p];
  const int32_t dst = pairs[2 * p + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const u32x4* s = cache + (int64_t)src * vecs_per_block;
  u32x4* d = cache + (int64_t)dst * vecs_per_block;
  for (int64_t i = threadIdx.x; i < vecs_per_block; i += blockDim.x) d[i] = s[i];
}

// dst[b_dst] <- src[b_src] for every pair, K (blockIdx.y 0) and V (1).
__global__ void __launch_bounds__(256)
block_swap_kernel(const u32x4* __restrict__ k_src, const u32x4* __restrict__ v_src, u32x4* __restrict__ k_dst,
                  u32x4* __restrict__ v_dst, const int32_t* __restrict__ pairs, int n_src_blocks,
                  int n_dst_blocks, int64_t vecs_per_block) {
  const int p = blockIdx.x;
  const u32x4* src_c = blockIdx.y == 0 ? k_src : v_src;
  u32x4* dst_c = blockIdx.y == 0 ? k_dst : v_dst;
  const int32_t src = pairs[2 * p];
  const int32_t dst = pairs[2 * p + 1];
  if (src < 0 || src >= n_src_blocks || dst < 0 || dst >= n_dst_blocks) return;
  const u32x4* s = src_c + (int64_t)src * vecs_per_block;
  u32x4* d = dst_c + (int64_t)dst * vecs_per_block;
  constexpr int U = 4;
  int64_t i = threadIdx.x;
  for (; i + (U - 1) * 256 < vecs_per_block; i += U * 256) {
    u32x4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = s[i + u * 256];
#pragma unroll
    for (int u = 0; u < U; ++u) d[i + u * 256] = r[u];
  }
  for (; i < vecs_per_block; i += 256) d[i] = s[i];
}

}  // namespace
}  // namespace pkv

extern "C" int paged_block_swap(void* k_cache, void* v_cache, void* k_host, void* v_host, const int32_t* pairs,
                                int num_pairs, int num_blocks, int num_host_blocks, size_t block_bytes,
                                int direction, void* stream) {
  if (num_pairs < 0 || num_blocks <= 0 || num_host_blocks <= 0 || block_bytes == 0 || block_bytes % 16 != 0 ||
      (direction != PKV_SWAP_OUT && direction != PKV_SWAP_IN))
    return PKV_ERR_INVALID;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !k_host || !v_host || !pairs) return PKV_ERR_INVALID;
  if (!pkv::vec_aligned(k_cache) || !pkv::vec_aligned(v_cache) || !pkv::vec_aligned(k_host) ||
      !pkv::vec_aligned(v_host) || !pkv::aligned_to(pairs, 4))
    return PKV_ERR_INVALID;
  if (num_pairs > 0x7FFFFFFF / 2) return PKV_ERR_INVALID;
  const bool out = direction == PKV_SWAP_OUT;
  using pkv::u32x4;
  const u32x4* ks = static_cast<const u32x4*>(out ? k_cache : k_host);
  const u32x4* vs = static_cast<const u32x4*>(out ? v_cache : v_host);
  u32x4* kd = static_cast<u32x4*>(out ? k_host : k_cache);
  u32x4* vd = static_cast<u32x4*>(out ? v_host : v_cache);
  hipLaunchKernelGGL(pkv::block_swap_kernel, dim3(num_pairs, 2), dim3(256), 0, static_cast<hipStream_t>(stream),
                     ks, vs, kd, vd, pairs, out ? num_blocks : num_host_blocks, out ? num_host_blocks : num_blocks,
                     (int64_t)(block_bytes / 16));
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

extern "C" int paged_block_copy(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs,
                                int num_blocks, size_t block_bytes, void* stream) {
  if (num_pairs < 0 || num_blocks <= 0 || block_bytes == 0 || block_bytes % 16 != 0)
    return PKV_ERR_INVALID;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !pairs) return PKV_ERR_INVALID;
  if (!pkv::vec_aligned(k_cache) || !pkv::vec_aligned(v_cache) || !pkv::aligned_to(pairs, 4))
    return PKV_ERR_INVALID;
  if (num_pairs > 65535) return PKV_ERR_INVALID;
  hipLaunchKernelGGL(pkv::block_copy_kernel, dim3(num_pairs, 2), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<pkv::u32x4*>(k_cache),
                     static_cast<pkv::u32x4*>(v_cache), pairs, num_blocks,
                     (int64_t)(block_bytes / 16));
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
