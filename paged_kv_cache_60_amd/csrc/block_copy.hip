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

}  // namespace
}  // namespace pkv

extern "C" int paged_block_copy(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs,
                                int num_blocks, size_t block_bytes, void* stream) {
  if (num_pairs < 0 || num_blocks <= 0 || block_bytes == 0 || block_bytes % 16 != 0)
    return PKV_ERR_INVALID;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !pairs) return PKV_ERR_INVALID;
  if (num_pairs > 65535) return PKV_ERR_INVALID;
  hipLaunchKernelGGL(pkv::block_copy_kernel, dim3(num_pairs, 2), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<pkv::u32x4*>(k_cache),
                     static_cast<pkv::u32x4*>(v_cache), pairs, num_blocks,
                     (int64_t)(block_bytes / 16));
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
