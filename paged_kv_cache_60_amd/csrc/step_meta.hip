// paged_step_metadata: the host-to-device part of one decode step.
//
// After the host block manager has appended one token per sequence
// ("From OOM to Smooth Inference (RAG memory management)", §2.3: a new block
// only when the last one is full; "vLLM Architecture and Memory Use, ch. 3",
// §3.3: a fresh block replaces a shared one before a write), the device needs
// the new tokens' slots, the new context lengths, the copy-on-write pairs and
// the few block-table entries that changed. The block tables stay resident on
// the device; only their changed entries travel.
//
// The sources are normally pinned host memory, read directly by this kernel
// over the bus (a few KiB), which is cheaper than queuing a DMA copy for such
// a small payload.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pagedkv.h"
#include "device_common.hpp"

namespace pkv {
namespace {

__global__ void __launch_bounds__(256)
step_meta_kernel(const int64_t* __restrict__ slots_src, int64_t* __restrict__ slots_dst,
                 const int32_t* __restrict__ ctx_src, int32_t* __restrict__ ctx_dst, int n,
                 const int32_t* __restrict__ cow_src, int32_t* __restrict__ cow_dst, int n_cow,
                 const int32_t* __restrict__ upd, int n_upd, int32_t* __restrict__ tables,
                 int rows, int max_blocks) {
  const int stride = gridDim.x * blockDim.x;
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  for (int i = tid; i < n; i += stride) {
    slots_dst[i] = slots_src[i];
    ctx_dst[i] = ctx_src[i];
  }
  for (int i = tid; i < 2 * n_cow; i += stride) cow_dst[i] = cow_src[i];
  for (int k = tid; k < n_upd; k += stride) {
    const int row = upd[3 * k];
    const int idx = upd[3 * k + 1];
    if (row >= 0 && row < rows && idx >= 0 && idx < max_blocks)
      tables[(int64_t)row * max_blocks + idx] = upd[3 * k + 2];
  }
}

}  // namespace
}  // namespace pkv

extern "C" int paged_step_metadata(const int64_t* slots_src, int64_t* slots_dst,
                                   const int32_t* ctx_src, int32_t* ctx_dst, int n_seqs,
                                   const int32_t* cow_src, int32_t* cow_dst, int n_cow,
                                   const int32_t* updates, int n_updates, int32_t* block_tables,
                                   int num_rows, int max_blocks, void* stream) {
  if (n_seqs < 0 || n_cow < 0 || n_updates < 0 || num_rows < 0 || max_blocks < 0) return PKV_ERR_INVALID;
  if (n_seqs > 0 && (!slots_src || !slots_dst || !ctx_src || !ctx_dst)) return PKV_ERR_INVALID;
  if (n_cow > 0 && (!cow_src || !cow_dst)) return PKV_ERR_INVALID;
  if (n_updates > 0 && (!updates || !block_tables)) return PKV_ERR_INVALID;
  if (!pkv::aligned_to(slots_src, 8) || !pkv::aligned_to(slots_dst, 8) || !pkv::aligned_to(ctx_src, 4) ||
      !pkv::aligned_to(ctx_dst, 4) || !pkv::aligned_to(cow_src, 4) || !pkv::aligned_to(cow_dst, 4) ||
      !pkv::aligned_to(updates, 4) || !pkv::aligned_to(block_tables, 4))
    return PKV_ERR_INVALID;
  const int work = n_seqs > n_updates ? (n_seqs > 2 * n_cow ? n_seqs : 2 * n_cow)
                                      : (n_updates > 2 * n_cow ? n_updates : 2 * n_cow);
  if (work == 0) return PKV_OK;
  int blocks = (work + 255) / 256;
  if (blocks > 64) blocks = 64;
  hipLaunchKernelGGL(pkv::step_meta_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     slots_src, slots_dst, ctx_src, ctx_dst, n_seqs, cow_src, cow_dst, n_cow, updates,
                     n_updates, block_tables, num_rows, max_blocks);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
