// paged_attn_decode: one query token per sequence attends over its paged KV.
//
// The cache is reached through a per-sequence block table: logical block i of
// a sequence lives in physical block table[i] ("From OOM to Smooth Inference
// (RAG memory management)", §2.1; "Inference Engine Memory Optimisation",
// §2.2). The output is plain softmax attention over the sequence's tokens.
// With an fp8 e4m3 cache K and V are dequantised with one scale per tensor
// ("Where Did the VRAM Go (KV cache tutorial)", §6.1-6.3).
//
// Pass 1 (partition kernel). One workgroup per (partition, sequence, KV
// head); the KV head index varies fastest across workgroup ids, so that the
// round-robin dispatch of workgroups over the eight XCDs spreads heads (and
// not partitions) over XCDs: every XCD gets an equal share of long and short
// partitions, and the workgroups that read one KV head of a shared prefix
// land on the same XCD and share its L2.
//   - A partition is `part_tokens` consecutive tokens, cut into 16-token
//     tiles; a tile never straddles two blocks (block sizes are multiples of
//     16), so each tile needs one block-table entry (wave-uniform).
//   - Lane mapping: each lane loads 16 contiguous bytes of a token row, so one
//     wave load covers 64 x 16 B = 1 KiB of contiguous K (or V) rows of one
//     block: LPR = row bytes / 16 lanes per token, 64 / LPR tokens per load.
//   - q.k: per-lane fp16 dot products (fp8 rows are first widened to fp16
//     exactly by the hardware conversion) and a DPP butterfly over the LPR
//     lanes of the row.
//   - Each group of LPR lanes keeps its own online softmax state (running
//     max m, sum l, unnormalised output slice) over the tokens it sees, so the
//     hot loop has no cross-row traffic; rows, then waves (through LDS), are
//     merged once at the end of the partition.
//   - All query heads of a GQA group are handled by the workgroup that loads
//     their KV head, so K/V are read once per group. Groups of 4 or 8 heads
//     run on the matrix cores instead (attn_gqa_mfma.hpp).
//   - A sequence that fits in one partition is normalised and written here.
// Pass 2 (reduce kernel). One wave per (sequence, query head): combines the
// partitions' (m, l, o) with weights exp(m_p - max m) and writes fp16.
//
// Exponentials are taken base 2 with log2(e) folded into the logit scale.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pagedkv.h"
#include "device_common.hpp"

namespace pkv {
namespace {

constexpr int kTile = 16;
constexpr int kWaves = 4;

struct AttnArgs {
  const f16* q;
  const uint8_t* kc;
  const uint8_t* vc;
  const int32_t* tables;
  const int32_t* ctx_lens;
  float* ws_o;   // [B][Hq][max_parts][D]
  float* ws_ml;  // [B][Hq][max_parts][2] = (max, sum)
  f16* out;
  int max_blocks;
  int B;
  int Hkv;
  int Hq;
  int bs_log2;
  int num_blocks;
  int part_tokens;
  int max_parts;
  float qk_scale;     // sm_scale * log2(e), times k_scale for fp8
  float v_out_scale;  // v_scale for fp8, else 1
};

__device__ __forceinline__ int clamp_len(int L, int Lmax) { return L < 0 ? 0 : (L > Lmax ? Lmax : L); }

__device__ __forceinline__ float safe_max(float m) { return m == -INFINITY ? 0.0f : m; }

template <int D, int G, bool FP8, int NW>
__global__ void __launch_bounds__(NW * 64) attn_partition_kernel(AttnArgs a) {
  constexpr int ELEM = FP8 ? 1 : 2;
  constexpr int RB = D * ELEM;       // bytes of one token row of one head
  constexpr int LPR = RB / 16;       // lanes per row
  constexpr int RPL = 64 / LPR;      // rows per wave load
  constexpr int NLD = kTile / RPL;   // loads per tile, per tensor
  constexpr int E = 16 / ELEM;       // elements per lane per row
  constexpr int W = E / 2;           // fp16 pairs per lane per row
  static_assert(NLD >= 1 && kTile % RPL == 0, "tile shape");

  const int wg = blockIdx.x;
  const int head = wg % a.Hkv;
  const int rest = wg / a.Hkv;
  const int seq = rest % a.B;
  const int part = rest / a.B;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane / LPR;
  const int c = lane % LPR;
  const int hq0 = head * G;

  const int L = clamp_len(a.ctx_lens[seq], a.max_blocks << a.bs_log2);
  const int nparts = (L + a.part_tokens - 1) / a.part_tokens;
  if (L == 0) {
    if (part == 0)
      for (int i = threadIdx.x; i < G * D; i += NW * 64)
        a.out[((size_t)seq * a.Hq + hq0) * D + i] = (f16)0.0f;
    return;
  }
  if (part >= nparts) return;
  const int t_begin = part * a.part_tokens;
  const int t_end = min(L, t_begin + a.part_tokens);

  // Query fragments: head hq0+g, elements c*E .. c*E+E-1, as fp16 pairs.
  uint32_t qf[G][W];
  {
    const uint32_t* qrow = reinterpret_cast<const uint32_t*>(a.q + ((size_t)seq * a.Hq + hq0) * D);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int w = 0; w < W; w += 4) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + g * (D / 2) + c * W + w);
        qf[g][w] = v[0];
        qf[g][w + 1] = v[1];
        qf[g][w + 2] = v[2];
        qf[g][w + 3] = v[3];
      }
  }

  float m[G], l[G], acc[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = 0.0f;
  }

  const int32_t* tab = a.tables + (size_t)seq * a.max_blocks;
  const int ntiles = (t_end - t_begin + kTile - 1) / kTile;
  // this wave takes tiles wave, wave + NW, wave + 2 NW, ...
  const int my_tiles = ntiles > wave ? (ntiles - wave + NW - 1) / NW : 0;
  const size_t head_bytes = (size_t)RB << a.bs_log2;
  const size_t blk_stride = (size_t)a.Hkv * head_bytes;
  const uint8_t* kc_head = a.kc + (size_t)head * head_bytes;
  const uint8_t* vc_head = a.vc + (size_t)head * head_bytes;
  const int bs_mask = (1 << a.bs_log2) - 1;
  const uint32_t lane_off = (uint32_t)(r * RB + c * 16);

  for (int j0 = 0; j0 < my_tiles; j0 += 64) {
    // Block ids of up to 64 of this wave's tiles, one per lane, fetched
    // together so that no tile waits on its own table read.
    int my_blk = -1;
    if (j0 + lane < my_tiles) {
      const int t = t_begin + (wave + NW * (j0 + lane)) * kTile;
      my_blk = tab[t >> a.bs_log2];
    }
    const int nj = min(64, my_tiles - j0);
    for (int j = 0; j < nj; ++j) {
      const int blk = __builtin_amdgcn_readlane(my_blk, j);
      if ((unsigned)blk >= (unsigned)a.num_blocks) continue;  // never followed
      const int t0 = t_begin + (wave + NW * (j0 + j)) * kTile;
      // A tile lies inside one block, so all 16 rows are in bounds even past
      // the sequence end; rows at or past t_end are masked below.
      const bool full = t0 + kTile <= t_end;
      const size_t boff = (size_t)blk * blk_stride + (size_t)(t0 & bs_mask) * RB;
      const uint8_t* kb = kc_head + boff;
      const uint8_t* vb = vc_head + boff;

      u32x4 kr[NLD], vr[NLD];
      bool valid[NLD];
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        // non-temporal: K/V are streamed once per step; not allocating them in
        // the caches measured 12% faster than default loads on this path
        kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + lane_off + i * RPL * RB));
        vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + lane_off + i * RPL * RB));
        valid[i] = full || (t0 + i * RPL + r < t_end);
      }
      if (!full) {
#pragma unroll
        for (int i = 0; i < NLD; ++i)
          if (!valid[i]) vr[i] = u32x4{0u, 0u, 0u, 0u};
      }

      // logits z[i][g] (log2 domain)
      float z[NLD][G];
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        uint32_t kw[W];
#pragma unroll
        for (int w = 0; w < W; ++w) {
          if constexpr (FP8)
            kw[w] = (w & 1) ? fp8x2_hi_to_f16x2(kr[i][w / 2]) : fp8x2_lo_to_f16x2(kr[i][w / 2]);
          else
            kw[w] = kr[i][w];
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float s = 0.0f;
#pragma unroll
          for (int w = 0; w < W; ++w) s = dot2(qf[g][w], kw[w], s);
          s = group_sum<LPR>(s);
          z[i][g] = valid[i] ? s * a.qk_scale : -INFINITY;
        }
      }

      // online softmax update and P.V for each head of the group
      float p[NLD][G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float mt = z[0][g];
#pragma unroll
        for (int i = 1; i < NLD; ++i) mt = fmaxf(mt, z[i][g]);
        const float mn = fmaxf(m[g], mt);
        const float ms = safe_max(mn);
        const float alpha = fast_exp2(m[g] - ms);
        float ps = 0.0f;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          p[i][g] = fast_exp2(z[i][g] - ms);
          ps += p[i][g];
        }
        l[g] = l[g] * alpha + ps;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[g][e] *= alpha;
        m[g] = mn;
      }
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        float vf[E];
#pragma unroll
        for (int w = 0; w < W; ++w) {
          uint32_t pw;
          if constexpr (FP8)
            pw = (w & 1) ? fp8x2_hi_to_f16x2(vr[i][w / 2]) : fp8x2_lo_to_f16x2(vr[i][w / 2]);
          else
            pw = vr[i][w];
          vf[2 * w] = h_lo(pw);
          vf[2 * w + 1] = h_hi(pw);
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < E; ++e) acc[g][e] = fmaf(p[i][g], vf[e], acc[g][e]);
      }
    }
  }

  // merge the RPL row states of this wave (lanes with equal c hold equal slices)
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = shfl_xor_f32(m[g], off);
      const float lo = shfl_xor_f32(l[g], off);
      const float mn = fmaxf(m[g], mo);
      const float ms = safe_max(mn);
      const float a1 = fast_exp2(m[g] - ms);
      const float a2 = fast_exp2(mo - ms);
      l[g] = l[g] * a1 + lo * a2;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[g][e] = acc[g][e] * a1 + shfl_xor_f32(acc[g][e], off) * a2;
      m[g] = mn;
    }
  }

  // merge the waves through LDS and write
  __shared__ float s_acc[NW][G][D];
  __shared__ float s_m[NW][G];
  __shared__ float s_l[NW][G];
  if (lane < LPR) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < E; ++e) s_acc[wave][g][c * E + e] = acc[g][e];
      if (lane == 0) {
        s_m[wave][g] = m[g];
        s_l[wave][g] = l[g];
      }
    }
  }
  __syncthreads();
  const bool single = nparts == 1;
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = s_m[0][g];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][g]);
    const float Ms = safe_max(M);
    float lsum = 0.0f, o = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(s_m[w][g] - Ms);
      lsum += s_l[w][g] * f;
      o += s_acc[w][g][d] * f;
    }
    const size_t hrow = (size_t)seq * a.Hq + hq0 + g;
    if (single) {
      a.out[hrow * D + d] = (f16)(lsum > 0.0f ? o * a.v_out_scale / lsum : 0.0f);
    } else {
      const size_t pi = hrow * a.max_parts + part;
      a.ws_o[pi * D + d] = o * a.v_out_scale;
      if (d == 0) {
        a.ws_ml[2 * pi] = M;
        a.ws_ml[2 * pi + 1] = lsum;
      }
    }
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, shfl_xor_f32(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += shfl_xor_f32(v, off);
  return v;
}

__device__ __forceinline__ float readlane_f32(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// One wave per (sequence, query head). Lane p holds partition p's (m, l) for
// up to 64 partitions at a time; each lane owns D/64 output elements and
// issues the loads of all partitions' slices before summing.
template <int D>
__global__ void __launch_bounds__(256) attn_reduce_kernel(AttnArgs a) {
  constexpr int DL = D / 64;  // output elements per lane
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= a.B * a.Hq) return;
  const int lane = threadIdx.x & 63;
  const int seq = wid / a.Hq;
  const int L = clamp_len(a.ctx_lens[seq], a.max_blocks << a.bs_log2);
  const int nparts = (L + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;  // finished by pass 1
  const size_t pbase = (size_t)wid * a.max_parts;
  const float* ml = a.ws_ml + 2 * pbase;
  const float* o = a.ws_o + pbase * D + lane * DL;
  float M = -INFINITY;
  for (int p = lane; p < nparts; p += 64) M = fmaxf(M, ml[2 * p]);
  M = wave_max(M);
  const float Ms = safe_max(M);
  float lsum = 0.0f;
  float acc[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) acc[e] = 0.0f;
  for (int p0 = 0; p0 < nparts; p0 += 64) {
    float w = 0.0f;
    if (p0 + lane < nparts) {
      w = fast_exp2(ml[2 * (p0 + lane)] - Ms);
      lsum += ml[2 * (p0 + lane) + 1] * w;
    }
    const int np = min(64, nparts - p0);
    int q = 0;
    for (; q + 4 <= np; q += 4) {
      float v[4][DL];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < DL; ++e) v[u][e] = o[(size_t)(p0 + q + u) * D + e];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float wu = readlane_f32(w, q + u);
#pragma unroll
        for (int e = 0; e < DL; ++e) acc[e] = fmaf(wu, v[u][e], acc[e]);
      }
    }
    for (; q < np; ++q) {
      const float wq = readlane_f32(w, q);
#pragma unroll
      for (int e = 0; e < DL; ++e) acc[e] = fmaf(wq, o[(size_t)(p0 + q) * D + e], acc[e]);
    }
  }
  lsum = wave_sum(lsum);
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
#pragma unroll
  for (int e = 0; e < DL; ++e) a.out[(size_t)wid * D + lane * DL + e] = (f16)(acc[e] * inv);
}

}  // namespace
}  // namespace pkv

#include "attn_gqa_mfma.hpp"

namespace pkv {
namespace {

typedef void (*PartFn)(AttnArgs);

template <int D, bool FP8>
PartFn pick_partition_kernel(int G) {
  switch (G) {
    case 1: return attn_partition_kernel<D, 1, FP8, kWaves>;
    case 2: return attn_partition_kernel<D, 2, FP8, kWaves>;
    case 4: return attn_partition_mfma_kernel<D, 4, FP8, kWaves>;
    case 8: return attn_partition_mfma_kernel<D, 8, FP8, kWaves>;
    default: return nullptr;
  }
}

PartFn pick(int D, int G, bool fp8) {
  if (D == 64) return fp8 ? pick_partition_kernel<64, true>(G) : pick_partition_kernel<64, false>(G);
  if (D == 128) return fp8 ? pick_partition_kernel<128, true>(G) : pick_partition_kernel<128, false>(G);
  return nullptr;
}

int log2_exact(int v) {
  int k = 0;
  while ((1 << k) < v) ++k;
  return (1 << k) == v ? k : -1;
}

// Default partition: the largest power of two in [256, 2048] that is at most
// a quarter (one query head per KV head) or half (grouped heads) of the
// largest context the block table can hold. Measured on MI355X: 512 for the
// Llama-2-7B batch-64 workload, 1024-2048 for 4k contexts and for grouped heads.
int default_partition(int group, int max_blocks, int block_size) {
  const int64_t max_ctx = (int64_t)max_blocks * block_size;
  const int64_t target = max_ctx / (group >= 2 ? 2 : 4);
  int p = 256;
  while (p < 2048 && 2 * (int64_t)p <= target) p *= 2;
  return p;
}

int resolve_partition(int partition_tokens, int group, int max_blocks, int block_size) {
  if (partition_tokens == 0) return default_partition(group, max_blocks, block_size);
  if (partition_tokens < 64 || partition_tokens % 64 != 0) return -1;
  return partition_tokens;
}

int max_partitions(int max_blocks, int block_size, int part) {
  const int64_t lmax = (int64_t)max_blocks * block_size;
  return (int)((lmax + part - 1) / part);
}

}  // namespace
}  // namespace pkv

extern "C" int paged_attn_default_partition(int num_q_heads, int num_kv_heads, int head_dim,
                                            int block_size, int max_blocks_per_seq, int kv_dtype) {
  (void)head_dim;
  (void)kv_dtype;
  if (num_kv_heads <= 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0 || block_size <= 0) return -1;
  return pkv::default_partition(num_q_heads / num_kv_heads, max_blocks_per_seq, block_size);
}

extern "C" size_t paged_attn_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                                    int head_dim, int max_blocks_per_seq,
                                                    int block_size, int partition_tokens) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_blocks_per_seq <= 0 || block_size <= 0)
    return 0;
  const int part = pkv::resolve_partition(partition_tokens, num_q_heads / num_kv_heads,
                                          max_blocks_per_seq, block_size);
  if (part < 0) return 0;
  const int mp = pkv::max_partitions(max_blocks_per_seq, block_size, part);
  if (mp <= 1) return 0;
  return (size_t)num_seqs * num_q_heads * mp * (size_t)(head_dim + 2) * sizeof(float);
}

extern "C" int paged_attn_decode_passes(void* out, const void* q, const void* k_cache,
                                        const void* v_cache, const int32_t* block_tables,
                                        int max_blocks_per_seq, const int32_t* ctx_lens,
                                        int num_seqs, int num_q_heads, int num_kv_heads,
                                        int head_dim, int block_size, int num_blocks,
                                        float sm_scale, int kv_dtype, float k_scale,
                                        float v_scale, int partition_tokens, void* workspace,
                                        size_t workspace_bytes, int passes, void* stream) {
  using namespace pkv;
  if (passes < 1 || passes > 3) return PKV_ERR_INVALID;
  if (num_seqs < 0 || num_kv_heads <= 0 || num_q_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0)
    return PKV_ERR_INVALID;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_INVALID;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_INVALID;
  if (block_size != 16 && block_size != 32 && block_size != 64) return PKV_ERR_INVALID;
  if (kv_dtype != PKV_KV_F16 && kv_dtype != PKV_KV_FP8_E4M3) return PKV_ERR_INVALID;
  const int G = num_q_heads / num_kv_heads;
  const int part = resolve_partition(partition_tokens, G, max_blocks_per_seq, block_size);
  if (part < 0) return PKV_ERR_INVALID;
  const bool fp8 = kv_dtype == PKV_KV_FP8_E4M3;
  PartFn fn = pick(head_dim, G, fp8);
  if (!fn) return PKV_ERR_INVALID;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !ctx_lens) return PKV_ERR_INVALID;
  const int mp = max_partitions(max_blocks_per_seq, block_size, part);
  const size_t need = paged_attn_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                        max_blocks_per_seq, block_size, part);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_INVALID;
  const int64_t grid1 = (int64_t)num_kv_heads * num_seqs * mp;
  if (grid1 > 0x7FFFFFFF) return PKV_ERR_INVALID;

  AttnArgs a;
  a.q = static_cast<const f16*>(q);
  a.kc = static_cast<const uint8_t*>(k_cache);
  a.vc = static_cast<const uint8_t*>(v_cache);
  a.tables = block_tables;
  a.ctx_lens = ctx_lens;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_ml = need > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                (size_t)num_seqs * num_q_heads * mp * head_dim * sizeof(float))
                     : nullptr;
  a.out = static_cast<f16*>(out);
  a.max_blocks = max_blocks_per_seq;
  a.B = num_seqs;
  a.Hkv = num_kv_heads;
  a.Hq = num_q_heads;
  a.bs_log2 = log2_exact(block_size);
  a.num_blocks = num_blocks;
  a.part_tokens = part;
  a.max_parts = mp;
  const float kLog2e = 1.4426950408889634f;
  a.qk_scale = sm_scale * kLog2e * (fp8 ? k_scale : 1.0f);
  a.v_out_scale = fp8 ? v_scale : 1.0f;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (passes & 1) {
    hipLaunchKernelGGL(fn, dim3((unsigned)grid1), dim3(kWaves * 64), 0, s, a);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  }
  if ((passes & 2) && mp > 1) {
    const int waves = num_seqs * num_q_heads;
    const unsigned grid2 = (unsigned)((waves + 3) / 4);
    if (head_dim == 64)
      hipLaunchKernelGGL(attn_reduce_kernel<64>, dim3(grid2), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(attn_reduce_kernel<128>, dim3(grid2), dim3(256), 0, s, a);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  }
  return PKV_OK;
}

extern "C" int paged_attn_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, int max_blocks_per_seq,
                                 const int32_t* ctx_lens, int num_seqs, int num_q_heads,
                                 int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                 float sm_scale, int kv_dtype, float k_scale, float v_scale,
                                 int partition_tokens, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return paged_attn_decode_passes(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                                  ctx_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                  block_size, num_blocks, sm_scale, kv_dtype, k_scale, v_scale,
                                  partition_tokens, workspace, workspace_bytes, 3, stream);
}
