// paged_attn_decode: one query token per sequence attends over its paged KV.
//
// The cache is reached through a per-sequence block table: logical block i of
// a sequence lives in physical block table[i] ("From OOM to Smooth Inference
// (RAG memory management)", §2.1; "Inference Engine Memory Optimisation",
// §2.2). The output is plain softmax attention over the sequence's tokens.
// With an fp8 cache (e4m3 or e5m2) K and V are dequantised with one scale per
// tensor or one per KV head ("Where Did the VRAM Go (KV cache tutorial)",
// §6.1-6.3).
//
// Work decomposition (split-sequence, stream-K style). A segment is one
// (sequence, KV head); its tokens are cut into units of 16 tokens (32 on the
// matrix-core path). The segments are laid end to end, sequence-major, and the
// unit range is divided into equal contiguous shares, one per worker. A worker
// is one wave; by default there are as many workers as fit on the chip at
// once. A worker walks its share piece by piece (a piece = the part of one
// segment inside the share):
//   - a piece that is its whole segment is normalised and written to the
//     output directly;
//   - otherwise the piece's online-softmax state (max m, sum l, and its
//     output: unnormalised fp32 on the vector path, divided by l as fp16 on
//     the matrix-core path) goes to one of the worker's two partial slots:
//     slot 0 for the first piece of the share, slot 1 for the last (any piece
//     between them is a whole segment).
// Pass 2 combines, for every (sequence, query head) whose segment was split,
// the pieces of the consecutive workers that hold it, with weights
// exp(m_p - max m) (times l_p for the normalised ones), and writes zeros for
// empty sequences. The split depends
// only on the context lengths and the worker count, so results are
// deterministic and independent of block placement. Every worker streams the
// same number of tokens, no workgroup is idle and none waits on another.
//
// Pass 1, vector path (1 or 2 query heads per KV head):
//   - a 16-token tile never straddles two blocks (block sizes are multiples
//     of 16), so one table entry serves a tile; the block ids of up to 64
//     tiles are fetched together (one lane each) and broadcast with readlane;
//   - lane mapping: each lane loads 16 contiguous bytes of a token row, LPR =
//     row bytes / 16 lanes per row, 64 / LPR rows per wave load (1 KiB);
//   - q.k: per-lane fp16 dot products (fp8 rows widened to fp16 exactly by
//     the hardware conversion) and a DPP butterfly over the row's LPR lanes;
//   - each group of LPR lanes keeps its own online softmax over the rows it
//     sees; the groups are merged once per piece;
//   - K/V loads are non-temporal: streamed once, not kept in the caches.
// Groups of 4 or 8 query heads run on the matrix cores (attn_gqa_mfma.hpp).
//
// Exponentials are taken base 2 with log2(e) folded into the logit scale.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "../../include/pagedkv.h"
#include "device_common.hpp"

namespace pkv {
namespace {

constexpr int kTile = 16;
constexpr int kWaves = 4;          // waves (workers) per workgroup
constexpr int kMaxWorkers = 8192;  // the workspace holds partials for this many workers
constexpr int kMaxSeqs = 4096;     // sequences per launch (their unit prefix lives in LDS)
constexpr int kMaxGroupWorkers = 2048;  // the shared-prefix workspace holds partials for this many workers

struct AttnArgs {
  const f16* q;
  const uint8_t* kc;
  const uint8_t* vc;
  const int32_t* tables;
  const int32_t* ctx_lens;
  float* ws_o;     // [kMaxWorkers][2][G][D]  outputs of partial pieces (fp32, or fp16 for G >= 4)
  float* ws_ml;    // [kMaxWorkers][2][G][2]  (max, sum) of partial pieces
  int32_t* ws_pt;  // [B + 1]                 unit prefix over sequences (pass 1 -> pass 2)
  f16* out;
  int max_blocks;
  int B;
  int Hkv;
  int Hq;
  int bs_log2;
  int num_blocks;
  int unit_tokens;    // 16 (vector path) or 32 (matrix cores)
  int workers;        // W, a multiple of kWaves
  float qk_scale;     // sm_scale * log2(e), times k_scale for fp8
  float v_out_scale;  // v_scale for fp8, else 1
  // one scale per KV head (device memory), or null: then qk_scale and
  // v_out_scale hold for every head; else head h uses qk_base * k_scale_h[h]
  // and v_scale_h[h]
  const float* k_scale_h;
  const float* v_scale_h;
  float qk_base;      // sm_scale * log2(e)
  // Shared-prefix groups (paged_attn_decode_shared; NG = 0 otherwise). Group
  // g is the batch sequences grp_first[g] .. + grp_size[g] - 1; their first
  // group_tokens(grp_prefix[g]) tokens are read through the table of sequence
  // grp_first[g] once for all of them (attn_group_mfma.hpp).
  const int32_t* grp_first = nullptr;
  const int32_t* grp_size = nullptr;
  const int32_t* grp_prefix = nullptr;
  int NG = 0;
  int g_log2 = 0;              // log2(query heads per KV head)
  int32_t* ws_part = nullptr;  // [B] each sequence's part record (grouped pass 1 -> merge)
  int32_t* ws_seg = nullptr;   // [B][2] the unit range of each sequence's part (grouped pass 1 -> merge)
  // W / Hkv when the waves are dealt to the shares in head groups (W a
  // multiple of Hkv), else 0; see worker_index
  int head_groups = 0;
};

__device__ __forceinline__ int clamp_len(int L, int Lmax) { return L < 0 ? 0 : (L > Lmax ? Lmax : L); }

__device__ __forceinline__ float safe_max(float m) { return m == -INFINITY ? 0.0f : m; }

__device__ __forceinline__ int64_t share_start(int64_t w, int64_t total, int64_t W) { return w * total / W; }

// A value the caller knows is equal on all lanes of the wave, moved to a scalar
// register so that the arithmetic that depends on it stays scalar.
__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The clamped context length of sequence s.
__device__ __forceinline__ int seq_len(const AttnArgs& a, int s) {
  return clamp_len(a.ctx_lens[s], a.max_blocks << a.bs_log2);
}

// Members inside the batch of a group entry (first, size): 0 for an entry
// outside it.
__device__ __forceinline__ int group_members(const AttnArgs& a, int first, int size) {
  if (first < 0 || first >= a.B) return 0;
  return size < 0 ? 0 : min(size, a.B - first);
}

// Shared tokens of a group entry's prefix: a multiple of 16 (tiles never
// straddle the edge), within the table width.
__device__ __forceinline__ int group_tokens(const AttnArgs& a, int prefix) {
  return clamp_len(prefix, a.max_blocks << a.bs_log2) & ~15;
}

// pt[0] = 0, pt[i + 1] = pt[i] + units(i) for i < n, by all threads of the
// workgroup. units(i) may read pt[i + 1], which the caller may have filled
// with entry i's own value (a context length) before a barrier. Each wave
// scans a contiguous quarter of the entries (each lane a run of them, the
// runs combined with shuffles), the waves' totals go through `scan`
// (blockDim / 64 ints), and each wave adds the totals of the waves before
// it: two barriers in all. Ends with a barrier.
template <class Units>
__device__ void build_scan(int n, int* pt, int* scan, Units units) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int per_wave = (n + nw - 1) / nw;
  const int w0 = min(n, wv * per_wave);
  const int w1 = min(n, w0 + per_wave);
  const int per = (w1 - w0 + 63) / 64;
  const int b0 = min(w1, w0 + lane * per);
  const int b1 = min(w1, b0 + per);
  int s = 0;
  for (int i = b0; i < b1; ++i) {
    const int u = units(i);
    pt[i + 1] = u;
    s += u;
  }
  int x = s;  // inclusive scan of the runs over the wave's lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) scan[wv] = x;
  __syncthreads();
  int run = x - s;
  for (int k = 0; k < wv; ++k) run += scan[k];
  for (int i = b0; i < b1; ++i) {
    run += pt[i + 1];
    pt[i + 1] = run;
  }
  if (threadIdx.x == 0) pt[0] = 0;
  __syncthreads();
}

// Dynamic LDS of a pass-1 workgroup: pt[B + 1], scan[blockDim]. The context
// lengths are loaded by every thread at once into pt[i + 1] first.
__device__ void build_prefix(const AttnArgs& a, int* pt, int* scan) {
  for (int i = threadIdx.x; i < a.B; i += blockDim.x) pt[i + 1] = seq_len(a, i);
  __syncthreads();
  build_scan(a.B, pt, scan, [&](int i) { return (pt[i + 1] + a.unit_tokens - 1) / a.unit_tokens; });
}

// The last sequence s in [0, B) with pt[s] <= q; pt is non-decreasing, so
// empty sequences before a non-empty one are skipped.
__device__ __forceinline__ int find_seq(const int* pt, int B, int64_t q) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (wave_uniform(pt[mid]) <= q) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The piece of a share that starts at flattened unit t (< end). The unit
// space is head-major: KV head h holds units [h P, (h + 1) P), P = pt[B], and
// within a head the sequences follow one another.
struct Piece {
  int seq;
  int head;  // KV head
  int u0;    // first unit within the segment
  int u1;    // one past the last unit within the segment
  int n_u;   // units of the whole segment
  int64_t next_t;
};

__device__ __forceinline__ Piece locate(const int* pt, int B, int P, int64_t t, int64_t end) {
  Piece p;
  p.head = (int)(t / P);
  const int rem = (int)(t - (int64_t)p.head * P);
  p.seq = find_seq(pt, B, rem);
  const int p0 = wave_uniform(pt[p.seq]);
  p.n_u = wave_uniform(pt[p.seq + 1]) - p0;
  p.u0 = rem - p0;
  const int64_t seg_end = t - p.u0 + p.n_u;
  p.next_t = end < seg_end ? end : seg_end;
  p.u1 = p.u0 + (int)(p.next_t - t);
  return p;
}

// Worker index of wave `wave` of this workgroup. Workgroups are dispatched to
// The worker index of a wave: which equal share of the head-major unit space
// it streams. The eight XCDs take workgroups round-robin (workgroup g runs on
// XCD g % 8); workgroups g, g + 8, g + 16, ... take consecutive positions, so
// that each XCD, and its L2, holds one contiguous run of positions.
// Without head groups the position is the worker index: an XCD streams one
// contiguous slice of the unit space, a few KV heads of every sequence.
// With head groups (hg = W / Hkv), the Hkv consecutive positions p of a group
// take worker (p % Hkv) * hg + p / Hkv: the same share of every KV head's unit
// space (the shares of the head-major space fall on head boundaries when W is
// a multiple of Hkv), one head each. The waves of a group then walk the same
// tiles of the same sequences at about the same pace, and a block's heads,
// which lie side by side in the pool, are read together: the same bytes from
// fewer, larger regions of memory at once, which streams a few percent faster
// than every wave reading a region of its own.
__device__ __forceinline__ int64_t worker_index(int wave, int NW, const AttnArgs& a) {
  const int n = gridDim.x;
  const int xcd = blockIdx.x % 8;
  const int q = n / 8, r = n % 8;
  const int wg = xcd * q + min(xcd, r) + (int)(blockIdx.x / 8);
  const int64_t p = (int64_t)wg * NW + wave;
  const int hg = a.head_groups;
  if (hg > 0 && hg * a.Hkv == a.workers) return (int64_t)((int)p % a.Hkv) * hg + (int)p / a.Hkv;
  return p;
}

template <int D, int G, int FMT, int NW>
__global__ void __launch_bounds__(NW * 64) attn_partition_kernel(AttnArgs a) {
  constexpr bool FP8 = FMT != kF16;
  constexpr int ELEM = FP8 ? 1 : 2;
  constexpr int RB = D * ELEM;       // bytes of one token row of one head
  constexpr int LPR = RB / 16;       // lanes per row
  constexpr int RPL = 64 / LPR;      // rows per wave load
  constexpr int NLD = kTile / RPL;   // loads per tile, per tensor
  constexpr int E = 16 / ELEM;       // elements per lane per row
  constexpr int W = E / 2;           // fp16 pairs per lane per row
  static_assert(NLD >= 1 && kTile % RPL == 0, "tile shape");

  extern __shared__ int dyn_smem[];
  int* pt = dyn_smem;
  build_prefix(a, pt, pt + a.B + 1);

  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int r = lane / LPR;
  const int c = lane % LPR;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= a.B; i += NW * 64) a.ws_pt[i] = pt[i];
  const int P = wave_uniform(pt[a.B]);
  const int64_t total = (int64_t)a.Hkv * P;
  const int64_t w = worker_index(wave, NW, a);
  const int64_t start = share_start(w, total, a.workers);
  const int64_t end = share_start(w + 1, total, a.workers);

  const size_t head_bytes = (size_t)RB << a.bs_log2;
  const size_t blk_stride = (size_t)a.Hkv * head_bytes;
  const int bs_mask = (1 << a.bs_log2) - 1;
  const uint32_t lane_off = (uint32_t)(r * RB + c * 16);

  for (int64_t t = start; t < end;) {
    const Piece pc = locate(pt, a.B, P, t, end);
    const int seq = pc.seq;
    const int hq0 = pc.head * G;
    // The piece's setup loads (its length, the query fragments, the first 64
    // tiles' block ids) are all issued before the first wait: one round trip.
    const int L_raw = seq_len(a, seq);
    const int32_t* tab = a.tables + (size_t)seq * a.max_blocks;
    // lane l: the block of tile u0 + l (lanes past the piece read an entry
    // inside the row that no tile uses)
    auto tile_block = [&](int j0) {
      return tab[min(((j0 + lane) * kTile) >> a.bs_log2, a.max_blocks - 1)];
    };
    int my_blk = tile_block(pc.u0);

    // Query fragments: head hq0+g, elements c*E .. c*E+E-1, as fp16 pairs.
    uint32_t qf[G][W];
    {
      const uint32_t* qrow = reinterpret_cast<const uint32_t*>(a.q + ((size_t)seq * a.Hq + hq0) * D);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int x = 0; x < W; x += 4) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + g * (D / 2) + c * W + x);
          qf[g][x] = v[0];
          qf[g][x + 1] = v[1];
          qf[g][x + 2] = v[2];
          qf[g][x + 3] = v[3];
        }
    }

    // the logit and output scales of the head (both loads at once)
    float qk_scale = a.qk_scale, v_scale = a.v_out_scale;
    if (a.k_scale_h) {
      const float ks = a.k_scale_h[pc.head];
      const float vs = a.v_scale_h[pc.head];
      qk_scale = a.qk_base * ks;
      v_scale = vs;
    }
    const int L = wave_uniform(L_raw);

    float m[G], l[G], acc[G][E];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[g][e] = 0.0f;
    }

    const uint8_t* kc_head = a.kc + (size_t)pc.head * head_bytes;
    const uint8_t* vc_head = a.vc + (size_t)pc.head * head_bytes;
    for (int j0 = pc.u0; j0 < pc.u1; j0 += 64) {
      // block ids of up to 64 tiles, one per lane, fetched together so that
      // no tile waits on its own table read (the first 64 with the setup)
      if (j0 != pc.u0) my_blk = tile_block(j0);
      const int nj = min(64, pc.u1 - j0);
      for (int j = 0; j < nj; ++j) {
        const int blk = __builtin_amdgcn_readlane(my_blk, j);
        if ((unsigned)blk >= (unsigned)a.num_blocks) continue;  // never followed
        const int t0 = (j0 + j) * kTile;
        // A tile lies inside one block, so all 16 rows are in bounds even past
        // the sequence end; rows at or past L are masked below.
        const bool full = t0 + kTile <= L;
        const size_t boff = (size_t)blk * blk_stride + (size_t)(t0 & bs_mask) * RB;
        const uint8_t* kb = kc_head + boff;
        const uint8_t* vb = vc_head + boff;

        u32x4 kr[NLD], vr[NLD];
        bool valid[NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          // non-temporal: K/V are streamed once per step; not allocating them
          // in the caches measured 12% faster than default loads on this path
          kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + lane_off + i * RPL * RB));
          vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + lane_off + i * RPL * RB));
          valid[i] = full || (t0 + i * RPL + r < L);
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
          for (int x = 0; x < W; ++x) {
            if constexpr (FP8)
              kw[x] = fp8x2_to_f16x2<FMT>(kr[i][x / 2], x & 1);
            else
              kw[x] = kr[i][x];
          }
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float s = 0.0f;
#pragma unroll
            for (int x = 0; x < W; ++x) s = dot2(qf[g][x], kw[x], s);
            s = group_sum<LPR>(s);
            z[i][g] = valid[i] ? s * qk_scale : -INFINITY;
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
          for (int x = 0; x < W; ++x) {
            uint32_t pw;
            if constexpr (FP8)
              pw = fp8x2_to_f16x2<FMT>(vr[i][x / 2], x & 1);
            else
              pw = vr[i][x];
            vf[2 * x] = h_lo(pw);
            vf[2 * x + 1] = h_hi(pw);
          }
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < E; ++e) acc[g][e] = fmaf(p[i][g], vf[e], acc[g][e]);
        }
      }
    }

    // merge the RPL row states (lanes with equal c hold equal output slices)
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

    // the whole segment -> output; part of one -> this worker's slot
    const bool whole = pc.u0 == 0 && pc.u1 == pc.n_u;
    const int slot = t == start ? 0 : 1;
    if (lane < LPR) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (whole) {
          const float sc = l[g] > 0.0f ? v_scale / l[g] : 0.0f;
          f16* o = a.out + ((size_t)seq * a.Hq + hq0 + g) * D + c * E;
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = (f16)(acc[g][e] * sc);
        } else {
          const size_t pi = ((size_t)w * 2 + slot) * G + g;
          float* o = a.ws_o + pi * D + c * E;
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = acc[g][e] * v_scale;
          if (lane == 0) {
            a.ws_ml[2 * pi] = m[g];
            a.ws_ml[2 * pi + 1] = l[g];
          }
        }
      }
    }
    t = pc.next_t;
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

// Online-softmax state of one output row in a wave: max M (log2 units), sum
// l, and the lane's DL output elements, unnormalised, relative to M.
template <int DL>
struct Row {
  float M = -INFINITY;
  float l = 0.0f;
  float acc[DL] = {};
};

// Folds one partial state (max m, sum l, the lane's DL output elements o,
// relative to m) into r.
template <int DL>
__device__ __forceinline__ void fold(Row<DL>& r, float m, float l, const float* o) {
  const float Mn = fmaxf(r.M, m);
  const float Ms = safe_max(Mn);
  const float a1 = fast_exp2(r.M - Ms);
  const float a2 = fast_exp2(m - Ms);
  r.l = r.l * a1 + l * a2;
#pragma unroll
  for (int e = 0; e < DL; ++e) r.acc[e] = r.acc[e] * a1 + o[e] * a2;
  r.M = Mn;
}

// The lane's DL elements of the output rows of pieces j0 .. j0+NB-1 of a
// batch of nk <= 64 pieces, lane j holding the start of piece j's row (any
// readable address for a piece that adds nothing); past nk, the last piece
// again. Rows are fp32 (unnormalised partials) or fp16 (partials divided by
// their own sum), widened to fp32 here.
template <int DL, int NB>
struct RowBatch {
  float v[NB][DL];
};
template <int DL, int NB, typename T>
__device__ __forceinline__ RowBatch<DL, NB> load_rows(const T* row, int j0, int nk) {
  const int lane = threadIdx.x & 63;
  const uint64_t rp = reinterpret_cast<uint64_t>(row);
  RowBatch<DL, NB> b;
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int j = min(j0 + u, nk - 1);
    const uint64_t pj = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(rp >> 32), j) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)rp, j);
    const T* oj = reinterpret_cast<const T*>(pj) + lane * DL;
#pragma unroll
    for (int e = 0; e < DL; ++e) b.v[u][e] = (float)oj[e];
  }
  return b;
}

// acc += the rows of b weighted by lane j's wgt for piece j0 + u, in piece
// order (a weight of 0: no piece, or one that underflowed, adds nothing)
template <int DL, int NB>
__device__ __forceinline__ void add_rows(float* acc, float wgt, const RowBatch<DL, NB>& b, int j0, int nk) {
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const float w = j0 + u < nk ? readlane_f32(wgt, min(j0 + u, nk - 1)) : 0.0f;
    if (w == 0.0f) continue;
#pragma unroll
    for (int e = 0; e < DL; ++e) acc[e] = fmaf(w, b.v[u][e], acc[e]);
  }
}

// Adds to acc (the lane's DL elements) the weighted output rows of nk <= 64
// pieces: lane j holds piece j's weight (0: no piece, nothing is added) and
// the start of its row (any readable address when the weight is 0). The rows
// of the first NB pieces come in `first`, loaded by the caller before it had
// the weights; the rest are loaded NB pieces at a time, so that their
// latencies overlap. The sum runs in piece order.
template <int DL, int NB, typename T>
__device__ __forceinline__ void sum_rows(float* acc, float wgt, const T* row, int nk,
                                         const RowBatch<DL, NB>& first) {
  add_rows<DL, NB>(acc, wgt, first, 0, nk);
  for (int j0 = NB; j0 < nk; j0 += NB) add_rows<DL, NB>(acc, wgt, load_rows<DL, NB>(row, j0, nk), j0, nk);
}

// Folds into r the pieces of the segment holding units [s0, s1) of a unit
// space of `total` units cut into W shares. The piece of worker w sits in
// slot 0 if it starts the worker's share, else in slot 1; a slot holds `cols`
// columns of D outputs in ws_o and (max, sum) in ws_ml, and the row is column
// `col`. Outputs of type float are unnormalised (relative to the max); of type
// f16 they are divided by the piece's sum, so a row then weighs sum times the
// max's factor. Pieces are taken 64 at a time (lane k: piece k of the batch),
// NB rows at a time, each batch folded into r; each lane owns D/64 outputs.
template <int D, typename T = float, int NB = 8>
__device__ void fold_pieces(Row<D / 64>& r, const T* ws_o, const float* ws_ml, int cols, int col,
                            int64_t s0, int64_t s1, int64_t total, int64_t W) {
  constexpr int DL = D / 64;
  constexpr bool kNormalised = !std::is_same<T, float>::value;
  const int lane = threadIdx.x & 63;
  if (s0 < 0 || s0 >= s1 || s1 > total) return;  // only inconsistent group entries get here
  // worker holding unit u: the largest w with share_start(w) <= u
  const int64_t wa = ((s0 + 1) * W - 1) / total;
  const int64_t wb = (s1 * W - 1) / total;
  const int np = (int)(wb - wa + 1);
  for (int k0 = 0; k0 < np; k0 += 64) {
    // every lane loads a slot of the buffers (past np, the last piece's), so
    // that the loads are unconditional and the row loads below do not wait
    // for them; lanes past np and empty shares then count as no piece
    const int k = k0 + lane;
    const int64_t wk = wa + min(k, np - 1);
    const int64_t st = share_start(wk, total, W);
    const bool live = k < np && share_start(wk + 1, total, W) != st;
    const int64_t pi = (wk * 2 + (st >= s0 ? 0 : 1)) * cols + col;
    const float m_ld = ws_ml[2 * pi];
    const float l_ld = ws_ml[2 * pi + 1];
    const T* row = ws_o + pi * D;
    const int nk = min(64, np - k0);
    const RowBatch<DL, NB> first = load_rows<DL, NB>(row, 0, nk);  // in flight while the weights are made
    __builtin_amdgcn_sched_barrier(0);  // keep the uses of m_ld and l_ld below the row loads
    const float m = live ? m_ld : -INFINITY;
    const float l = live ? l_ld : 0.0f;
    const float M = wave_max(m);
    const float wgt = m == -INFINITY ? 0.0f : fast_exp2(m - safe_max(M));
    float acc[DL];
#pragma unroll
    for (int e = 0; e < DL; ++e) acc[e] = 0.0f;
    sum_rows<DL, NB>(acc, kNormalised ? wgt * l : wgt, row, nk, first);
    fold(r, M, wave_sum(l * wgt), acc);
  }
}

// Writes r, normalised, to the lane's DL elements of an output row.
template <int DL>
__device__ __forceinline__ void write_row(const Row<DL>& r, f16* out) {
  const float inv = r.l > 0.0f ? 1.0f / r.l : 0.0f;
#pragma unroll
  for (int e = 0; e < DL; ++e) out[e] = (f16)(r.acc[e] * inv);
}

// Workers holding the first and last unit of the segment [s0, s1).
__device__ __forceinline__ bool held_whole(int64_t s0, int64_t s1, int64_t total, int64_t W) {
  return ((s0 + 1) * W - 1) / total == (s1 * W - 1) / total;
}

// Pass 2. One wave per (sequence, query head): combines the pieces of a
// segment that pass 1 split between workers; writes zeros for empty
// sequences.
template <int D, int G>
__global__ void __launch_bounds__(256) attn_reduce_kernel(AttnArgs a) {
  constexpr int DL = D / 64;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= a.B * a.Hq) return;
  const int lane = threadIdx.x & 63;
  const int seq = wid / a.Hq;
  const int hq = wid - seq * a.Hq;
  const int kvh = hq / G;
  const int g = hq - kvh * G;
  // the three prefix entries in one round trip
  const int p0 = a.ws_pt[seq];
  const int p1 = a.ws_pt[seq + 1];
  const int P = a.ws_pt[a.B];
  const int n_u = p1 - p0;
  f16* out = a.out + (size_t)wid * D + lane * DL;
  Row<DL> r;
  if (n_u > 0) {
    const int64_t total = (int64_t)a.Hkv * P;
    const int64_t s0 = (int64_t)kvh * P + p0;  // the segment's units: [s0, s1)
    if (held_whole(s0, s0 + n_u, total, a.workers)) return;  // written by pass 1
    // the matrix-core pass (G >= 4) leaves its pieces as fp16 divided by their
    // sums; the vector pass as fp32 relative to their maxima
    if constexpr (G >= 4)
      fold_pieces<D, f16, 8>(r, reinterpret_cast<const f16*>(a.ws_o), a.ws_ml, G, g, s0, s0 + n_u, total,
                              a.workers);
    else
      fold_pieces<D>(r, a.ws_o, a.ws_ml, G, g, s0, s0 + n_u, total, a.workers);
  }
  write_row(r, out);
}

}  // namespace
}  // namespace pkv

#include "attn_gqa_mfma.hpp"
#include "attn_group_mfma.hpp"

namespace pkv {
namespace {

typedef void (*KernFn)(AttnArgs);

// Events that the next pass-1 launch of this thread records as its own start
// and stop (pkv_time_next_pass1); null when not armed.
thread_local hipEvent_t g_pass1_start = nullptr;
thread_local hipEvent_t g_pass1_stop = nullptr;

// A pass-1 launch: through hipExtLaunchKernel with the armed events (which
// it consumes), else an ordinary launch. Returns the launch's status.
hipError_t launch_pass1(KernFn fn, dim3 grid, dim3 block, uint32_t lds, hipStream_t s, const AttnArgs& a) {
  if (g_pass1_start) {
    hipEvent_t e0 = g_pass1_start, e1 = g_pass1_stop;
    g_pass1_start = g_pass1_stop = nullptr;
    hipExtLaunchKernelGGL(fn, grid, block, lds, s, e0, e1, 0u, a);
  } else {
    hipLaunchKernelGGL(fn, grid, block, lds, s, a);
  }
  return hipGetLastError();
}

template <int D, int FMT>
KernFn pick_partition_kernel(int G) {
  switch (G) {
    case 1: return attn_partition_kernel<D, 1, FMT, kWaves>;
    case 2: return attn_partition_kernel<D, 2, FMT, kWaves>;
    case 4: return attn_partition_mfma_kernel<D, 4, FMT, kWaves>;
    case 8: return attn_partition_mfma_kernel<D, 8, FMT, kWaves>;
    default: return nullptr;
  }
}

template <int D>
KernFn pick_fmt(int G, int fmt) {
  switch (fmt) {
    case kF16: return pick_partition_kernel<D, kF16>(G);
    case kE4M3: return pick_partition_kernel<D, kE4M3>(G);
    case kE5M2: return pick_partition_kernel<D, kE5M2>(G);
    default: return nullptr;
  }
}

KernFn pick(int D, int G, int fmt) {
  if (D == 64) return pick_fmt<64>(G, fmt);
  if (D == 128) return pick_fmt<128>(G, fmt);
  return nullptr;
}

template <int D>
KernFn pick_reduce_d(int G) {
  switch (G) {
    case 1: return attn_reduce_kernel<D, 1>;
    case 2: return attn_reduce_kernel<D, 2>;
    case 4: return attn_reduce_kernel<D, 4>;
    case 8: return attn_reduce_kernel<D, 8>;
    default: return nullptr;
  }
}

KernFn pick_reduce(int D, int G) {
  if (D == 64) return pick_reduce_d<64>(G);
  if (D == 128) return pick_reduce_d<128>(G);
  return nullptr;
}

template <int D>
KernFn pick_reduce_group_d(int G) {
  switch (G) {
    case 1: return attn_reduce_group_kernel<D, 1>;
    case 2: return attn_reduce_group_kernel<D, 2>;
    case 4: return attn_reduce_group_kernel<D, 4>;
    case 8: return attn_reduce_group_kernel<D, 8>;
    default: return nullptr;
  }
}

template <int D>
KernFn pick_group_d(int fmt) {
  switch (fmt) {
    case kF16: return attn_group_mfma_kernel<D, kF16, kWaves>;
    case kE4M3: return attn_group_mfma_kernel<D, kE4M3, kWaves>;
    case kE5M2: return attn_group_mfma_kernel<D, kE5M2, kWaves>;
    default: return nullptr;
  }
}

// (grouped pass 1, merge) kernels of paged_attn_decode_shared
bool pick_group(int D, int G, int fmt, KernFn* pass1, KernFn* reduce) {
  *pass1 = D == 64 ? pick_group_d<64>(fmt) : D == 128 ? pick_group_d<128>(fmt) : nullptr;
  *reduce = D == 64 ? pick_reduce_group_d<64>(G) : D == 128 ? pick_reduce_group_d<128>(G) : nullptr;
  return *pass1 && *reduce;
}

int log2_exact(int v) {
  int k = 0;
  while ((1 << k) < v) ++k;
  return (1 << k) == v ? k : -1;
}

int unit_tokens_for(int group) { return group >= 4 ? 32 : kTile; }

// pt[B + 1] and scan[blockDim]; the grouped pass 1 adds the part records [B]
size_t dyn_lds_bytes(int B, bool groups = false) {
  return (size_t)(B + 1 + kWaves * 64 + (groups ? B : 0)) * sizeof(int);
}

// Workgroups of a pass-1 kernel that can be resident at once on the current
// device (occupancy x compute units) and the compute-unit count, cached per
// (kernel, LDS size, device); false on error.
bool device_capacity(KernFn fn, size_t dyn_lds, int* resident_wgs, int* cus) {
  struct Entry {
    KernFn fn;
    size_t lds;
    int dev;
    int wgs;
    int cus;
  };
  static std::mutex mu;
  static Entry cache[128];
  static int n_cache = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n_cache; ++i)
    if (cache[i].fn == fn && cache[i].lds == dyn_lds && cache[i].dev == dev) {
      *resident_wgs = cache[i].wgs;
      *cus = cache[i].cus;
      return true;
    }
  int per_cu = 0, n_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), kWaves * 64,
                                                   dyn_lds) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return false;
  if (n_cache < 128) cache[n_cache++] = Entry{fn, dyn_lds, dev, per_cu * n_cu, n_cu};
  *resident_wgs = per_cu * n_cu;
  *cus = n_cu;
  return per_cu > 0 && n_cu > 0;
}

// Default workers per SIMD. The SIMD issues for its resident waves in slot
// order, so with several streaming waves per SIMD the low slots run ahead and
// an equal share per wave leaves the last slots finishing long after the first
// (measured on MI355X with 7 waves per SIMD: median finish 65 us for slot 0 vs
// 182 us for slot 6). One wave per SIMD removes that skew and still keeps
// enough loads in flight when a tile's arithmetic is light (fp16, one query
// head per KV head: pass 1 of the Llama-2-7B batch-64 workload went from 201
// to 185 us); heavier tiles (grouped heads, fp8 widening, matrix cores) need a
// second wave per SIMD to overlap arithmetic with loads.
int waves_per_simd(int group, bool fp8) { return group == 1 && !fp8 ? 1 : 2; }

// Units of B sequences of the longest context the block table can hold.
int64_t unit_upper_bound(int B, int max_blocks, int block_size, int unit) {
  const int64_t lmax = (int64_t)max_blocks * block_size;
  return (int64_t)B * ((lmax + unit - 1) / unit);
}

// Head groups for W workers over Hkv KV heads (worker_index) on a batch that
// shares no blocks: W / Hkv, or 0 (one slice of the unit space per wave) when
// W is not a multiple of Hkv or when the slice of a block that one XCD reads
// in head-major order -- Hkv / 8 heads side by side, head_bytes each -- is
// already 32 KiB or more. Measured on MI355X: Llama-2-7B layer (16 KiB per
// XCD per block) pass 1 186 us with head groups against 189 us; OPT-13B layer
// (40 KiB) 1156 us against 1151 us.
int head_groups_for(int W, int Hkv, size_t head_bytes) {
  if (Hkv <= 0 || W % Hkv != 0) return 0;
  const size_t slice = (size_t)((Hkv + 7) / 8) * head_bytes;
  return slice < 32768 ? W / Hkv : 0;
}

struct Plan {
  KernFn fn;
  KernFn reduce;
  int unit;
  int workers;  // for a launch of kMaxSeqs sequences or fewer
};

// Validates the shape and picks the kernels and the worker count; returns a
// status code.
int plan(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
         int max_blocks_per_seq, int kv_dtype, int partition_tokens, bool need_workers, Plan* p) {
  if (num_seqs < 0 || num_kv_heads <= 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0)
    return PKV_ERR_INVALID;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_INVALID;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_INVALID;
  if (block_size != 16 && block_size != 32 && block_size != 64) return PKV_ERR_INVALID;
  if (kv_dtype != PKV_KV_F16 && kv_dtype != PKV_KV_FP8_E4M3 && kv_dtype != PKV_KV_FP8_E5M2)
    return PKV_ERR_INVALID;
  if (partition_tokens < 0 || partition_tokens % kTile != 0) return PKV_ERR_INVALID;
  const int G = num_q_heads / num_kv_heads;
  p->fn = pick(head_dim, G, kv_dtype);
  p->reduce = pick_reduce(head_dim, G);
  if (!p->fn || !p->reduce) return PKV_ERR_INVALID;
  p->unit = unit_tokens_for(G);
  const int B = num_seqs < kMaxSeqs ? num_seqs : kMaxSeqs;
  // unit counts and prefixes are int32 on the device
  const int64_t ub = unit_upper_bound(B, max_blocks_per_seq, block_size, p->unit);
  if ((int64_t)max_blocks_per_seq * block_size > 0x7FFFFFFF || ub > 0x7FFFFFFF) return PKV_ERR_INVALID;
  p->workers = 0;
  if (!need_workers || B == 0) return PKV_OK;
  const int64_t ub_all = ub * num_kv_heads;
  int64_t W;
  if (partition_tokens > 0) {
    const int64_t per = (partition_tokens + p->unit - 1) / p->unit;
    W = (ub_all + per - 1) / per;
  } else {
    int wgs = 0, cus = 0;
    if (!device_capacity(p->fn, dyn_lds_bytes(B), &wgs, &cus)) return PKV_ERR_HIP;
    W = (int64_t)wgs * kWaves;
    const int64_t by_simd = (int64_t)waves_per_simd(G, kv_dtype != PKV_KV_F16) * 4 * cus;
    if (W > by_simd) W = by_simd;
    // a multiple of Hkv where that keeps whole workgroups and loses under 1/16
    // of the workers: the shares then fall on KV-head boundaries, which
    // head groups need (worker_index)
    const int64_t Wh = W / num_kv_heads * num_kv_heads;
    if (Wh % kWaves == 0 && Wh * 16 >= W * 15) W = Wh;
  }
  if (W > ub_all) W = ub_all;
  if (W > kMaxWorkers) W = kMaxWorkers;
  if (W < 1) W = 1;
  W = (W + kWaves - 1) / kWaves * kWaves;  // every wave of the grid is a worker
  p->workers = (int)W;
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

extern "C" int paged_attn_decode_workers(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                         int block_size, int max_blocks_per_seq, int kv_dtype,
                                         int partition_tokens) {
  pkv::Plan p;
  if (num_seqs <= 0) return PKV_ERR_INVALID;
  const int rc = pkv::plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                           kv_dtype, partition_tokens, true, &p);
  return rc == PKV_OK ? p.workers : rc;
}

extern "C" size_t paged_attn_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                                    int head_dim, int max_blocks_per_seq,
                                                    int block_size, int partition_tokens) {
  (void)max_blocks_per_seq;
  (void)block_size;
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return 0;
  if (head_dim != 64 && head_dim != 128) return 0;
  if (partition_tokens < 0 || partition_tokens % pkv::kTile != 0) return 0;
  const int G = num_q_heads / num_kv_heads;
  const int b = num_seqs < pkv::kMaxSeqs ? num_seqs : pkv::kMaxSeqs;
  const size_t pieces = (size_t)pkv::kMaxWorkers * 2 * G;
  const size_t bytes = pieces * (size_t)(head_dim + 2) * sizeof(float) + (size_t)(b + 1) * sizeof(int32_t);
  return (bytes + 255) / 256 * 256;
}

namespace pkv {
namespace {

// Workspace of paged_attn_decode_shared, byte offsets of its regions (each
// 256-byte aligned): the grouped pass 1's slots ([kMaxGroupWorkers][2]
// [kGroupCols] columns of D fp16 outputs, then of fp32 (max, sum)), the unit prefix
// over the sequences, their part records and their parts' unit ranges.
// Without groups the call is
// paged_attn_decode's, so the total also covers that workspace.
struct GroupLayout {
  size_t o, ml, pt, part, seg, total;
};

GroupLayout group_layout(int B, int Hq, int Hkv, int D) {
  GroupLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = (off + bytes + 255) / 256 * 256;
    return at;
  };
  const size_t cols = (size_t)kMaxGroupWorkers * 2 * kGroupCols;
  L.o = take(cols * D * sizeof(f16));  // fp16, each divided by its piece's sum
  L.ml = take(cols * 2 * sizeof(float));
  L.pt = take((size_t)(B + 1) * sizeof(int32_t));
  L.part = take((size_t)B * sizeof(int32_t));
  L.seg = take((size_t)B * 2 * sizeof(int32_t));
  const size_t plain = paged_attn_decode_workspace_bytes(B, Hq, Hkv, D, 1, 16, 0);
  L.total = off > plain ? off : plain;
  return L;
}

// Workers of the grouped pass 1: group_waves_per_simd per SIMD (one for fp16,
// two for fp8), within
// what the device holds at once; with partition_tokens, about that
// many tokens each of the largest unit space the batch can describe (every
// sequence's tail plus a part's shared units, each at most the table width,
// and a part's setup charge).
int group_workers(KernFn fn, int B, int Hkv, int max_blocks, int block_size, int kv_dtype, int partition_tokens,
                  int* W_out) {
  const int64_t max_units = ((int64_t)max_blocks * block_size + 31) / 32;
  const int64_t ub = (int64_t)Hkv * B * (2 * max_units + kPieceCost);
  int64_t W;
  if (partition_tokens > 0) {
    const int64_t per = (partition_tokens + 31) / 32;
    W = (ub + per - 1) / per;
  } else {
    int wgs = 0, cus = 0;
    if (!device_capacity(fn, dyn_lds_bytes(B, true), &wgs, &cus)) return PKV_ERR_HIP;
    W = (int64_t)wgs * kWaves;
    const int per_simd = kv_dtype == PKV_KV_F16 ? group_waves_per_simd<kF16>() : group_waves_per_simd<kE4M3>();
    const int64_t by_simd = (int64_t)per_simd * 4 * cus;
    if (W > by_simd) W = by_simd;
  }
  if (W > ub) W = ub;
  if (W > kMaxGroupWorkers) W = kMaxGroupWorkers;
  if (W < kWaves) W = kWaves;
  *W_out = (int)(W / kWaves * kWaves);
  return PKV_OK;
}

// Bytes of pass-1 partials and unit prefix for W workers: [W][2][G][D] outputs,
// [W][2][G][2] (max, sum), then [B + 1] ints, each region 256-byte aligned.
// paged_attn_decode lays them out for kMaxWorkers workers, so that its
// workspace size does not depend on the device; the allocation-free call
// for the workers it actually launches.
struct DecodeLayout {
  size_t o, ml, pt, total;
};

DecodeLayout decode_layout(int W, int G, int D, int B) {
  DecodeLayout L;
  const size_t pieces = (size_t)W * 2 * G;
  L.o = 0;
  L.ml = (pieces * D * sizeof(float) + 255) / 256 * 256;
  L.pt = L.ml + (pieces * 2 * sizeof(float) + 255) / 256 * 256;
  L.total = L.pt + ((size_t)(B + 1) * sizeof(int32_t) + 255) / 256 * 256;
  return L;
}

// compact_ws: partials laid out for the workers launched (decode_layout with
// the plan's worker count) instead of kMaxWorkers.
int decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                int max_blocks_per_seq, const int32_t* ctx_lens, int num_seqs, int num_q_heads, int num_kv_heads,
                int head_dim, int block_size, int num_blocks, float sm_scale, int kv_dtype, float k_scale,
                float v_scale, const float* k_scales, const float* v_scales, int partition_tokens,
                void* workspace, size_t workspace_bytes, int passes, void* stream, bool compact_ws = false,
                bool disjoint = false) {
  if (passes < 1 || passes > 3 || num_blocks <= 0) return PKV_ERR_INVALID;
  Plan pl;
  int rc = plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, kv_dtype,
                partition_tokens, false, &pl);
  if (rc != PKV_OK) return rc;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !ctx_lens) return PKV_ERR_INVALID;
  if (!vec_aligned(out) || !vec_aligned(q) || !vec_aligned(k_cache) || !vec_aligned(v_cache) ||
      !vec_aligned(workspace) || !aligned_to(block_tables, 4) || !aligned_to(ctx_lens, 4) ||
      !aligned_to(k_scales, 4) || !aligned_to(v_scales, 4))
    return PKV_ERR_INVALID;
  const int G = num_q_heads / num_kv_heads;
  DecodeLayout lay{};
  if (!compact_ws) {
    const size_t need = paged_attn_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                          max_blocks_per_seq, block_size, partition_tokens);
    if (!workspace || workspace_bytes < need) return PKV_ERR_INVALID;
  }
  rc = plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, kv_dtype,
            partition_tokens, true, &pl);
  if (rc != PKV_OK) return rc;
  if (compact_ws) {
    lay = decode_layout(pl.workers, G, head_dim, num_seqs < kMaxSeqs ? num_seqs : kMaxSeqs);
    if (!workspace || workspace_bytes < lay.total) return PKV_ERR_INVALID;
  }

  const bool fp8 = kv_dtype != PKV_KV_F16;
  const float kLog2e = 1.4426950408889634f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // more than kMaxSeqs sequences: consecutive launches, in order on the stream
  for (int b0 = 0; b0 < num_seqs; b0 += kMaxSeqs) {
    const int B = num_seqs - b0 < kMaxSeqs ? num_seqs - b0 : kMaxSeqs;
    AttnArgs a;
    a.q = static_cast<const f16*>(q) + (size_t)b0 * num_q_heads * head_dim;
    a.kc = static_cast<const uint8_t*>(k_cache);
    a.vc = static_cast<const uint8_t*>(v_cache);
    a.tables = block_tables + (size_t)b0 * max_blocks_per_seq;
    a.ctx_lens = ctx_lens + b0;
    if (compact_ws) {
      uint8_t* ws = static_cast<uint8_t*>(workspace);
      a.ws_o = reinterpret_cast<float*>(ws + lay.o);
      a.ws_ml = reinterpret_cast<float*>(ws + lay.ml);
      a.ws_pt = reinterpret_cast<int32_t*>(ws + lay.pt);
    } else {
      a.ws_o = static_cast<float*>(workspace);
      a.ws_ml = a.ws_o + (size_t)kMaxWorkers * 2 * G * head_dim;
      a.ws_pt = reinterpret_cast<int32_t*>(a.ws_ml + (size_t)kMaxWorkers * 2 * G * 2);
    }
    a.out = static_cast<f16*>(out) + (size_t)b0 * num_q_heads * head_dim;
    a.max_blocks = max_blocks_per_seq;
    a.B = B;
    a.Hkv = num_kv_heads;
    a.Hq = num_q_heads;
    a.bs_log2 = log2_exact(block_size);
    a.num_blocks = num_blocks;
    a.unit_tokens = pl.unit;
    a.workers = pl.workers;
    a.head_groups = disjoint ? head_groups_for(pl.workers, num_kv_heads,
                                               (size_t)block_size * head_dim * (fp8 ? 1 : 2))
                             : 0;
    a.qk_scale = sm_scale * kLog2e * (fp8 ? k_scale : 1.0f);
    a.v_out_scale = fp8 ? v_scale : 1.0f;
    a.k_scale_h = fp8 ? k_scales : nullptr;
    a.v_scale_h = fp8 ? v_scales : nullptr;
    a.qk_base = sm_scale * kLog2e;
    if (passes & 1) {
      if (launch_pass1(pl.fn, dim3((unsigned)(pl.workers / kWaves)), dim3(kWaves * 64),
                       (uint32_t)dyn_lds_bytes(B), s, a) != hipSuccess)
        return PKV_ERR_HIP;
    }
    if (passes & 2) {
      const int waves = B * num_q_heads;
      hipLaunchKernelGGL(pl.reduce, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a);
      if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
    }
  }
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

extern "C" int paged_attn_decode_passes(void* out, const void* q, const void* k_cache,
                                        const void* v_cache, const int32_t* block_tables,
                                        int max_blocks_per_seq, const int32_t* ctx_lens,
                                        int num_seqs, int num_q_heads, int num_kv_heads,
                                        int head_dim, int block_size, int num_blocks,
                                        float sm_scale, int kv_dtype, float k_scale,
                                        float v_scale, int partition_tokens, void* workspace,
                                        size_t workspace_bytes, int passes, void* stream) {
  return pkv::decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, ctx_lens, num_seqs,
                          num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, sm_scale, kv_dtype,
                          k_scale, v_scale, nullptr, nullptr, partition_tokens, workspace, workspace_bytes,
                          passes, stream);
}

extern "C" int paged_attn_decode_scaled(void* out, const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables, int max_blocks_per_seq,
                                        const int32_t* ctx_lens, int num_seqs, int num_q_heads,
                                        int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                        float sm_scale, int kv_dtype, const float* k_scales,
                                        const float* v_scales, int partition_tokens, void* workspace,
                                        size_t workspace_bytes, int passes, void* stream) {
  if (kv_dtype != PKV_KV_F16 && num_seqs > 0 && (!k_scales || !v_scales)) return PKV_ERR_INVALID;
  return pkv::decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, ctx_lens, num_seqs,
                          num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, sm_scale, kv_dtype,
                          1.0f, 1.0f, k_scales, v_scales, partition_tokens, workspace, workspace_bytes, passes,
                          stream);
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

// ---------------------------------------------------------------------------
// Allocation-free decode: the pass-1 partials live in a file-scope device
// array instead of a caller workspace. Each device holds its own copy of the
// array (for the life of the process); its address on a device is looked up
// once, with that device current, and kept.

namespace pkv {
namespace {

constexpr size_t kNoAllocBytes = PKV_DECODE_NOALLOC_SCRATCH_BYTES;
constexpr int kNoAllocDevices = 64;

__device__ __align__(256) uint8_t scratch[kNoAllocBytes];

// The device address of `scratch` on the current device, or null on error.
void* scratch_ptr() {
  static std::mutex mu;
  static void* ptrs[kNoAllocDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

}  // namespace
}  // namespace pkv

extern "C" int paged_attn_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_tables, int max_blocks_per_seq,
                                         const int32_t* ctx_lens, int num_seqs, int num_q_heads,
                                         int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                         float sm_scale, int kv_dtype, float k_scale, float v_scale,
                                         int partition_tokens, void* stream) {
  using namespace pkv;
  // shape errors first (no device query), then the scratch address
  Plan pl;
  int rc = plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, kv_dtype,
                partition_tokens, false, &pl);
  if (rc != PKV_OK) return rc;
  if (num_seqs == 0) return PKV_OK;
  void* ws = scratch_ptr();
  if (!ws) return PKV_ERR_HIP;
  return decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, ctx_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, sm_scale, kv_dtype, k_scale, v_scale, nullptr,
                     nullptr, partition_tokens, ws, kNoAllocBytes, 3, stream, true);
}

extern "C" size_t paged_attn_decode_shared_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                                           int head_dim) {
  if (num_seqs <= 0 || num_seqs > pkv::kMaxSeqs || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0)
    return 0;
  if (head_dim != 64 && head_dim != 128) return 0;
  return pkv::group_layout(num_seqs, num_q_heads, num_kv_heads, head_dim).total;
}

extern "C" int paged_attn_decode_shared(void* out, const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables, int max_blocks_per_seq,
                                        const int32_t* ctx_lens, int num_seqs, int num_q_heads,
                                        int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                        float sm_scale, int kv_dtype, float k_scale, float v_scale,
                                        const float* k_scales, const float* v_scales,
                                        const int32_t* group_first, const int32_t* group_size,
                                        const int32_t* group_prefix, int num_groups, int partition_tokens,
                                        void* workspace, size_t workspace_bytes, int passes, void* stream) {
  using namespace pkv;
  if (passes < 1 || passes > 7 || num_blocks <= 0 || num_seqs > kMaxSeqs) return PKV_ERR_INVALID;
  if (num_groups < 0 || num_groups > (num_seqs > 0 ? num_seqs : 0)) return PKV_ERR_INVALID;
  if ((k_scales == nullptr) != (v_scales == nullptr)) return PKV_ERR_INVALID;
  Plan pl;
  int rc = plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, kv_dtype,
                partition_tokens, false, &pl);
  if (rc != PKV_OK) return rc;
  const int G = num_q_heads / num_kv_heads;
  KernFn group_fn, reduce_fn;
  if (!pick_group(head_dim, G, kv_dtype, &group_fn, &reduce_fn)) return PKV_ERR_INVALID;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !ctx_lens) return PKV_ERR_INVALID;
  if (num_groups > 0 && (!group_first || !group_size || !group_prefix)) return PKV_ERR_INVALID;
  if (!vec_aligned(out) || !vec_aligned(q) || !vec_aligned(k_cache) || !vec_aligned(v_cache) ||
      !vec_aligned(workspace) || !aligned_to(block_tables, 4) || !aligned_to(ctx_lens, 4) ||
      !aligned_to(k_scales, 4) || !aligned_to(v_scales, 4) || !aligned_to(group_first, 4) ||
      !aligned_to(group_size, 4) || !aligned_to(group_prefix, 4))
    return PKV_ERR_INVALID;
  const GroupLayout lay = group_layout(num_seqs, num_q_heads, num_kv_heads, head_dim);
  if (!workspace || workspace_bytes < lay.total) return PKV_ERR_INVALID;
  const bool fp8 = kv_dtype != PKV_KV_F16;
  const bool per_head = fp8 && k_scales != nullptr;
  // No groups: the batch is declared to share no blocks. paged_attn_decode's
  // kernels, shares and sums (the same bits), with the waves dealt in head
  // groups (worker_index): no block is read by two sequences, so nothing is
  // lost by spreading a block's KV heads over one XCD instead of giving each
  // XCD a few heads of every sequence.
  if (num_groups == 0) {
    const int p = ((passes & 3) ? 1 : 0) | ((passes & 4) ? 2 : 0);
    return decode_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, ctx_lens, num_seqs,
                       num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, sm_scale, kv_dtype, k_scale,
                       v_scale, per_head ? k_scales : nullptr, per_head ? v_scales : nullptr, partition_tokens,
                       workspace, workspace_bytes, p, stream, false, true);
  }
  // every unit of the batch (tail, shared units and setup charge of one part
  // per sequence at most) must fit the int32 prefix
  if ((int64_t)num_seqs * (2 * (((int64_t)max_blocks_per_seq * block_size + 31) / 32) + kPieceCost) > 0x7FFFFFFF)
    return PKV_ERR_INVALID;
  int W = kWaves;
  rc = group_workers(group_fn, num_seqs, num_kv_heads, max_blocks_per_seq, block_size, kv_dtype, partition_tokens,
                     &W);
  if (rc != PKV_OK) return rc;

  const float kLog2e = 1.4426950408889634f;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  AttnArgs a;
  a.q = static_cast<const f16*>(q);
  a.kc = static_cast<const uint8_t*>(k_cache);
  a.vc = static_cast<const uint8_t*>(v_cache);
  a.tables = block_tables;
  a.ctx_lens = ctx_lens;
  a.ws_o = reinterpret_cast<float*>(ws + lay.o);
  a.ws_ml = reinterpret_cast<float*>(ws + lay.ml);
  a.ws_pt = reinterpret_cast<int32_t*>(ws + lay.pt);
  a.ws_part = reinterpret_cast<int32_t*>(ws + lay.part);
  a.ws_seg = reinterpret_cast<int32_t*>(ws + lay.seg);
  a.out = static_cast<f16*>(out);
  a.max_blocks = max_blocks_per_seq;
  a.B = num_seqs;
  a.Hkv = num_kv_heads;
  a.Hq = num_q_heads;
  a.bs_log2 = log2_exact(block_size);
  a.num_blocks = num_blocks;
  a.unit_tokens = 32;
  a.workers = W;
  a.qk_scale = sm_scale * kLog2e * (fp8 && !per_head ? k_scale : 1.0f);
  a.v_out_scale = fp8 && !per_head ? v_scale : 1.0f;
  a.k_scale_h = per_head ? k_scales : nullptr;
  a.v_scale_h = per_head ? v_scales : nullptr;
  a.qk_base = sm_scale * kLog2e;
  a.grp_first = group_first;
  a.grp_size = group_size;
  a.grp_prefix = group_prefix;
  a.NG = num_groups;
  a.g_log2 = log2_exact(G);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (passes & 3) {
    if (launch_pass1(group_fn, dim3((unsigned)(W / kWaves)), dim3(kWaves * 64),
                     (uint32_t)dyn_lds_bytes(num_seqs, true), s, a) != hipSuccess)
      return PKV_ERR_HIP;
  }
  if (passes & 4) {
    const int waves = num_seqs * num_q_heads;
    hipLaunchKernelGGL(reduce_fn, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  }
  return PKV_OK;
}

extern "C" int pkv_time_next_pass1(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr)) return PKV_ERR_INVALID;
  pkv::g_pass1_start = static_cast<hipEvent_t>(start_event);
  pkv::g_pass1_stop = static_cast<hipEvent_t>(stop_event);
  return PKV_OK;
}
