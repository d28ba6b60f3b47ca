// paged_attn_prefill: chunked (multi-token, causal) attention over the paged
// KV cache, on the matrix cores of gfx950.
//
// A request whose leading blocks were found in the prefix cache maps them into
// its block table and prefills only the positions that missed ("Where Did the
// VRAM Go (KV cache tutorial)", §4.2); a prompt cut into chunks does the same
// chunk by chunk. Sequence s holds ctx_lens[s] = L tokens, reached through its
// block table as in decode ("From OOM to Smooth Inference (RAG memory
// management)", §2.1); its n query rows q[q_start[s] .. q_start[s+1]) are the
// last n positions of the context, and row i (position p = L - n + i) attends
// over positions 0..p.
//
// Work decomposition. A workgroup (4 waves) owns one tile: 128 query columns
// of one (sequence, KV head), where a column is one (query token, query head)
// pair of that KV head's group of G heads -- 128 / G consecutive query tokens.
// Each wave holds 32 columns (two 16-column MFMA operands). The workgroup walks
// the tokens the tile can see, 32 at a time (two 16-token tiles, each inside
// one block): all 256 threads load the chunk's K and V rows from the cache
// into LDS as fp16 (fp8 rows, e4m3 or e5m2, widened exactly), double-buffered so that the
// next chunk's loads are in flight while this one is computed, and every wave
// then runs, per chunk:
//   S = K . Q^T       v_mfma_f32_16x16x32_f16, M = 16 tokens, N = 16 columns,
//                     K rows read from LDS in the A layout (no transpose)
//   online softmax    per column; the accumulator gives lane (column j,
//                     group g) tokens 4g..4g+3 of each tile, so the column's
//                     max and sum need only two cross-group shuffles
//   O^T += V^T . P^T  M = 16 head-dim rows, K-dim = the chunk's 32 tokens; the
//                     logits of both tiles are exactly the B operand P^T, and
//                     V^T comes from LDS through ds_read_b64_tr_b16
// The causal mask and the end of the sequence are applied to the logits (a
// masked logit is -inf); V rows past the sequence are zero in LDS.
//
// Tiles are numbered head-major (KV head h owns tiles [h T, (h+1) T)), and
// the workgroups that run on one XCD (g, g + 8, ...) take one contiguous range
// of that numbering, so the K/V of a (sequence, head) is read through one L2.
// Inside a head the tiles run in reverse order: the last tile of a sequence
// sees the longest context and starts first.
//
// Exponentials are base 2 with log2(e) folded into the logit scale.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pagedkv.h"
#include "device_common.hpp"

namespace pkv {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kCols = 32;                 // query columns per wave
constexpr int kNcg = kCols / 16;          // 16-column MFMA operands per wave
constexpr int kTileCols = kWaves * kCols; // query columns per workgroup
constexpr int kMinBlocks = 3;             // workgroups per compute unit the launch bound asks for
constexpr int kChunk = 32;                // tokens per step of the token loop
constexpr int kMaxSeqs = 4096;            // sequences per launch (tile prefix in LDS)
constexpr float kLazy = 8.0f;             // log2 headroom before the running max moves

struct PrefillArgs {
  const f16* q;
  const uint8_t* kc;
  const uint8_t* vc;
  const int32_t* tables;
  const int32_t* ctx_lens;
  const int32_t* q_start;
  f16* out;
  int max_blocks;
  int B;
  int Hkv;
  int Hq;
  int bs_log2;
  int num_blocks;
  int total_q;
  int tiles_bound;    // tiles per KV head the grid provides (>= the real count)
  float qk_scale;     // sm_scale * log2(e), times k_scale for fp8
  float v_out_scale;  // v_scale for fp8, else 1
  const float* k_scale_h;  // one scale per KV head (device), or null: qk_scale / v_out_scale hold
  const float* v_scale_h;
  float qk_base;           // sm_scale * log2(e)
};

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float safe_max(float m) { return m == -INFINITY ? 0.0f : m; }

// max of three floats in one v_max3_f32. fmaxf on matrix-core results costs
// two extra instructions per call: the compiler first quiets possible
// signalling NaNs, which these logits never are.
__device__ __forceinline__ float max3_f32(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// A float the caller knows is equal on all lanes, moved to a scalar register.
__device__ __forceinline__ float uniform_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// Query rows of sequence s: [first, first + count), or none if q_start puts
// them outside [0, total_q).
__device__ __forceinline__ void seq_rows(const PrefillArgs& a, int s, int* first, int* count) {
  const int r0 = a.q_start[s];
  const int r1 = a.q_start[s + 1];
  const bool ok = r0 >= 0 && r1 >= r0 && r1 <= a.total_q;
  *first = ok ? r0 : 0;
  *count = ok ? r1 - r0 : 0;
}

// pt[0] = 0, pt[s + 1] = pt[s] + tiles of sequence s, in LDS; scan[] is
// blockDim.x ints of scratch. Ends with a barrier.
__device__ void build_tile_prefix(const PrefillArgs& a, int G, int* pt, int* scan) {
  const int n = a.B;
  const int T = blockDim.x;
  const int tid = threadIdx.x;
  for (int i = tid; i < n; i += T) {
    int first, count;
    seq_rows(a, i, &first, &count);
    pt[i + 1] = (count * G + kTileCols - 1) / kTileCols;
  }
  __syncthreads();
  const int per = (n + T - 1) / T;
  const int b0 = min(n, tid * per);
  const int b1 = min(n, b0 + per);
  int s = 0;
  for (int i = b0; i < b1; ++i) s += pt[i + 1];
  scan[tid] = s;
  __syncthreads();
  for (int off = 1; off < T; off <<= 1) {
    const int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  int run = scan[tid] - s;
  for (int i = b0; i < b1; ++i) {
    run += pt[i + 1];
    pt[i + 1] = run;
  }
  if (tid == 0) pt[0] = 0;
  __syncthreads();
}

// The sequence that owns tile t (< pt[B]): the last s with pt[s] <= t.
__device__ __forceinline__ int find_seq(const int* pt, int B, int t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pt[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Workgroup g runs on XCD g % 8; workgroups g, g + 8, ... get consecutive
// logical indices, so each XCD takes one contiguous range of tiles.
__device__ __forceinline__ int logical_index() {
  const int n = gridDim.x;
  const int xcd = blockIdx.x % 8;
  const int q = n / 8, r = n % 8;
  return xcd * q + min(xcd, r) + (int)(blockIdx.x / 8);
}

// 8 fp8 bytes (two dwords) -> 8 fp16 values, exactly
template <int FMT>
__device__ __forceinline__ f16x8 fp8x8_to_f16x8(uint32_t w0, uint32_t w1) {
  u32x4 r;
  r[0] = fp8x2_to_f16x2<FMT>(w0, false);
  r[1] = fp8x2_to_f16x2<FMT>(w0, true);
  r[2] = fp8x2_to_f16x2<FMT>(w1, false);
  r[3] = fp8x2_to_f16x2<FMT>(w1, true);
  return __builtin_bit_cast(f16x8, r);
}

template <int D, bool FP8>
struct ChunkShape {
  static constexpr int ELEM = FP8 ? 1 : 2;
  static constexpr int RB = D * ELEM;                  // cache bytes of one token row
  static constexpr int LPR = RB / 16;                  // 16-byte pieces per row
  static constexpr int PIECES = kChunk * LPR;          // pieces per chunk, per tensor
  static constexpr int PPT = (PIECES + kWaves * 64 - 1) / (kWaves * 64);  // per thread
  static constexpr int HPP = 16 / ELEM;                // fp16 values per piece
  static constexpr int KS = D + 8;                     // LDS row stride of K, halves
  static constexpr int VS = D + 8;                     // LDS row stride of V, halves
  static constexpr int BUF = kChunk * (KS + VS);       // halves per buffer (K then V)
};

// The chunk's K and V pieces that this thread moves: global -> registers.
template <int D, int FMT>
struct Stage {
  static constexpr bool FP8 = FMT != kF16;
  using S = ChunkShape<D, FP8>;
  u32x4 k[S::PPT];
  u32x4 v[S::PPT];
  bool live[S::PPT];

  // Rows t0 .. t0+31 of the chunk: rows 0-15 live in block blk_a, rows 16-31
  // in blk_b (wave-uniform). Rows at or past `end`, or in a block outside the
  // pool, are loaded from the head's first rows instead and replaced by zeros.
  // The per-row offset within a 16-token tile is fixed per thread; only the
  // two tile bases change from chunk to chunk, and they are scalar.
  __device__ __forceinline__ void load(const PrefillArgs& a, int blk_a, int blk_b, const uint8_t* kc_head,
                                       const uint8_t* vc_head, size_t blk_stride, int t0, int end) {
    const int bsm = (1 << a.bs_log2) - 1;
    const bool oka = (unsigned)blk_a < (unsigned)a.num_blocks;
    const bool okb = (unsigned)blk_b < (unsigned)a.num_blocks;
    const size_t base_a = oka ? (size_t)blk_a * blk_stride + (size_t)(t0 & bsm) * S::RB : 0;
    const size_t base_b = okb ? (size_t)blk_b * blk_stride + (size_t)((t0 + 16) & bsm) * S::RB : 0;
#pragma unroll
    for (int i = 0; i < S::PPT; ++i) {
      const int p = threadIdx.x + i * kWaves * 64;
      const int r = p / S::LPR;
      const bool ok = p < S::PIECES && t0 + r < end && (r < 16 ? oka : okb);
      const uint32_t in_tile = (uint32_t)((r & 15) * S::RB + (p % S::LPR) * 16);
      const size_t off = (r < 16 ? base_a : base_b) + in_tile;
      // ordinary (cached) loads: every tile of the sequence reads these rows
      // the rows are zeroed at store time, so nothing here waits for the loads
      k[i] = *reinterpret_cast<const u32x4*>(kc_head + off);
      v[i] = *reinterpret_cast<const u32x4*>(vc_head + off);
      live[i] = ok;
    }
  }

  // registers -> LDS buffer as fp16 rows (rows past the end were loaded as zeros)
  __device__ __forceinline__ void store(_Float16* buf) const {
#pragma unroll
    for (int i = 0; i < S::PPT; ++i) {
      const int p = threadIdx.x + i * kWaves * 64;
      if (p >= S::PIECES) continue;
      const int r = p / S::LPR;
      const int h = (p % S::LPR) * S::HPP;
      _Float16* kd = buf + r * S::KS + h;
      _Float16* vd = buf + kChunk * S::KS + r * S::VS + h;
      const u32x4 kk = live[i] ? k[i] : u32x4{0u, 0u, 0u, 0u};
      const u32x4 vv = live[i] ? v[i] : u32x4{0u, 0u, 0u, 0u};
      if constexpr (FP8) {
        *reinterpret_cast<f16x8*>(kd) = fp8x8_to_f16x8<FMT>(kk[0], kk[1]);
        *reinterpret_cast<f16x8*>(kd + 8) = fp8x8_to_f16x8<FMT>(kk[2], kk[3]);
        *reinterpret_cast<f16x8*>(vd) = fp8x8_to_f16x8<FMT>(vv[0], vv[1]);
        *reinterpret_cast<f16x8*>(vd + 8) = fp8x8_to_f16x8<FMT>(vv[2], vv[3]);
      } else {
        *reinterpret_cast<u32x4*>(kd) = kk;
        *reinterpret_cast<u32x4*>(vd) = vv;
      }
    }
  }
};

// fp16 chunks staged straight from global memory into LDS (global_load_lds,
// 16 bytes per lane; lane i of a wave instruction lands in LDS slot i). The
// LDS layout is pair-major: for each pair p of 16-byte chunks of a row
// (halves 16p .. 16p + 15), the 32 rows of the chunk follow one another, 32
// bytes each: byte p * 1024 + r * 32 + 16 (c % 2) holds chunk c of row r. One
// instruction fills one pair for all 32 rows; the q.k and transposing V reads
// then differ only by immediate offsets between pairs, and a quarter-wave's K
// read touches each bank at most twice.
template <int D>
struct Direct {
  static constexpr int RB = D * 2;               // bytes of one fp16 row
  static constexpr int NP = D / 16;              // chunk pairs per row
  static constexpr int PAIR_HALVES = kChunk * 16;  // halves of one pair block (1 KiB)
  static constexpr int HALVES = NP * PAIR_HALVES;  // halves of one tensor's chunk
  static constexpr int PPW = NP / kWaves;        // pairs per wave, per tensor
  static_assert(PPW >= 1 && NP % kWaves == 0, "chunk shape");

  // halves offset of 16-byte chunk c of row r, plus e halves within the chunk.
  // Rows 8-15 and 24-31 hold the two chunks of a pair swapped, so that the 16
  // lanes of a K read (16 rows, one chunk each) fall on 16 different 16-byte
  // bank groups instead of two rows per group.
  __device__ static __forceinline__ int at(int r, int c, int e) {
    return (c >> 1) * PAIR_HALVES + r * 16 + (((c & 1) ^ ((r >> 3) & 1)) * 8) + e;
  }

  // This lane's byte offset within its 16-token tile (the same for every pair,
  // and every chunk of the token loop): row lane / 2 mod 16, and the chunk of
  // the pair that at() places in LDS slot lane, i.e. lane % 2 swapped on rows
  // 8-15 and 24-31 (lane / 16 odd).
  __device__ static __forceinline__ uint32_t lane_off(int lane) {
    return (uint32_t)(((lane >> 1) & 15) * RB + (((lane & 1) ^ ((lane >> 4) & 1)) * 16));
  }

  // K rows to buf[0, HALVES), V rows to buf[HALVES, 2 HALVES). Lanes 0-31 hold
  // rows 0-15 (block blk_a), lanes 32-63 rows 16-31 (blk_b); a tile in a block
  // outside the pool reads the head's first rows (V zeroed later).
  __device__ static __forceinline__ void issue(const PrefillArgs& a, int blk_a, int blk_b, const uint8_t* kc_head,
                                               const uint8_t* vc_head, size_t blk_stride, int t0, _Float16* buf,
                                               int wave, int lane, uint32_t loff) {
    const int bsm = (1 << a.bs_log2) - 1;
    const bool oka = (unsigned)blk_a < (unsigned)a.num_blocks;
    const bool okb = (unsigned)blk_b < (unsigned)a.num_blocks;
    const size_t base_a = oka ? (size_t)blk_a * blk_stride + (size_t)(t0 & bsm) * RB : 0;
    const size_t base_b = okb ? (size_t)blk_b * blk_stride + (size_t)((t0 + 16) & bsm) * RB : 0;
    const size_t off = (lane < 32 ? base_a : base_b) + loff;
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int pp = wave * PPW + i;  // wave-uniform
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(kc_head + off + pp * 32),
                                       (__attribute__((address_space(3))) void*)(buf + pp * PAIR_HALVES), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(vc_head + off + pp * 32),
                                       (__attribute__((address_space(3))) void*)(buf + HALVES + pp * PAIR_HALVES),
                                       16, 0, 0);
    }
  }

  // V rows that must read as zeros: past `end`, or in a tile outside the pool
  __device__ static __forceinline__ void zero_invalid(_Float16* buf, int t0, int end, bool oka, bool okb) {
    _Float16* vb = buf + HALVES;
    for (int idx = threadIdx.x; idx < kChunk * NP; idx += kWaves * 64) {
      const int r = idx % kChunk;
      const int pp = idx / kChunk;
      const bool ok = (r < 16 ? oka : okb) && t0 + r < end;
      if (!ok) {
        u32x4* d = reinterpret_cast<u32x4*>(vb + pp * PAIR_HALVES + r * 16);
        d[0] = u32x4{0u, 0u, 0u, 0u};
        d[1] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
};

// Where a chunk buffer keeps row r's 16-byte piece c (8 halves), plus e
// halves, for K and for V (offsets in halves from the buffer's start).
template <int D, bool FP8>
struct PaddedLayout {  // rows padded to D + 8 halves (Stage)
  using S = ChunkShape<D, FP8>;
  __device__ static __forceinline__ int k(int r, int c) { return r * S::KS + c * 8; }
  __device__ static __forceinline__ int v(int r, int c, int e) { return kChunk * S::KS + r * S::VS + c * 8 + e; }
};
template <int D>
struct PairLayout {  // pair-major rows (Direct)
  __device__ static __forceinline__ int k(int r, int c) { return Direct<D>::at(r, c, 0); }
  __device__ static __forceinline__ int v(int r, int c, int e) { return Direct<D>::HALVES + Direct<D>::at(r, c, e); }
};

// three workgroups per compute unit (3 waves per SIMD) hide the LDS and
// matrix-core latencies of the token loop far better than two (measured on
// MI355X: 10.7 -> 8.4 ms on the Qwen3-shaped prefix-cache prefill)
template <int D, int G, int FMT>
__global__ void __launch_bounds__(kWaves * 64, kMinBlocks) attn_prefill_kernel(PrefillArgs a) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr bool FP8 = FMT != kF16;
  using S = ChunkShape<D, FP8>;
  constexpr int KM = D / 32;   // q.k MFMAs per 16-token tile and column group
  constexpr int NT = D / 16;   // output head-dim tiles
  constexpr int DQ = D / 4;    // head-dim elements per lane group in the q.k operands
  constexpr int QT = kTileCols / G;  // query tokens per workgroup tile
  // fp16 chunks go straight from global memory to LDS (Direct); fp8 chunks are
  // widened on the way through registers (Stage)
  constexpr bool DIRECT = !FP8;
  constexpr int PREFIX_HALVES = (kMaxSeqs + 1 + kWaves * 64) * 2;
  constexpr int LDS_HALVES = !DIRECT && 2 * S::BUF > PREFIX_HALVES ? 2 * S::BUF : PREFIX_HALVES;

  // the tile prefix; with Stage the same memory then holds the two chunk buffers
  __shared__ __align__(16) _Float16 lds[LDS_HALVES];
  // the two chunk buffers of Direct: separate arrays, so that the compiler can
  // tell the buffer being read from the one the loads are landing in
  __shared__ __align__(16) _Float16 dbuf0[DIRECT ? 2 * Direct<D>::HALVES : 8];
  __shared__ __align__(16) _Float16 dbuf1[DIRECT ? 2 * Direct<D>::HALVES : 8];
  int* pt = reinterpret_cast<int*>(lds);
  build_tile_prefix(a, G, pt, pt + a.B + 1);

  const int total_tiles = pt[a.B];
  const int li = logical_index();
  const int head = li / a.tiles_bound;
  const int tr = li - head * a.tiles_bound;
  if (head >= a.Hkv || tr >= total_tiles) return;  // uniform over the workgroup
  const int tile = total_tiles - 1 - tr;            // longest contexts first
  const int seq = find_seq(pt, a.B, tile);
  const int k_tile = tile - pt[seq];
  __syncthreads();  // the prefix is dead from here on; the buffers take over

  int qfirst, n;
  seq_rows(a, seq, &qfirst, &n);
  const int L = min(max(a.ctx_lens[seq], 0), a.max_blocks << a.bs_log2);
  const int row0 = k_tile * QT;             // first query token of the tile, within the chunk
  const int nt = min(QT, n - row0);         // query tokens in this tile
  const int pos0 = L - n + row0;            // position of the tile's first query token
  const int kend = min(L, pos0 + nt);       // tokens the tile can see: [0, kend)
  const int nchunks = kend > 0 ? (kend + kChunk - 1) / kChunk : 0;

  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;
  // The softmax below takes the running max of the raw logits before scaling
  // them and masks a logit by setting it to -inf, which needs a scale > 0. A
  // negative scale is moved into the sign of the query operands (exact), and
  // a zero one becomes the smallest normal float: every visible p is then
  // exactly 1, as with scale 0, and a masked one still 0.
  const float qk_signed = uniform_f32(a.k_scale_h ? a.qk_base * a.k_scale_h[head] : a.qk_scale);
  const bool q_neg = qk_signed < 0.0f;
  const float qk_mag = q_neg ? -qk_signed : qk_signed;
  const float qk_scale = qk_mag == 0.0f ? __FLT_MIN__ : qk_mag;

  // Q^T operands (B of S = K Q^T): column c = 32 wave + 16 cg + col holds query
  // token c / G, head c % G of the group; d = grp * DQ + 8 m + slot
  f16x8 qb[kNcg][KM];
  int qpos[kNcg];
#pragma unroll
  for (int cg = 0; cg < kNcg; ++cg) {
    const int c = wave * kCols + cg * 16 + col;
    const int tl = c / G;
    const bool live = tl < nt;
    qpos[cg] = live ? pos0 + tl : -1;  // -1: every token is masked
    const size_t qoff = live ? ((size_t)(qfirst + row0 + tl) * a.Hq + head * G + c % G) * D + grp * DQ : 0;
#pragma unroll
    for (int m = 0; m < KM; ++m) {
      qb[cg][m] = live ? *reinterpret_cast<const f16x8*>(a.q + qoff + 8 * m) : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (q_neg) qb[cg][m] = -qb[cg][m];
    }
  }
  const bool all_live = nt == QT;

  // Softmax state per column, in the lanes of its column: the running max
  // m (log2 units) is kept as two derived values that the token loop uses
  // directly, so that a step without a move of the max spends no vector
  // instructions on it: thr = (m + kLazy) / qk_scale, the raw logit above
  // which the max must move (-inf while m is -inf), and neg_m = -m (0 while
  // m is -inf). l_part is the lane's share of the column's sum.
  f32x4 o[kNcg][NT];
  float thr[kNcg], neg_m[kNcg], l_part[kNcg];
#pragma unroll
  for (int cg = 0; cg < kNcg; ++cg) {
#pragma unroll
    for (int c = 0; c < NT; ++c) o[cg][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    thr[cg] = -INFINITY;
    neg_m[cg] = 0.0f;
    l_part[cg] = 0.0f;
  }

  const int32_t* tab = a.tables + (size_t)seq * a.max_blocks;
  const size_t head_bytes = (size_t)S::RB << a.bs_log2;
  const size_t blk_stride = (size_t)a.Hkv * head_bytes;
  const uint8_t* kc_head = a.kc + (size_t)head * head_bytes;
  const uint8_t* vc_head = a.vc + (size_t)head * head_bytes;

  // tr16 read addresses for V^T (A operand of O^T += V^T P^T): lane 16g + 4e +
  // mm names row 4g + e (tile a) or 16 + 4g + e (tile b), elements 16c + 4mm .. +3
  const int tr_row = 4 * grp + (col >> 2);
  const int tr_col = 4 * (col & 3);

  // block ids of a chunk's two 16-token tiles (wave-uniform; -1 past the
  // end). Lane l holds the block of 16-token tile tile0 + l, refilled with one
  // vector load every 32 chunks, and each chunk reads its two with readlane.
  int tile0 = 0;
  int lane_blk = (lane * 16 < kend) ? tab[(lane * 16) >> a.bs_log2] : -1;
  auto chunk_blocks = [&](int t0, int* ba, int* bb) {
    const int tl = t0 >> 4;
    if (tl + 1 - tile0 >= 64) {
      tile0 = tl;
      const int tt = (tile0 + lane) * 16;
      lane_blk = tt < kend ? tab[tt >> a.bs_log2] : -1;
    }
    *ba = __builtin_amdgcn_readlane(lane_blk, tl - tile0);
    *bb = t0 + 16 < kend ? __builtin_amdgcn_readlane(lane_blk, tl + 1 - tile0) : -1;
  };

  // The arithmetic of the chunk at token t0, whose tiles lie in blocks ba and
  // bb, from the chunk buffer buf laid out as Lay: S = K Q^T, the online
  // softmax, O^T += V^T P^T.
  auto compute_chunk = [&](const _Float16* buf, int t0, int ba, int bb, auto lay) {
    using Lay = decltype(lay);
    // tokens of a block outside the pool are skipped
    const bool ok_a = (unsigned)ba < (unsigned)a.num_blocks;
    const bool ok_b = (unsigned)bb < (unsigned)a.num_blocks;

    // S = K . Q^T for both tiles and both column groups
    f32x4 s[2][kNcg];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int cg = 0; cg < kNcg; ++cg) s[tt][cg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int kr = 16 * tt + col;
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        const f16x8 ka = *reinterpret_cast<const f16x8*>(buf + Lay::k(kr, grp * (DQ / 8) + m));
#pragma unroll
        for (int cg = 0; cg < kNcg; ++cg)
          s[tt][cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb[cg][m], s[tt][cg], 0, 0, 0);
      }
    }

    // online softmax per column; lane (col, grp) sees tokens t0 + 4grp + v and
    // t0 + 16 + 4grp + v. Raw logits are masked to -inf where needed; the
    // running max m (log2 units) is moved only when some lane's logit exceeds
    // it by more than kLazy (a raw logit above thr), so between moves no lane
    // shuffles and the accumulators are not rescaled (p <= 2^kLazy then, well
    // inside fp16).
    const bool plain = all_live && ok_a && ok_b && t0 + kChunk - 1 <= pos0;
    float z[kNcg][8];
    float mt[kNcg];
#pragma unroll
    for (int cg = 0; cg < kNcg; ++cg) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        z[cg][v] = s[0][cg][v];
        z[cg][4 + v] = s[1][cg][v];
      }
      if (!plain) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int ta = t0 + 4 * grp + v;
          const int tb = t0 + 16 + 4 * grp + v;
          z[cg][v] = (ok_a && ta <= qpos[cg]) ? z[cg][v] : -INFINITY;
          z[cg][4 + v] = (ok_b && tb <= qpos[cg]) ? z[cg][4 + v] : -INFINITY;
        }
      }
      // the lane's largest raw logit
      const float ma = max3_f32(z[cg][0], z[cg][1], z[cg][2]);
      const float mb = max3_f32(z[cg][3], z[cg][4], z[cg][5]);
      const float mc = max3_f32(z[cg][6], z[cg][7], ma);
      mt[cg] = max3_f32(mb, mc, mc);
    }
    bool need = false;
#pragma unroll
    for (int cg = 0; cg < kNcg; ++cg) need = need || mt[cg] > thr[cg];
    if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
      for (int cg = 0; cg < kNcg; ++cg) {
        float m = mt[cg];
        m = fmaxf(m, shfl_xor_f32(m, 16));
        m = fmaxf(m, shfl_xor_f32(m, 32));
        m *= qk_scale;
        const float m_old = thr[cg] == -INFINITY ? -INFINITY : -neg_m[cg];
        const float mn = fmaxf(m_old, m);
        const float alpha = fast_exp2(m_old - safe_max(mn));
        l_part[cg] *= alpha;
#pragma unroll
        for (int c = 0; c < NT; ++c) o[cg][c] *= alpha;
        neg_m[cg] = -safe_max(mn);
        thr[cg] = (mn + kLazy) / qk_scale;
      }
    }
    f16x8 pb[kNcg];
#pragma unroll
    for (int cg = 0; cg < kNcg; ++cg) {
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = fast_exp2(__builtin_fmaf(z[cg][i], qk_scale, neg_m[cg]));
        pb[cg][i] = (_Float16)p[i];
      }
      l_part[cg] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    }

    // O^T += V^T . P^T, one 16-row head-dim tile at a time
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      const int pc = 2 * c + (tr_col >> 3);  // the 16-byte piece holding elements 16c + tr_col ..
      const _Float16* p1 = buf + Lay::v(tr_row, pc, tr_col & 7);
      const _Float16* p2 = buf + Lay::v(16 + tr_row, pc, tr_col & 7);
      const f16x4 r1 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1)));
      const f16x4 r2 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p2)));
      const f16x8 va = __builtin_shufflevector(r1, r2, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int cg = 0; cg < kNcg; ++cg)
        o[cg][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[cg], o[cg][c], 0, 0, 0);
    }
  };

  if constexpr (DIRECT) {
    // chunk j + 1 lands in one buffer while chunk j is computed from the other;
    // each wave waits for its own loads, then the barrier makes all of them
    // visible (and ends every read of the buffer the next loads overwrite)
    using DS = Direct<D>;
    const uint32_t loff = DS::lane_off(lane);
    auto zero_if_needed = [&](_Float16* buf, int t0, int ba, int bb) {
      const bool oka = (unsigned)ba < (unsigned)a.num_blocks;
      const bool okb = (unsigned)bb < (unsigned)a.num_blocks;
      if (!(oka && okb && t0 + kChunk - 1 < kend)) {  // uniform over the workgroup
        DS::zero_invalid(buf, t0, kend, oka, okb);
        __syncthreads();
      }
    };
    int ba = -1, bb = -1;
    if (nchunks > 0) {
      chunk_blocks(0, &ba, &bb);
      DS::issue(a, ba, bb, kc_head, vc_head, blk_stride, 0, dbuf0, wave, lane, loff);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (nchunks > 0) zero_if_needed(dbuf0, 0, ba, bb);
    auto step = [&](int j, _Float16* cur, _Float16* nxt) {
      const int t0 = j * kChunk;
      int nba = -1, nbb = -1;
      if (j + 1 < nchunks) {
        chunk_blocks(t0 + kChunk, &nba, &nbb);
        DS::issue(a, nba, nbb, kc_head, vc_head, blk_stride, t0 + kChunk, nxt, wave, lane, loff);
      }
      compute_chunk(cur, t0, ba, bb, PairLayout<D>{});
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (j + 1 < nchunks) zero_if_needed(nxt, t0 + kChunk, nba, nbb);
      ba = nba;
      bb = nbb;
    };
    for (int j = 0; j < nchunks; j += 2) {
      step(j, dbuf0, dbuf1);
      if (j + 1 < nchunks) step(j + 1, dbuf1, dbuf0);
    }
  } else {
    Stage<D, FMT> st;
    int ba = -1, bb = -1;
    if (nchunks > 0) {
      chunk_blocks(0, &ba, &bb);
      st.load(a, ba, bb, kc_head, vc_head, blk_stride, 0, kend);
      st.store(lds);
    }
    __syncthreads();

    for (int j = 0; j < nchunks; ++j) {
      const int t0 = j * kChunk;
      int nba = -1, nbb = -1;
      if (j + 1 < nchunks) {
        chunk_blocks(t0 + kChunk, &nba, &nbb);
        st.load(a, nba, nbb, kc_head, vc_head, blk_stride, t0 + kChunk, kend);
      }
      compute_chunk(lds + (j & 1) * S::BUF, t0, ba, bb, PaddedLayout<D, FP8>{});

      if (j + 1 < nchunks) st.store(lds + ((j + 1) & 1) * S::BUF);
      __syncthreads();
      ba = nba;
      bb = nbb;
    }
  }

  const float v_scale = uniform_f32(a.v_scale_h ? a.v_scale_h[head] : a.v_out_scale);
  // per-column sums over the four lane groups (the max is already common);
  // lane (col, grp) holds d = 16c + 4grp + v of its column
#pragma unroll
  for (int cg = 0; cg < kNcg; ++cg) {
    float l = l_part[cg];
    l += shfl_xor_f32(l, 16);
    l += shfl_xor_f32(l, 32);
    const int c = wave * kCols + cg * 16 + col;
    const int tl = c / G;
    if (tl < nt) {
      const float sc = l > 0.0f ? v_scale / l : 0.0f;
      f16* orow = a.out + ((size_t)(qfirst + row0 + tl) * a.Hq + head * G + c % G) * D + 4 * grp;
#pragma unroll
      for (int cc = 0; cc < NT; ++cc) {
        f16x4 h;
#pragma unroll
        for (int v = 0; v < 4; ++v) h[v] = (f16)(o[cg][cc][v] * sc);
        *reinterpret_cast<f16x4*>(orow + 16 * cc) = h;
      }
    }
  }
}

typedef void (*PrefillFn)(PrefillArgs);

template <int D, int FMT>
PrefillFn pick_d(int G) {
  switch (G) {
    case 1: return attn_prefill_kernel<D, 1, FMT>;
    case 2: return attn_prefill_kernel<D, 2, FMT>;
    case 4: return attn_prefill_kernel<D, 4, FMT>;
    case 8: return attn_prefill_kernel<D, 8, FMT>;
    default: return nullptr;
  }
}

template <int D>
PrefillFn pick_fmt(int G, int fmt) {
  switch (fmt) {
    case kF16: return pick_d<D, kF16>(G);
    case kE4M3: return pick_d<D, kE4M3>(G);
    case kE5M2: return pick_d<D, kE5M2>(G);
    default: return nullptr;
  }
}

PrefillFn pick(int D, int G, int fmt) {
  if (D == 64) return pick_fmt<64>(G, fmt);
  if (D == 128) return pick_fmt<128>(G, fmt);
  return nullptr;
}

int log2_exact(int v) {
  int k = 0;
  while ((1 << k) < v) ++k;
  return (1 << k) == v ? k : -1;
}

}  // namespace
}  // namespace pkv

namespace pkv {
namespace {

int prefill_impl(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                 int max_blocks_per_seq, const int32_t* ctx_lens, const int32_t* q_start, int num_seqs, int total_q,
                 int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks, float sm_scale,
                 int kv_dtype, float k_scale, float v_scale, const float* k_scales, const float* v_scales,
                 void* stream) {
  if (num_seqs < 0 || total_q < 0 || num_kv_heads <= 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0 ||
      num_blocks <= 0)
    return PKV_ERR_INVALID;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_INVALID;
  if (block_size != 16 && block_size != 32 && block_size != 64) return PKV_ERR_INVALID;
  if (kv_dtype != PKV_KV_F16 && kv_dtype != PKV_KV_FP8_E4M3 && kv_dtype != PKV_KV_FP8_E5M2)
    return PKV_ERR_INVALID;
  const int G = num_q_heads / num_kv_heads;
  PrefillFn fn = pick(head_dim, G, kv_dtype);
  if (!fn) return PKV_ERR_INVALID;
  if ((int64_t)max_blocks_per_seq * block_size > 0x7FFFFFFF) return PKV_ERR_INVALID;
  if (num_seqs == 0 || total_q == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !ctx_lens || !q_start) return PKV_ERR_INVALID;
  if (!vec_aligned(out) || !vec_aligned(q) || !vec_aligned(k_cache) || !vec_aligned(v_cache) ||
      !aligned_to(block_tables, 4) || !aligned_to(ctx_lens, 4) || !aligned_to(q_start, 4) ||
      !aligned_to(k_scales, 4) || !aligned_to(v_scales, 4))
    return PKV_ERR_INVALID;

  const bool fp8 = kv_dtype != PKV_KV_F16;
  const float kLog2e = 1.4426950408889634f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int b0 = 0; b0 < num_seqs; b0 += kMaxSeqs) {
    const int B = num_seqs - b0 < kMaxSeqs ? num_seqs - b0 : kMaxSeqs;
    // tiles of one KV head: sum over sequences of ceil(n_s G / 128) <= total_q G / 128 + B
    const int64_t tiles = ((int64_t)total_q * G + kTileCols - 1) / kTileCols + B;
    const int64_t grid = tiles * num_kv_heads;
    if (grid > 0x7FFFFFFF) return PKV_ERR_INVALID;
    PrefillArgs a;
    a.q = static_cast<const f16*>(q);
    a.kc = static_cast<const uint8_t*>(k_cache);
    a.vc = static_cast<const uint8_t*>(v_cache);
    a.tables = block_tables + (size_t)b0 * max_blocks_per_seq;
    a.ctx_lens = ctx_lens + b0;
    a.q_start = q_start + b0;
    a.out = static_cast<f16*>(out);
    a.max_blocks = max_blocks_per_seq;
    a.B = B;
    a.Hkv = num_kv_heads;
    a.Hq = num_q_heads;
    a.bs_log2 = log2_exact(block_size);
    a.num_blocks = num_blocks;
    a.total_q = total_q;
    a.tiles_bound = (int)tiles;
    a.qk_scale = sm_scale * kLog2e * (fp8 ? k_scale : 1.0f);
    a.v_out_scale = fp8 ? v_scale : 1.0f;
    a.k_scale_h = fp8 ? k_scales : nullptr;
    a.v_scale_h = fp8 ? v_scales : nullptr;
    a.qk_base = sm_scale * kLog2e;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(kWaves * 64), 0, s, a);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  }
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

extern "C" int paged_attn_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, int max_blocks_per_seq,
                                  const int32_t* ctx_lens, const int32_t* q_start, int num_seqs,
                                  int total_q, int num_q_heads, int num_kv_heads, int head_dim,
                                  int block_size, int num_blocks, float sm_scale, int kv_dtype,
                                  float k_scale, float v_scale, void* stream) {
  return pkv::prefill_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, ctx_lens, q_start,
                           num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                           sm_scale, kv_dtype, k_scale, v_scale, nullptr, nullptr, stream);
}

extern "C" int paged_attn_prefill_scaled(void* out, const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_tables, int max_blocks_per_seq,
                                         const int32_t* ctx_lens, const int32_t* q_start, int num_seqs,
                                         int total_q, int num_q_heads, int num_kv_heads, int head_dim,
                                         int block_size, int num_blocks, float sm_scale, int kv_dtype,
                                         const float* k_scales, const float* v_scales, void* stream) {
  if (kv_dtype != PKV_KV_F16 && num_seqs > 0 && total_q > 0 && (!k_scales || !v_scales)) return PKV_ERR_INVALID;
  return pkv::prefill_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, ctx_lens, q_start,
                           num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                           sm_scale, kv_dtype, 1.0f, 1.0f, k_scales, v_scales, stream);
}
