// Pass 1 of paged decode attention for grouped-query heads (G = 4 or 8 query
// heads per KV head), on the matrix cores. Included by attn_decode.hip, whose
// AttnArgs, work split (shares, pieces, partial slots) and pass 2 it shares.
//
// With G query heads per KV head, q.K over a 16-token tile is a small dense
// contraction (16 tokens x G heads x D), so it runs as v_mfma_f32_16x16x32_f16:
//   S = K . Q^T   M = 16 tokens, N = 16 heads (G used, the rest zero), K-dim = d
//   O^T += V^T . P^T   M = 16 d, N = 16 heads, K-dim = 32 tokens
// Operand layouts (16x16x32 f16): A[i][k] in lane i + 16g, B[k][j] in lane
// j + 16g, both holding 8 k values chosen by (g, slot); C[i][j] in lane
// j + 16(i/4), register i%4.
//   - K rows need no transpose: lane (token t, group g) loads 16-byte chunks
//     g, 4 + g, 8 + g, .. of row t, so the four lanes of a row read 64
//     contiguous bytes per load instruction; the d index of each MFMA slot
//     (and of the query's B operand) is chosen to match (k_dim_of).
//   - S's accumulator gives lane (head h, group g) the logits of tokens
//     4g..4g+3 of a tile; two tiles give exactly the 8 token slots that P^T
//     needs as the B operand of the P.V product, so P never moves between lanes.
//   - V^T is the A operand: V rows are written to LDS as fp16 and read back with
//     ds_read_b64_tr_b16, which returns, per lane, one d column of four token
//     rows (lanes 4e..4e+3 of a 16-lane group name the four 4-element pieces of
//     row e; lane i receives element i of rows e = 0..3).
//   - The O^T accumulator puts head h in lane column h, where that head's
//     online-softmax max and rescale factor already live.
// A unit is a 32-token chunk (two 16-token tiles, each inside one block). Each
// wave is a worker with its own LDS buffer for V; rows at or past the end of
// the sequence are masked in the logits and written to LDS as zeros.

namespace pkv {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLazy = 8.0f;  // log2 headroom before a running max moves

__device__ __forceinline__ f16x8 f16x8_from_u32x4(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

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

// First d index of the 8 that lane group g supplies to the q.k MFMA m, when
// the lane holds 16-byte chunks g, 4 + g, .. of its K row (each chunk feeds one
// fp16 MFMA or two fp8 MFMAs)
template <int ELEM>
__device__ __forceinline__ int k_dim_of(int m, int g) {
  constexpr int EPC = 16 / ELEM;  // elements per chunk
  constexpr int MPC = EPC / 8;    // MFMAs per chunk
  return (4 * (m / MPC) + g) * EPC + 8 * (m % MPC);
}

template <int D, int G, int FMT, int NW>
__global__ void __launch_bounds__(NW * 64) attn_partition_mfma_kernel(AttnArgs a) {
  static_assert(G == 4 || G == 8, "group size");
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr bool FP8 = FMT != kF16;
  constexpr int ELEM = FP8 ? 1 : 2;
  constexpr int RB = D * ELEM;          // bytes of one token row of one head
  constexpr int KM = D / 32;            // q.k MFMAs per tile
  constexpr int NT = D / 16;            // output d tiles
  constexpr int DQ = D / 4;             // d elements per lane in the K operand
  constexpr int KLD = DQ * ELEM / 16;   // 16-byte K loads per lane per tile
  constexpr int LPR = RB / 16;          // lanes per row in the V load
  constexpr int RPL = 64 / LPR;         // rows per V load
  constexpr int VLD = 32 / RPL;         // V loads per lane per 32-token chunk
  constexpr int VS = D + 16;            // LDS row stride of V, halves (16-byte aligned)
  static_assert(RPL <= 16 && 16 % RPL == 0, "a V load stays inside one tile");

  __shared__ __align__(16) _Float16 vlds[NW * 32 * VS];
  extern __shared__ int dyn_smem[];
  int* pt = dyn_smem;
  build_prefix(a, pt, pt + a.B + 1);

  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;
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
  _Float16* vbuf = vlds + wave * 32 * VS;
  const uint32_t k_lane_off = (uint32_t)(col * RB + grp * 16);  // + 64 per chunk
  const int v_row = lane / LPR;        // row within a V load
  const int v_cb = (lane % LPR) * 16;  // byte offset within the row
  // tr16 read addresses: lane 16g + 4e + mm names row 4g + e (tile a) or
  // 16 + 4g + e (tile b), elements 16c + 4mm .. +3
  const int tr_row = 4 * grp + (col >> 2);
  const int tr_col = 4 * (col & 3);

  for (int64_t t = start; t < end;) {
    const Piece pc = locate(pt, a.B, P, t, end);
    const int seq = pc.seq;
    const int hq0 = pc.head * G;
    // The piece's setup loads (its length, the query columns, the first 32
    // units' block ids, the head's scales) are all issued before the first
    // wait: one round trip.
    const int L_raw = seq_len(a, seq);
    const int32_t* tab = a.tables + (size_t)seq * a.max_blocks;
    // lane l: tile l & 1 of unit j0 + l / 2; read whatever the length (the
    // index kept inside the row), tiles past the sequence are dropped below
    auto unit_block = [&](int j0) {
      const int tt = 32 * (j0 + (lane >> 1)) + 16 * (lane & 1);
      return tab[min(tt >> a.bs_log2, a.max_blocks - 1)];
    };
    int blk_raw = unit_block(pc.u0);

    // Q^T as the B operand: head = col (zero past G), d = k_dim_of(m, grp) + slot
    f16x8 qb[KM];
#pragma unroll
    for (int m = 0; m < KM; ++m) {
      const f16* qrow = a.q + ((size_t)seq * a.Hq + hq0 + (col < G ? col : 0)) * D + k_dim_of<ELEM>(m, grp);
      qb[m] = *reinterpret_cast<const f16x8*>(qrow);
    }
    float qk_scale = a.qk_scale, v_scale = a.v_out_scale;
    if (a.k_scale_h) {
      const float ks = a.k_scale_h[pc.head];
      const float vs = a.v_scale_h[pc.head];
      qk_scale = a.qk_base * ks;
      v_scale = vs;
    }
    const int L = wave_uniform(L_raw);
    if (col >= G) {
#pragma unroll
      for (int m = 0; m < KM; ++m) qb[m] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }

    f32x4 o[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_part = 0.0f;

    const uint8_t* kc_head = a.kc + (size_t)pc.head * head_bytes;
    const uint8_t* vc_head = a.vc + (size_t)pc.head * head_bytes;
    for (int j0 = pc.u0; j0 < pc.u1; j0 += 32) {
      // block ids of up to 32 chunks (two tiles each), one per lane (the
      // first 32 with the setup); -1 for a tile past the sequence
      if (j0 != pc.u0) blk_raw = unit_block(j0);
      int my_blk;
      {
        const int jj = j0 + (lane >> 1);
        const int tt = 32 * jj + 16 * (lane & 1);
        my_blk = jj < pc.u1 && tt < L ? blk_raw : -1;
      }
      const int nj = min(32, pc.u1 - j0);
      for (int j = 0; j < nj; ++j) {
        const int ta = 32 * (j0 + j);
        const int blk_a = __builtin_amdgcn_readlane(my_blk, 2 * j);
        const int blk_b = __builtin_amdgcn_readlane(my_blk, 2 * j + 1);
        const bool ok_a = (unsigned)blk_a < (unsigned)a.num_blocks;
        const bool ok_b = (unsigned)blk_b < (unsigned)a.num_blocks;
        // a tile outside the pool reads block 0 and is masked below; a unit
        // with both tiles in the pool and all 32 tokens inside the sequence
        // (every unit but a sequence's last) skips the masking altogether
        const size_t off_a = ok_a ? (size_t)blk_a * blk_stride + (size_t)(ta & bs_mask) * RB : 0;
        const size_t off_b = ok_b ? (size_t)blk_b * blk_stride + (size_t)((ta + 16) & bs_mask) * RB : 0;
        const bool full = ok_a && ok_b && ta + 32 <= L;

        // K rows (A operand of S) and V rows (to LDS)
        u32x4 ka[KLD], kb[KLD], vv[VLD];
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
          ka[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kc_head + off_a + k_lane_off + 64 * i));
          kb[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kc_head + off_b + k_lane_off + 64 * i));
        }
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
          const size_t off = i * RPL >= 16 ? off_b : off_a;
          const int r = (i * RPL + v_row) & 15;
          vv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vc_head + off + r * RB + v_cb));
        }

        // S = K . Q^T for both tiles
        f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 sb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < KM; ++m) {
          f16x8 aa, ab;
          if constexpr (FP8) {
            aa = fp8x8_to_f16x8<FMT>(ka[m / 2][(m % 2) * 2], ka[m / 2][(m % 2) * 2 + 1]);
            ab = fp8x8_to_f16x8<FMT>(kb[m / 2][(m % 2) * 2], kb[m / 2][(m % 2) * 2 + 1]);
          } else {
            aa = f16x8_from_u32x4(ka[m]);
            ab = f16x8_from_u32x4(kb[m]);
          }
          sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(aa, qb[m], sa, 0, 0, 0);
          sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(ab, qb[m], sb, 0, 0, 0);
        }

        // online softmax per head (lane column); tokens of this lane: ta+4grp+v, ta+16+4grp+v
        float z[8];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          z[v] = sa[v] * qk_scale;
          z[4 + v] = sb[v] * qk_scale;
        }
        if (!full) {
          // rows past the end of the sequence (possibly not finite in the
          // pool) and tiles outside the pool: no logit, zero V rows
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            if (!(ok_a && ta + 4 * grp + v < L)) z[v] = -INFINITY;
            if (!(ok_b && ta + 16 + 4 * grp + v < L)) z[4 + v] = -INFINITY;
          }
#pragma unroll
          for (int i = 0; i < VLD; ++i) {
            const int r = i * RPL + v_row;  // 0..31
            if (!((r < 16 ? ok_a : ok_b) && ta + r < L)) vv[i] = u32x4{0u, 0u, 0u, 0u};
          }
        }
        // the running max (log2 units) moves only when some lane's logits exceed
        // it by more than kLazy: between moves the accumulators are not
        // rescaled and no lane shuffles run (p <= 2^kLazy, well inside fp16)
        float mt = z[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mt = fmaxf(mt, z[i]);
        if (__builtin_amdgcn_ballot_w64(mt > m_run + kLazy)) {
          mt = fmaxf(mt, shfl_xor_f32(mt, 16));
          mt = fmaxf(mt, shfl_xor_f32(mt, 32));
          const float mn = fmaxf(m_run, mt);
          const float alpha = fast_exp2(m_run - safe_max(mn));
          l_part *= alpha;
#pragma unroll
          for (int c = 0; c < NT; ++c) o[c] *= alpha;
          m_run = mn;
        }
        const float ms = safe_max(m_run);
        f16x8 pb;
        float ps = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = fast_exp2(z[i] - ms);
          ps += p;
          pb[i] = (_Float16)p;
        }
        l_part += ps;

        // V rows -> LDS as fp16 (masked rows are zero bytes, which widen to +0)
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
          const int r = i * RPL + v_row;  // 0..31
          _Float16* dst = vbuf + r * VS + v_cb / ELEM;
          if constexpr (FP8) {
            *reinterpret_cast<f16x8*>(dst) = fp8x8_to_f16x8<FMT>(vv[i][0], vv[i][1]);
            *reinterpret_cast<f16x8*>(dst + 8) = fp8x8_to_f16x8<FMT>(vv[i][2], vv[i][3]);
          } else {
            *reinterpret_cast<u32x4*>(dst) = vv[i];
          }
        }

        // O^T += V^T . P^T, one 16-wide d tile at a time
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const _Float16* p1 = vbuf + tr_row * VS + 16 * c + tr_col;
          const _Float16* p2 = vbuf + (16 + tr_row) * VS + 16 * c + tr_col;
          // whole-vector casts: a bit_cast of single vector elements was lowered
          // to element 0 by this compiler
          const f16x4 r1 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1)));
          const f16x4 r2 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p2)));
          const f16x8 va = __builtin_shufflevector(r1, r2, 0, 1, 2, 3, 4, 5, 6, 7);
          o[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb, o[c], 0, 0, 0);
        }
      }
    }

    // per-head sum over the four lane groups; the max is already common
    l_part += shfl_xor_f32(l_part, 16);
    l_part += shfl_xor_f32(l_part, 32);

    // lane (head col, group grp) holds d = 16c + 4grp + v of its head
    const bool whole = pc.u0 == 0 && pc.u1 == pc.n_u;
    const int slot = t == start ? 0 : 1;
    if (col < G) {
      if (whole) {
        const float sc = l_part > 0.0f ? v_scale / l_part : 0.0f;
        f16* orow = a.out + ((size_t)seq * a.Hq + hq0 + col) * D + 4 * grp;
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          f16x4 h;
#pragma unroll
          for (int v = 0; v < 4; ++v) h[v] = (f16)(o[c][v] * sc);
          *reinterpret_cast<f16x4*>(orow + 16 * c) = h;
        }
      } else {
        // the piece's output divided by its own sum, as fp16 (a weighted mean
        // of V rows, so within V's range), at half the bytes of fp32
        const size_t pi = ((size_t)w * 2 + slot) * G + col;
        const float sc = l_part > 0.0f ? v_scale / l_part : 0.0f;
        f16* orow = reinterpret_cast<f16*>(a.ws_o) + pi * D + 4 * grp;
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          f16x4 h;
#pragma unroll
          for (int v = 0; v < 4; ++v) h[v] = (f16)(o[c][v] * sc);
          *reinterpret_cast<f16x4*>(orow + 16 * c) = h;
        }
        if (grp == 0) {
          a.ws_ml[2 * pi] = m_run;
          a.ws_ml[2 * pi + 1] = l_part;
        }
      }
    }
    t = pc.next_t;
  }
}

}  // namespace
}  // namespace pkv
