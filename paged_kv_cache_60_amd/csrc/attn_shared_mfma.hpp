// The shared-prefix pass of paged_attn_decode_shared, on the matrix cores.
// Included by attn_decode.hip after attn_gqa_mfma.hpp, whose operand layouts
// it uses, and whose AttnArgs, work split and merge it shares.
//
// Sequences forked from one prompt (beams, parallel samples) and requests
// mapped onto the same prefix-cache blocks hold the same physical blocks at
// the start of their tables ("vLLM Architecture and Memory Use, ch. 3", §3.2;
// "Where Did the VRAM Go (KV cache tutorial)", §4.2-4.4). Decoding them one by
// one reads those blocks once per sequence. This pass reads them once per
// group and contracts them with all of the group's query heads at once:
//   S = K . Q^T      M = 16 tokens, N = 32 query columns (two 16-column blocks),
//                    K-dim = d
//   O^T += V^T . P^T M = 16 d, N = 32 query columns, K-dim = 32 tokens
// Query column c of a pass is member c / G of the pass, query head c % G of
// the KV head; a group with more than 32 / G members takes one pass (a "part")
// per 32 columns. Operands are laid out as on the grouped-head path, with the
// B operand, the logits and the accumulators doubled. As there, the running
// max of a column moves only when a logit exceeds it by more than 2^8.
// A unit is 32 tokens of the prefix (two 16-token tiles, each inside one
// block). The units of every (KV head, group, part) are laid end to end, KV
// head major, and cut into equal shares, one per worker (a wave), as in pass
// 1. The logits of each column are masked past its member's own context
// length, so a member shorter than the prefix sees only its own tokens. A
// piece's online-softmax state goes to the merge buffers: by (member, query
// head) when the piece is a whole (group, part, KV head) segment, else to the
// worker's slot 0 (first piece of the share) or 1 (last).

namespace pkv {
namespace {

template <int D, int FMT, int NW>
__global__ void __launch_bounds__(NW * 64, FMT == kF16 ? 1 : 2) attn_shared_mfma_kernel(AttnArgs a) {
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr bool FP8 = FMT != kF16;
  constexpr int ELEM = FP8 ? 1 : 2;
  constexpr int RB = D * ELEM;          // bytes of one token row of one head
  constexpr int KM = D / 32;            // q.k MFMAs per tile and column block
  constexpr int NT = D / 16;            // output d tiles
  constexpr int DQ = D / 4;             // d elements per lane in the K operand
  constexpr int KLD = DQ * ELEM / 16;   // 16-byte K loads per lane per tile
  constexpr int LPR = RB / 16;          // lanes per row in the V load
  constexpr int RPL = 64 / LPR;         // rows per V load
  constexpr int VLD = 32 / RPL;         // V loads per lane per 32-token unit
  constexpr int VS = D + 16;            // LDS row stride of V, halves
  constexpr int CB = kSharedCols / 16;  // 16-column blocks
  static_assert(CB == 2, "two column blocks");
  static_assert(RPL <= 16 && 16 % RPL == 0, "a V load stays inside one tile");

  __shared__ __align__(16) _Float16 vlds[NW * 32 * VS];
  // dynamic LDS: unit prefix over the groups, scan space, and each group's
  // first member, members and shared tokens (read once here)
  extern __shared__ int dyn_smem[];
  int* spt = dyn_smem;              // [NG + 1]
  int* scan = spt + a.NG + 1;       // [NW * 64]
  int* gfirst = scan + NW * 64;     // [NG]
  int* gmem = gfirst + a.NG;        // [NG]
  int* gpre = gmem + a.NG;          // [NG]
  const int gl = a.g_log2;
  for (int g = threadIdx.x; g < a.NG; g += NW * 64) {
    const int n = group_members(a, g);
    gmem[g] = n;
    gfirst[g] = n ? a.grp_first[g] : 0;
    gpre[g] = group_tokens(a, g);
  }
  __syncthreads();
  // units of group g: one run of its prefix's 32-token units per kSharedCols query columns
  build_scan(a.NG, spt, scan, [&](int g) {
    return ((gmem[g] << gl) + kSharedCols - 1) / kSharedCols * ((gpre[g] + 31) / 32);
  });

  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= a.NG; i += NW * 64) a.ws_spt[i] = spt[i];
  const int PS = wave_uniform(spt[a.NG]);
  if (PS <= 0) return;
  const int64_t total = (int64_t)a.Hkv * PS;
  const int64_t w = worker_index(wave, NW);
  const int64_t start = share_start(w, total, a.s_workers);
  const int64_t end = share_start(w + 1, total, a.s_workers);
  const int MP = kSharedCols >> gl;  // members per part

  const size_t head_bytes = (size_t)RB << a.bs_log2;
  const size_t blk_stride = (size_t)a.Hkv * head_bytes;
  const int bs_mask = (1 << a.bs_log2) - 1;
  _Float16* vbuf = vlds + wave * 32 * VS;
  const uint32_t k_lane_off = (uint32_t)(col * RB + grp * 16);  // + 64 per chunk
  const int v_row = lane / LPR;
  const int v_cb = (lane % LPR) * 16;
  const int tr_row = 4 * grp + (col >> 2);
  const int tr_col = 4 * (col & 3);

  for (int64_t t = start; t < end;) {
    // the piece at unit t: (KV head, group, part, units [u0, u1))
    const int head = (int)(t / PS);
    const int rem = (int)(t - (int64_t)head * PS);
    const int g = find_seq(spt, a.NG, rem);
    const int pre = wave_uniform(gpre[g]);
    const int ug = (pre + 31) / 32;
    const int off = rem - wave_uniform(spt[g]);
    if (ug <= 0 || off < 0) break;  // only inconsistent group entries get here
    const int part = off / ug;
    const int u0 = off - part * ug;
    const int members = wave_uniform(gmem[g]);
    if (part * MP >= members) break;
    const int64_t seg_end = t - u0 + ug;
    const int64_t next_t = end < seg_end ? end : seg_end;
    const int u1 = u0 + (int)(next_t - t);
    const int first = wave_uniform(gfirst[g]);
    const int lead = first + part * MP;          // first member of this part
    const int nm = min(MP, members - part * MP);  // members of this part (columns past them are masked)
    const float qk_scale = head_qk_scale(a, head);
    const float v_scale = head_v_scale(a, head);

    // this lane's columns: cb * 16 + col -> member m, query head gh
    f16x8 qb[CB][KM];
    int Lc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = cb * 16 + col;
      const int m = c >> gl;
      const int gh = c & ((1 << gl) - 1);
      Lc[cb] = 0;
#pragma unroll
      for (int mm = 0; mm < KM; ++mm) qb[cb][mm] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (m < nm) {
        Lc[cb] = min(pre, seq_len(a, lead + m));
        const f16* qrow = a.q + ((size_t)(lead + m) * a.Hq + (head << gl) + gh) * D;
#pragma unroll
        for (int mm = 0; mm < KM; ++mm) qb[cb][mm] = *reinterpret_cast<const f16x8*>(qrow + k_dim_of<ELEM>(mm, grp));
      }
    }

    f32x4 o[CB][NT];
    float m_run[CB], l_part[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      m_run[cb] = -INFINITY;
      l_part[cb] = 0.0f;
#pragma unroll
      for (int c = 0; c < NT; ++c) o[cb][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int32_t* tab = a.tables + (size_t)first * a.max_blocks;  // the group's first sequence
    const uint8_t* kc_head = a.kc + (size_t)head * head_bytes;
    const uint8_t* vc_head = a.vc + (size_t)head * head_bytes;
    // Units are software-pipelined: the loads of unit j + 1 are in flight while
    // unit j is computed. Every issue is unconditional (a tile outside the pool
    // reads block 0 and is masked after the load; the last issue of a run
    // repeats its last unit), so the wait before a unit's arithmetic covers
    // only that unit's loads.
    struct Ld {
      u32x4 ka[KLD], kb[KLD], vv[VLD];
    };
    for (int j0 = u0; j0 < u1; j0 += 32) {
      // block ids of up to 32 units (two tiles each), one per lane
      int my_blk = -1;
      {
        const int jj = j0 + (lane >> 1);
        const int tt = 32 * jj + 16 * (lane & 1);
        if (jj < u1 && tt < pre) my_blk = tab[tt >> a.bs_log2];
      }
      const int nj = min(32, u1 - j0);
      auto tile_ok = [&](int j, int half) {
        return (unsigned)__builtin_amdgcn_readlane(my_blk, 2 * j + half) < (unsigned)a.num_blocks;
      };
      auto issue = [&](int j, Ld& d) {
        const int ta = 32 * (j0 + j);
        const int blk_a = __builtin_amdgcn_readlane(my_blk, 2 * j);
        const int blk_b = __builtin_amdgcn_readlane(my_blk, 2 * j + 1);
        const size_t off_a = (unsigned)blk_a < (unsigned)a.num_blocks
                                 ? (size_t)blk_a * blk_stride + (size_t)(ta & bs_mask) * RB : 0;
        const size_t off_b = (unsigned)blk_b < (unsigned)a.num_blocks
                                 ? (size_t)blk_b * blk_stride + (size_t)((ta + 16) & bs_mask) * RB : 0;
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
          d.ka[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kc_head + off_a + k_lane_off + 64 * i));
          d.kb[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kc_head + off_b + k_lane_off + 64 * i));
        }
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
          const size_t voff = i * RPL >= 16 ? off_b : off_a;
          const int r = (i * RPL + v_row) & 15;
          d.vv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vc_head + voff + r * RB + v_cb));
        }
      };
      auto compute = [&](const Ld& d, int j) {
        const int ta = 32 * (j0 + j);
        const bool ok_a = tile_ok(j, 0);
        const bool ok_b = tile_ok(j, 1);

        // S = K . Q^T for both tiles and both column blocks
        f32x4 sa[CB], sb[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          sa[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
          sb[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int m = 0; m < KM; ++m) {
          f16x8 aa, ab;
          if constexpr (FP8) {
            aa = fp8x8_to_f16x8<FMT>(d.ka[m / 2][(m % 2) * 2], d.ka[m / 2][(m % 2) * 2 + 1]);
            ab = fp8x8_to_f16x8<FMT>(d.kb[m / 2][(m % 2) * 2], d.kb[m / 2][(m % 2) * 2 + 1]);
          } else {
            aa = f16x8_from_u32x4(d.ka[m]);
            ab = f16x8_from_u32x4(d.kb[m]);
          }
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            sa[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aa, qb[cb][m], sa[cb], 0, 0, 0);
            sb[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ab, qb[cb][m], sb[cb], 0, 0, 0);
          }
        }

        // online softmax per column; tokens of this lane: ta+4grp+v, ta+16+4grp+v
        f16x8 pb[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          float z[8];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int tka = ta + 4 * grp + v;
            const int tkb = ta + 16 + 4 * grp + v;
            z[v] = (ok_a && tka < Lc[cb]) ? sa[cb][v] * qk_scale : -INFINITY;
            z[4 + v] = (ok_b && tkb < Lc[cb]) ? sb[cb][v] * qk_scale : -INFINITY;
          }
          // the running max (log2 units) moves only when some lane's logits
          // exceed it by more than kLazy (p <= 2^kLazy, well inside fp16)
          float mt = z[0];
#pragma unroll
          for (int i = 1; i < 8; ++i) mt = fmaxf(mt, z[i]);
          if (__builtin_amdgcn_ballot_w64(mt > m_run[cb] + kLazy)) {
            mt = fmaxf(mt, shfl_xor_f32(mt, 16));
            mt = fmaxf(mt, shfl_xor_f32(mt, 32));
            const float mn = fmaxf(m_run[cb], mt);
            const float alpha = fast_exp2(m_run[cb] - safe_max(mn));
            l_part[cb] *= alpha;
#pragma unroll
            for (int c = 0; c < NT; ++c) o[cb][c] *= alpha;
            m_run[cb] = mn;
          }
          const float ms = safe_max(m_run[cb]);
          float ps = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float p = fast_exp2(z[i] - ms);
            ps += p;
            pb[cb][i] = (_Float16)p;
          }
          l_part[cb] += ps;
        }

        // V rows -> LDS as fp16 (rows of tiles outside the pool or past the prefix as zeros)
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
          const int r = i * RPL + v_row;  // 0..31
          const bool ok = r < 16 ? ok_a : ok_b;
          _Float16* dst = vbuf + r * VS + v_cb / ELEM;
          if constexpr (FP8) {
            const f16x8 lo = ok ? fp8x8_to_f16x8<FMT>(d.vv[i][0], d.vv[i][1]) : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
            const f16x8 hi = ok ? fp8x8_to_f16x8<FMT>(d.vv[i][2], d.vv[i][3]) : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
            *reinterpret_cast<f16x8*>(dst) = lo;
            *reinterpret_cast<f16x8*>(dst + 8) = hi;
          } else {
            *reinterpret_cast<u32x4*>(dst) = ok ? d.vv[i] : u32x4{0u, 0u, 0u, 0u};
          }
        }

        // O^T += V^T . P^T, one 16-wide d tile at a time, both column blocks
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const _Float16* p1 = vbuf + tr_row * VS + 16 * c + tr_col;
          const _Float16* p2 = vbuf + (16 + tr_row) * VS + 16 * c + tr_col;
          const f16x4 r1 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1)));
          const f16x4 r2 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p2)));
          const f16x8 va = __builtin_shufflevector(r1, r2, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) o[cb][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[cb], o[cb][c], 0, 0, 0);
        }
      };
      Ld A, B;
      issue(0, A);
      for (int j = 0; j < nj; j += 2) {
        issue(min(j + 1, nj - 1), B);
        compute(A, j);
        if (j + 1 >= nj) break;
        issue(min(j + 2, nj - 1), A);
        compute(B, j + 1);
      }
    }

    // per-column sums over the four lane groups; the max is already common
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      l_part[cb] += shfl_xor_f32(l_part[cb], 16);
      l_part[cb] += shfl_xor_f32(l_part[cb], 32);
    }

    // lane (column col, group grp) holds d = 16c + 4grp + v of its column
    const bool whole = u0 == 0 && u1 == ug;
    const int slot = t == start ? 0 : 1;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = cb * 16 + col;
      const int m = c >> gl;
      if (m < nm) {
        const size_t pi = whole ? (size_t)(lead + m) * a.Hq + (head << gl) + (c & ((1 << gl) - 1))
                                : ((size_t)w * 2 + slot) * kSharedCols + c;
        float* orow = (whole ? a.ws_swo : a.ws_so) + pi * D + 4 * grp;
        float* ml = whole ? a.ws_swml : a.ws_sml;
#pragma unroll
        for (int d = 0; d < NT; ++d) *reinterpret_cast<f32x4*>(orow + 16 * d) = o[cb][d] * v_scale;
        if (grp == 0) {
          ml[2 * pi] = m_run[cb];
          ml[2 * pi + 1] = l_part[cb];
        }
      }
    }
    t = next_t;
  }
}

}  // namespace
}  // namespace pkv
