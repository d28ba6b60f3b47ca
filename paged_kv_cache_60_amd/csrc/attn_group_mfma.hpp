// Pass 1 of paged_attn_decode_shared: decode attention for a batch in which
// runs of sequences share their leading blocks, on the matrix cores. Included
// by attn_decode.hip after attn_gqa_mfma.hpp, whose operand layouts it uses,
// and whose AttnArgs, work split and merge helpers it shares.
//
// Sequences forked from one prompt (beams, parallel samples) and requests
// mapped onto the same prefix-cache blocks hold the same physical blocks at
// the start of their tables ("vLLM Architecture and Memory Use, ch. 3", §3.2;
// "Where Did the VRAM Go (KV cache tutorial)", §4.2-4.4). Decoding them one by
// one reads those blocks once per sequence. Here a group's members are cut
// into parts of up to 32 query columns (member c / G, query head c % G of the
// KV head), and one pass over a part reads the shared blocks once and
// contracts them with every column at once:
//   S = K . Q^T      M = 16 tokens, N = 32 query columns (two 16-column blocks),
//                    K-dim = d
//   O^T += V^T . P^T M = 16 d, N = 32 query columns, K-dim = 32 tokens
// The same pass then walks each member's own tokens past the shared ones (its
// tail: the partly filled block, divergent beams, a private suffix) through
// that member's table, with only that member's columns live; the column block
// that holds no live column skips its matrix products. A sequence in no group
// is a part of one member with no shared tokens.
//
// Work split. A segment is one (KV head, part); its units (32 tokens) are
// kPieceCost units of setup charge (no data), the shared units, then each
// member's tail units in member order. The units of
// a part are counted against its members (the shared units against the first),
// so a prefix over the batch sequences locates any unit; segments are laid end
// to end, KV head major, and cut into equal shares, one per worker (a wave),
// as in pass 1 of paged_attn_decode. A worker walks its share piece by piece;
// a piece that is a whole segment writes its columns' outputs directly, any
// other piece leaves (max, sum, output / sum in fp16) per column in the
// worker's slot 0 (first piece of the share) or 1 (last), which
// attn_reduce_group_kernel combines.
//
// Online softmax per column, with the running max moving only when a logit
// exceeds it by more than 2^8 (as on the grouped-head path). Rows at or past
// a region's end and tiles outside the pool are masked in the logits and
// staged as zeros for the P.V product.

namespace pkv {
namespace {

constexpr int kGroupCols = 32;  // query columns of one part
// Units of work a segment's start is charged in the split, for the setup a
// piece pays before its first data (query and table reads, then K/V: about
// two units' streaming time, measured): a worker whose share crosses into a
// new segment then streams that much less, instead of finishing last.
constexpr int kPieceCost = 2;

// Per-sequence part record (LDS, and the workspace for the merge): member
// index within its part (5 bits), members of the part (6 bits), shared tokens
// of its group / 16 (20 bits).
__device__ __forceinline__ int pack_part(int pre16, int nm, int mi) { return (pre16 << 11) | (nm << 5) | mi; }
__device__ __forceinline__ int part_mi(int v) { return v & 31; }
__device__ __forceinline__ int part_nm(int v) { return (v >> 5) & 63; }
__device__ __forceinline__ int part_pre(int v) { return (v >> 11) << 4; }

// Units counted against sequence i: its tail past the shared tokens, plus the
// part's setup charge and shared units if it is the part's first member.
__device__ __forceinline__ int group_seq_units(int v, int L) {
  const int pre = part_pre(v);
  const int tail = L > pre ? (L - pre + 31) / 32 : 0;
  return tail + (part_mi(v) == 0 ? kPieceCost + (pre + 31) / 32 : 0);
}

// info[B]: every sequence's part record; pt[B + 1]: the unit prefix over the
// sequences. A group of n members splits into parts of kGroupCols / G members;
// a sequence in no group is a part of its own. The three entries of the first
// blockDim groups and the context lengths are all loaded before the first
// wait (one round trip to memory, not one per array); ends with a barrier.
__device__ void build_group_parts(const AttnArgs& a, int* pt, int* scan, int* info) {
  const int T = blockDim.x;
  const int tid = threadIdx.x;
  const int MP = kGroupCols >> a.g_log2;
  int f0 = -1, s0 = 0, p0 = 0;
  if (tid < a.NG) {
    f0 = a.grp_first[tid];
    s0 = a.grp_size[tid];
    p0 = a.grp_prefix[tid];
  }
  for (int i = tid; i < a.B; i += T) {
    info[i] = pack_part(0, 1, 0);
    pt[i + 1] = seq_len(a, i);
  }
  __syncthreads();
  for (int g = tid; g < a.NG; g += T) {
    const int f = g == tid ? f0 : a.grp_first[g];
    const int n = group_members(a, f, g == tid ? s0 : a.grp_size[g]);
    if (n == 0) continue;
    const int pre_g = group_tokens(a, g == tid ? p0 : a.grp_prefix[g]);
    for (int m = 0; m < n; ++m) {
      const int part = m / MP;
      // a part reads the shared tokens through its first member's table: no
      // more of them than that member holds (pt[i + 1] is still sequence i's
      // length here); past 2^20 * 16 shared tokens the rest are taken as each
      // member's own
      const int pre = min(pre_g, pt[f + part * MP + 1] & ~15);
      info[f + m] = pack_part(min(pre >> 4, (1 << 20) - 1), min(MP, n - part * MP), m - part * MP);
    }
  }
  __syncthreads();
  build_scan(a.B, pt, scan, [&](int i) { return group_seq_units(info[i], pt[i + 1]); });
}

// Waves per SIMD of the grouped pass 1: fp8 units hold half the bytes of
// fp16 ones, so with one wave per SIMD an fp8 unit's arithmetic (widening,
// the matrix products, the softmax, V through LDS) outlasts its loads; two
// waves per SIMD (221 registers, no spill) overlap one wave's arithmetic with
// the other's loads. fp16 keeps one wave per SIMD (two measured slower).
// Either way each wave has one unit of loads in flight: more bytes in flight
// only queue (fp16 with two units: 280.8 against 278.0 us on a Qwen3 batch,
// and 276.5 against 274.4 us with the arithmetic taken out).
template <int FMT>
constexpr int group_waves_per_simd() { return FMT != kF16 ? 2 : 1; }

template <int D, int FMT, int NW>
__global__ void __launch_bounds__(NW * 64, group_waves_per_simd<FMT>()) attn_group_mfma_kernel(AttnArgs a) {
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
  constexpr int CB = kGroupCols / 16;   // 16-column blocks
  // units whose loads are in flight at once, per wave (group_waves_per_simd)
  constexpr int DEPTH = 1;
  static_assert(CB == 2, "two column blocks");
  static_assert(RPL <= 16 && 16 % RPL == 0, "a V load stays inside one tile");

  __shared__ __align__(16) _Float16 vlds[NW * 32 * VS];
  extern __shared__ int dyn_smem[];
  int* pt = dyn_smem;              // [B + 1]
  int* scan = pt + a.B + 1;        // [NW * 64]
  int* info = scan + NW * 64;      // [B]
  build_group_parts(a, pt, scan, info);

  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int gl = a.g_log2;
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i <= a.B; i += NW * 64) a.ws_pt[i] = pt[i];
    for (int i = threadIdx.x; i < a.B; i += NW * 64) {
      const int v = info[i];
      a.ws_part[i] = v;
      // the part's units in the unit prefix ((0, 0), no units, for a part
      // that would reach past the batch: only inconsistent group entries)
      const int pf = i - part_mi(v), pe = pf + part_nm(v);
      const bool ok = pf >= 0 && pe <= a.B;
      *reinterpret_cast<int2*>(a.ws_seg + 2 * i) = ok ? make_int2(pt[pf], pt[pe]) : make_int2(0, 0);
    }
  }
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
  const int v_row = lane / LPR;
  const int v_cb = (lane % LPR) * 16;
  const int tr_row = 4 * grp + (col >> 2);
  const int tr_col = 4 * (col & 3);

  for (int64_t t = start; t < end;) {
    // the piece at unit t: (KV head, part), units [u0, u1) of the segment
    const int head = (int)(t / P);
    const int rem = (int)(t - (int64_t)head * P);
    const int s = find_seq(pt, a.B, rem);
    // the part from s's own record (every member's record names the same
    // part; taking one keeps pf + nm inside the batch even for overlapping
    // group entries)
    const int sinfo = wave_uniform(info[s]);
    const int pf = s - part_mi(sinfo);  // the part's first member
    const int nm = part_nm(sinfo);
    const int pre = part_pre(sinfo);
    const int US = kPieceCost + (pre + 31) / 32;  // end of the charge and the shared units
    const int seg0 = wave_uniform(pt[pf]);
    const int n_u = wave_uniform(pt[pf + nm]) - seg0;
    const int u0 = rem - seg0;
    const int64_t seg_end = t - u0 + n_u;
    const int64_t next_t = end < seg_end ? end : seg_end;
    const int u1 = u0 + (int)(next_t - t);
    // The piece's setup loads -- the members' lengths, the query columns and
    // the first batch's table entries -- are all issued before the first wait
    // (one round trip): a load behind a branch leaves the compiler unsure,
    // where the paths join, how many loads are in flight, and the wait it puts
    // there costs a round trip per load.
    // lane m < nm: member m's context length (lanes past nm read the last one's)
    const int Lraw = seq_len(a, pf + min(lane, nm - 1));
    // lane column cb*16+col -> member memc[cb], query head gh; a column past
    // the part's members reads the first member's query and is zeroed below
    f16x8 qb[CB][KM];
    int memc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = cb * 16 + col;
      const int m = c >> gl;
      const int gh = c & ((1 << gl) - 1);
      memc[cb] = m;
      const f16* qrow = a.q + ((size_t)(pf + (m < nm ? m : 0)) * a.Hq + (head << gl) + gh) * D;
#pragma unroll
      for (int mm = 0; mm < KM; ++mm) qb[cb][mm] = *reinterpret_cast<const f16x8*>(qrow + k_dim_of<ELEM>(mm, grp));
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

    const uint8_t* kc_head = a.kc + (size_t)head * head_bytes;
    const uint8_t* vc_head = a.vc + (size_t)head * head_bytes;

    struct Ld {
      u32x4 ka[KLD], kb[KLD], vv[VLD];
    };
    // Descriptors of a batch of up to 32 units of the piece: lane l holds tile
    // l & 1 of unit b0 + l / 2 -- its block id (-1 or past the pool: masked),
    // the unit's first token and its live member (-1: shared tokens,
    // every column live; nm: none). Every region of the batch is resolved here
    // at once, so that the loads run on across region edges without a
    // dependent table read between them. Every lane reads a table entry (the
    // index clamped into the row), so that the read is not behind a branch.
    struct Desc {
      int blk, ta, mem;
    };
    auto describe = [&](int b0) {
      Desc d{-1, 0, -1};
      const int u = b0 + (lane >> 1);
      int m = -1, ts = 0;
      if (u >= US && u < u1) {
        // the member whose tail holds unit u (tails follow one another);
        // none only for inconsistent group entries: the unit is then masked
        m = nm;
        for (int k = 0; k < nm; ++k) {
          const int s_k = pt[pf + k] - seg0 + (k == 0 ? US : 0);
          const int e_k = pt[pf + k + 1] - seg0;
          if (u >= s_k && u < e_k) {
            m = k;
            ts = s_k;
            break;
          }
        }
      }
      // the table entry is read whatever the member's length (an entry past
      // it is in the table and its rows are masked)
      const int row = m < 0 ? pf : pf + (m < nm ? m : 0);
      d.ta = m < 0 ? 32 * (u - kPieceCost) : pre + 32 * (u - ts);
      d.mem = m;
      const int idx = min(max((d.ta + 16 * (lane & 1)) >> a.bs_log2, 0), a.max_blocks - 1);
      // (lanes past the piece, u >= u1, are never read: a batch processes its
      // first min(32, u1 - b0) units)
      d.blk = a.tables[(size_t)row * a.max_blocks + idx];
      return d;
    };

    // the setup loads are in flight; their uses follow
    const int ud = max(u0, kPieceCost);  // the setup charge holds no data
    Desc cur = describe(ud);
    const int Lm = lane < nm ? Lraw : 0;
    int Lc[CB];  // each column's length against the shared tokens
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int m = memc[cb];
      const int Lmem = __shfl(Lm, m < nm ? m : 0, 64);
      Lc[cb] = m < nm ? min(pre, Lmem) : 0;
      if (m >= nm) {
#pragma unroll
        for (int mm = 0; mm < KM; ++mm) qb[cb][mm] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
    // the shortest live column's shared tokens: shared units below it need no masks
    int Lmin_sh = pre;
    for (int m = 0; m < nm; ++m) Lmin_sh = min(Lmin_sh, __builtin_amdgcn_readlane(Lm, m));
    // the logit and output scales of the head (both loads at once)
    float qk_scale = a.qk_scale, v_scale = a.v_out_scale;
    if (a.k_scale_h) {
      const float ks = a.k_scale_h[head];
      const float vs = a.v_scale_h[head];
      qk_scale = a.qk_base * ks;
      v_scale = vs;
    }

    // One unit: S for the live column blocks, online softmax, V to LDS, O += P.V.
    // mact: the live member (-1: every column, each masked at its Lc); live0,
    // live1 (wave-uniform): the column blocks holding live columns; rows are
    // valid below Lreg, and a unit whose 32 tokens all lie below Lfull (and
    // whose tiles are in the pool) needs no masks.
    auto compute = [&](const Ld& d, int ta, bool ok_a, bool ok_b, int Lreg, int Lfull, int mact, bool live0,
                       bool live1) {
      const bool full = ok_a && ok_b && ta + 32 <= Lfull;

      // S = K . Q^T for both tiles, live column blocks
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
        if (live0) {
          sa[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aa, qb[0][m], sa[0], 0, 0, 0);
          sb[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ab, qb[0][m], sb[0], 0, 0, 0);
        }
        if (live1) {
          sa[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aa, qb[1][m], sa[1], 0, 0, 0);
          sb[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ab, qb[1][m], sb[1], 0, 0, 0);
        }
      }

      // online softmax per live column; tokens of this lane: ta+4grp+v, ta+16+4grp+v
      f16x8 pb[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        if (!(cb == 0 ? live0 : live1)) continue;
        const int Lcol = mact < 0 ? Lc[cb] : Lreg;
        float z[8];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          z[v] = sa[cb][v] * qk_scale;
          z[4 + v] = sb[cb][v] * qk_scale;
        }
        if (!full) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            if (!(ok_a && ta + 4 * grp + v < Lcol)) z[v] = -INFINITY;
            if (!(ok_b && ta + 16 + 4 * grp + v < Lcol)) z[4 + v] = -INFINITY;
          }
        }
        if (mact >= 0 && memc[cb] != mact) {  // a column of another member
#pragma unroll
          for (int i = 0; i < 8; ++i) z[i] = -INFINITY;
        }
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

      // V rows -> LDS as fp16; rows past the region or in tiles outside the pool as zeros
#pragma unroll
      for (int i = 0; i < VLD; ++i) {
        const int r = i * RPL + v_row;  // 0..31
        const bool ok = full || ((r < 16 ? ok_a : ok_b) && ta + r < Lreg);
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

      // O^T += V^T . P^T, one 16-wide d tile at a time, live column blocks
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        const _Float16* p1 = vbuf + tr_row * VS + 16 * c + tr_col;
        const _Float16* p2 = vbuf + (16 + tr_row) * VS + 16 * c + tr_col;
        const f16x4 r1 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1)));
        const f16x4 r2 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p2)));
        const f16x8 va = __builtin_shufflevector(r1, r2, 0, 1, 2, 3, 4, 5, 6, 7);
        if (live0) o[0][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[0], o[0][c], 0, 0, 0);
        if (live1) o[1][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[1], o[1][c], 0, 0, 0);
      }
    };

    // batches of 32 units; the next batch's descriptors (table reads) are in
    // flight while the current batch streams
    for (int b0 = ud; b0 < u1; b0 += 32) {
      const Desc nxt = b0 + 32 < u1 ? describe(b0 + 32) : Desc{-1, 0, -1};
      const int nj = min(32, u1 - b0);
      auto issue = [&](int j, Ld& d) {
        const int ta = __builtin_amdgcn_readlane(cur.ta, 2 * j);
        const int blk_a = __builtin_amdgcn_readlane(cur.blk, 2 * j);
        const int blk_b = __builtin_amdgcn_readlane(cur.blk, 2 * j + 1);
        // a tile outside the pool (or past its region) reads block 0 and is masked
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
      auto unit = [&](const Ld& d, int j) {
        const int ta = __builtin_amdgcn_readlane(cur.ta, 2 * j);
        const int mem = __builtin_amdgcn_readlane(cur.mem, 2 * j);
        // rows are valid below the shared tokens, the live member's length, or
        // nowhere (no member)
        const int len = mem < 0 ? pre : (mem < nm ? __builtin_amdgcn_readlane(Lm, mem) : 0);
        const bool ok_a = (unsigned)__builtin_amdgcn_readlane(cur.blk, 2 * j) < (unsigned)a.num_blocks;
        const bool ok_b = (unsigned)__builtin_amdgcn_readlane(cur.blk, 2 * j + 1) < (unsigned)a.num_blocks;
        // a member's columns lie in one 16-column block
        const bool live0 = mem < 0 || ((mem << gl) >> 4) == 0;
        const bool live1 = mem < 0 || ((mem << gl) >> 4) != 0;
        compute(d, ta, ok_a, ok_b, len, mem < 0 ? Lmin_sh : len, mem, live0, live1);
      };
      // software pipelined over a ring of DEPTH load buffers: the loads of
      // units j + 1 .. j + DEPTH - 1 are in flight while unit j is computed
      Ld ring[DEPTH];
#pragma unroll
      for (int k = 0; k < DEPTH - 1; ++k)
        if (k < nj) issue(k, ring[k]);
      for (int j = 0; j < nj; j += DEPTH) {
#pragma unroll
        for (int k = 0; k < DEPTH; ++k) {
          if (j + k >= nj) break;
          if (j + k + DEPTH - 1 < nj) issue(j + k + DEPTH - 1, ring[(k + DEPTH - 1) % DEPTH]);
          unit(ring[k], j + k);
        }
      }
      cur = nxt;
    }

    // per-column sums over the four lane groups; the max is already common
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      l_part[cb] += shfl_xor_f32(l_part[cb], 16);
      l_part[cb] += shfl_xor_f32(l_part[cb], 32);
    }

    // lane (column col, group grp) holds d = 16c + 4grp + v of its column
    const bool whole = u0 == 0 && u1 == n_u;
    const int slot = t == start ? 0 : 1;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = cb * 16 + col;
      const int m = memc[cb];
      if (m >= nm) continue;
      if (whole) {
        const float sc = l_part[cb] > 0.0f ? v_scale / l_part[cb] : 0.0f;
        f16* orow = a.out + ((size_t)(pf + m) * a.Hq + (head << gl) + (c & ((1 << gl) - 1))) * D + 4 * grp;
#pragma unroll
        for (int d = 0; d < NT; ++d) {
          f16x4 h;
#pragma unroll
          for (int v = 0; v < 4; ++v) h[v] = (f16)(o[cb][d][v] * sc);
          *reinterpret_cast<f16x4*>(orow + 16 * d) = h;
        }
      } else {
        // the piece's output divided by its own sum, as fp16: a weighted mean
        // of V rows, so within V's range, at half the bytes of fp32 partials
        // (every share of a grouped launch is usually a piece of a segment,
        // so these bytes are written and read again on every step)
        const size_t pi = ((size_t)w * 2 + slot) * kGroupCols + c;
        const float sc = l_part[cb] > 0.0f ? v_scale / l_part[cb] : 0.0f;
        f16* orow = reinterpret_cast<f16*>(a.ws_o) + pi * D + 4 * grp;
#pragma unroll
        for (int d = 0; d < NT; ++d) {
          f16x4 h;
#pragma unroll
          for (int v = 0; v < 4; ++v) h[v] = (f16)(o[cb][d][v] * sc);
          *reinterpret_cast<f16x4*>(orow + 16 * d) = h;
        }
        if (grp == 0) {
          a.ws_ml[2 * pi] = m_run[cb];
          a.ws_ml[2 * pi + 1] = l_part[cb];
        }
      }
    }
    t = next_t;
  }
}

// Pass 2 of paged_attn_decode_shared. One wave per (sequence, query head):
// combines the pieces of its part's segment that pass 1 split between
// workers (column = member index * G + query head within the group); a part
// held whole by one worker was written by pass 1; a part with no units
// (every member empty) gets zeros.
template <int D, int G>
__global__ void __launch_bounds__(256) attn_reduce_group_kernel(AttnArgs a) {
  constexpr int DL = D / 64;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= a.B * a.Hq) return;
  const int lane = threadIdx.x & 63;
  const int seq = wid / a.Hq;
  const int hq = wid - seq * a.Hq;
  const int kvh = hq / G;
  const int g = hq - kvh * G;
  // the part record, the part's unit range and the unit total in one round trip
  const int v = a.ws_part[seq];
  const int2 sg = *reinterpret_cast<const int2*>(a.ws_seg + 2 * seq);
  const int P = a.ws_pt[a.B];
  const int mi = part_mi(v);
  f16* out = a.out + (size_t)wid * D + lane * DL;
  Row<DL> r;
  const int64_t total = (int64_t)a.Hkv * P;
  const int64_t s0 = (int64_t)kvh * P + sg.x;
  const int64_t s1 = (int64_t)kvh * P + sg.y;
  if (s1 > s0) {
    if (held_whole(s0, s1, total, a.workers)) return;  // written by pass 1
    fold_pieces<D, f16, 16>(r, reinterpret_cast<const f16*>(a.ws_o), a.ws_ml, kGroupCols, mi * G + g, s0, s1,
                            total, a.workers);
  }
  write_row(r, out);
}

}  // namespace
}  // namespace pkv
