// decode_mfma.hip — paged-attention decode for grouped-query heads on the matrix cores.
//
// Same method as the vector kernel ("vLLM 深度拆解：当 KV Cache 学会「分页」" §2.2 formula, §3.3
// block-table walk with the context-length stop, §6.2 arguments and scale), but one work
// segment is a (sequence, KV head) pair and all G = Hq / Hkv query heads that share the KV
// head are scored together: per 32-token unit (two 16-token blocks) the wavefront runs
//   S^T = K . Q^T  as 2 x (D/32) MFMA 16x16x32  (M = 16 tokens, N = 16 head columns, G used)
//   O  += P . V    as (D/16) MFMA 16x16x32     (M = 16 head rows, N = 16 dims, K = 32 tokens)
// Each K and V byte is read once for all G heads.  The 16 MFMA columns hold (row, head)
// pairs, so a sequence with nr <= 16 / G causal query rows (the verify pass of speculative
// decoding, "vLLM 深度拆解" §5.1: the target model checks several drafted tokens in one pass)
// is one segment of nr * G columns whose K and V are also read once.
//
// Operand layouts, the token permutation that keeps scores in place, and the hi/lo split
// of P are described in pa_mfma.h.
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma.h"

namespace pa {

// All query columns of KV head g for sequence s over the units [u0, u1) (32 tokens each).
// Without MULTI the columns are the G query heads of one decode row (nr = 1).  With MULTI a
// column is one (row, query head) pair: column c is row qsl[s] + c / G, head g * G + c % G,
// and the nr * G <= 16 columns of the sequence's nr rows are scored together.  Row j sits at
// position ctx - nr + j and sees keys [0, ctx - nr + j].
template <int DT, int D, bool MULTI, bool LEAN, bool B8>
__device__ void mfma_attend(const DecodeArgs& a, int s, int g, int u0, int u1, int ctx, int nr,
                            MfmaState<DT, D>& st) {
  using C = MfmaCfg<DT, D>;
  using T = op8_t<DT>;
  const int lane = lane_id();
  const int r = lane >> 4, n = lane & 15;
  // every per-piece value is wave-uniform: keep it in scalar registers
  s = __builtin_amdgcn_readfirstlane(s);
  g = __builtin_amdgcn_readfirstlane(g);
  u0 = __builtin_amdgcn_readfirstlane(u0);
  u1 = __builtin_amdgcn_readfirstlane(u1);
  ctx = __builtin_amdgcn_readfirstlane(ctx);
  const int G = a.num_q_heads / a.num_kv_heads;
  const int row0 = __builtin_amdgcn_readfirstlane(a.qsl ? a.qsl[s] : s);
  // this lane's column: row offset and head
  const int jr = MULTI ? n / G : 0;
  const int hc = MULTI ? n - jr * G : n;
  if constexpr (MULTI) nr = __builtin_amdgcn_readfirstlane(nr);

  // Scores are formed with the factor sl > 0: a negative factor is folded into q (sign flips
  // are exact) and a zero factor makes every score 0 (q = 0, factor 1).
  const float sl = a.scale_log2 == 0.f ? 1.f : fabsf(a.scale_log2);
  const uint32_t qflip = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  T qb[C::NKK];
  {
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     ((int64_t)(row0 + jr) * a.num_q_heads + (int64_t)g * G + hc) * D * 2;
    const bool live = (MULTI ? jr < nr : n < G) && a.scale_log2 != 0.f;
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
      uint4 v = live ? ld16(qp + (4 * kk + r) * 16) : make_uint4(0, 0, 0, 0);
      v.x ^= qflip;
      v.y ^= qflip;
      v.z ^= qflip;
      v.w ^= qflip;
      qb[kk] = __builtin_bit_cast(T, v);
    }
  }
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) st.acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if constexpr (!MULTI) {
    mfma_stream<DT, D, B8>(a, s, g, u0, u1, ctx, [&](MfmaK<DT, D>& kb, MfmaV<DT, D>& vb, int u) {
      const int valid = ctx - u * kMfmaUnit;
      if (valid >= kMfmaUnit)
        mfma_unit<DT, D, false, false>(st, kb, vb, qb, sl, kMfmaUnit - 1, kMfmaUnit);
      else
        mfma_unit<DT, D, true, false>(st, kb, vb, qb, sl, valid - 1, valid);
    });
  } else {
    const int last0 = ctx - nr;                 // last visible key of the first row
    const int mine = min(last0 + jr, ctx - 1);  // ... of this lane's column (padding: ctx - 1)
    auto scores = [&](MfmaK<DT, D>& kb, int u) {
      const int t0 = u * kMfmaUnit;
      if (last0 - t0 >= kMfmaUnit - 1)  // every column sees the whole unit
        return mfma_scores<DT, D, false, false>(st, kb, qb, sl, kMfmaUnit - 1);
      // per-column limits; a column may see no key of this piece yet
      return mfma_scores<DT, D, true, true>(st, kb, qb, sl, mine - t0);
    };
    auto pv = [&](MfmaV<DT, D>& vb, const MfmaP<DT>& p, int u) {
      const int t0 = u * kMfmaUnit;
      if (last0 - t0 >= kMfmaUnit - 1)
        mfma_pv<DT, D, false>(st, vb, p, kMfmaUnit);
      else
        mfma_pv<DT, D, true>(st, vb, p, ctx - t0);
    };
    if constexpr (LEAN) {
      mfma_stream_lean<DT, D, B8>(a, s, g, u0, u1, ctx, scores, pv);
    } else {
      mfma_stream<DT, D, B8>(a, s, g, u0, u1, ctx, [&](MfmaK<DT, D>& kb, MfmaV<DT, D>& vb, int u) {
        pv(vb, scores(kb, u), u);
      });
    }
  }
  if constexpr (is_fp8(DT)) {
    // a stored V value stands for its E4M3 value times v_scale (k_scale is in scale_log2)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) st.acc[j] *= a.v_factor;
  }
}

// Folds the np shared-prefix partials of (row, query head h) into a merged column held as
// (M, L, U): this lane's dimensions 16 j + 4 r + i are U[4 j + i].
template <int D>
__device__ __forceinline__ void m_fold(const DecodeArgs& a, float& M, float& L,
                                       float (&U)[4 * (D / 16)], int64_t row, int h, int np) {
  const int r = lane_id() >> 4;
  const int64_t e = (row * a.num_q_heads + h) * a.pre_parts;
  fold_prefix<4 * (D / 16), 2>(M, L, U, a.pre_m + e, a.pre_l + e, a.pre_o + e * D, D, np,
                               [&](int k) { return 16 * (k >> 2) + 4 * r + (k & 3); });
}

// Column n of a segment's first query row row0 and KV head g: its row and query head (one
// row without MULTI).
template <bool MULTI>
__device__ __forceinline__ void m_column(const DecodeArgs& a, int n, int row0, int g,
                                         int64_t& row, int& h, int& jr, int& hc) {
  const int G = a.num_q_heads / a.num_kv_heads;
  jr = MULTI ? n / G : 0;
  hc = MULTI ? n - jr * G : n;
  row = (int64_t)row0 + jr;
  h = g * G + hc;
}

// A whole segment of a sequence with a shared prefix: its keys past the prefix, folded with
// the prefix partials of each column, written to `out` (the segment's first column at ob).
template <int DT, int D, bool MULTI>
__device__ void m_prefix_emit(const DecodeArgs& a, const MfmaState<DT, D>& st, int ncols,
                              int row0, int g, int np, int64_t ob) {
  using C = MfmaCfg<DT, D>;
  constexpr int NE = 4 * C::NJ;
  const int lane = lane_id();
  const int r = lane >> 4, n = lane & 15;
  float L = cross_rows_sum(st.l);
  if (n >= ncols) return;
  float M = st.m * 0.69314718055994531f;
  float U[NE];
#pragma unroll
  for (int j = 0; j < C::NJ; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) U[4 * j + i] = st.acc[j][i];
  int64_t row;
  int h, jr, hc;
  m_column<MULTI>(a, n, row0, g, row, h, jr, hc);
  m_fold<D>(a, M, L, U, row, h, np);
  const int64_t ocol = ob + ((int64_t)jr * a.num_q_heads + hc) * D;
  const float rinv = 1.f / L;
#pragma unroll
  for (int j = 0; j < C::NJ; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      store_out<DT>(a.out, ocol + 16 * j + 4 * r + i, U[4 * j + i] * rinv, a.out_f32);
}

// A piece of a split segment (the ncols query columns of one KV head): publish it, or, as
// the segment's last arrival, merge every piece and write the output (the segment's first
// column at ob; with np > 0 folded with the shared-prefix partials of each column, the
// segment's first row being row0).  Each lane merges its own column n and dimensions
// 16 j + 4 r .. + 3, so no lanes interact.  Partial slots hold a.cols columns.  The merge
// loads MB pieces at a time (LEAN: one, which keeps it within the 256 registers of two waves
// per SIMD).
template <int DT, int D, bool MULTI, int MB>
__device__ void m_split_finish(const DecodeArgs& a, const MfmaState<DT, D>& st, int ncols,
                               const SplitSeg& sg, int64_t self, int32_t* cnt, int seen,
                               int64_t ob, int row0, int g, int np) {
  using C = MfmaCfg<DT, D>;
  constexpr int NE = 4 * C::NJ;
  const int lane = lane_id();
  const int r = lane >> 4, n = lane & 15;
  const bool col = n < ncols;
  const int CS = MULTI ? a.cols : ncols;
  // this piece's partial as published: normalised output, max (natural log), sum
  const float ltot = cross_rows_sum(st.l);  // sum of column n over the four lane rows
  // with several rows a piece may hold no key of a column
  const float inv = MULTI ? (ltot > 0.f ? 1.f / ltot : 0.f) : 1.f / ltot;
  const float mine_m = st.m * 0.69314718055994531f;
  f32x4_t mine_o[C::NJ];
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) mine_o[j] = st.acc[j] * inv;
  const bool last = split_arrive(cnt, (int)(sg.k1 - sg.k0), seen, [&] {
    const int64_t slot = piece_slot(sg, self);
    if (col) {
      float* po = a.part_o + slot * CS * D;  // wave-uniform base of the slot
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) coh_store4(po, n * D + 16 * j + 4 * r, mine_o[j]);
      if (r == 0) {
        coh_store(a.part_m + slot * CS + n, mine_m);
        coh_store(a.part_l + slot * CS + n, ltot);
      }
    }
  }, [] {});
  if (!last) return;
  float M[1], L[1], U[1][NE];
  merge_ordered<1, NE, MB>(M, L, U, sg.k0, sg.k1,
                          [&](int64_t k, float (&m)[1], float (&lk)[1], float (&ov)[1][NE]) {
    if (k == self || !col) {
      m[0] = mine_m;
      lk[0] = ltot;
#pragma unroll
      for (int j = 0; j < C::NJ; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[0][4 * j + i] = mine_o[j][i];
      return;
    }
    const int64_t slot = piece_slot(sg, k);
    m[0] = coh_load(a.part_m + slot * CS + n);
    lk[0] = coh_load(a.part_l + slot * CS + n);
    const float* po = a.part_o + slot * CS * D;  // wave-uniform base of the slot
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
      const f32x4_t v = coh_load4(po, n * D + 16 * j + 4 * r);
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[0][4 * j + i] = v[i];
    }
  });
  if (col) {
    // column n: row offset n / G, head n % G (one row without MULTI)
    int64_t row;
    int h, jr, hc;
    m_column<MULTI>(a, n, row0, g, row, h, jr, hc);
    if (np > 0) m_fold<D>(a, M[0], L[0], U[0], row, h, np);
    const int64_t ocol = ob + ((int64_t)jr * a.num_q_heads + hc) * D;
    const float rinv = 1.f / L[0];
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        store_out<DT>(a.out, ocol + 16 * j + 4 * r + i, U[0][4 * j + i] * rinv, a.out_f32);
  }
  counter_reset(cnt);
}

// LEAN (multi-row batches whose chunk kernel runs beside this one) streams with one operand
// buffer and is built for two waves per SIMD: with ~340 registers per wave the decode
// kernel's waves keep the chunk kernel's off the CUs, and the two then run one after the
// other (mixed chunked-prefill step: 788 -> 646 us).  Alone, the two-buffer stream is faster.
template <int DT, int D, int MODE, bool MULTI, bool LEAN, bool B8>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(LEAN ? 2 : 1))) void
mfma_decode_kernel(DecodeArgs a) {
  extern __shared__ int32_t lds[];
  int32_t* base = lds;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int segs = a.num_kv_heads;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int S = a.num_seqs;
  const int64_t W = (int64_t)gridDim.x * kWavesPerWG;
  const int64_t w = (int64_t)blockIdx.x * kWavesPerWG + wave;

  if constexpr (MODE == MODE_EVEN) {
    PlanIn pin{a.context_lens, a.qsl, S, kMfmaUnit, a.seg_extra, a.max_rows, a.skip};
    build_plan(base, pin);
    zero_empty_rows<DT>(pin, a.out, a.num_q_heads, D, w, W, a.out_f32, a.nan_rows);
    // units: (sequence, group of kWavesPerWG KV heads, unit); wave i runs KV head i of each
    // group
    const int groups = (a.num_kv_heads + kWavesPerWG - 1) / kWavesPerWG;
    const Part part = make_part((int64_t)base[S] * groups, gridDim.x, a.odd_skew);
    even_split_drive(part, [&](int64_t o, int64_t lo, int64_t hi) {
      for (int64_t i = lo; i < hi;) {
        const int s = find_seq(base, S, i, groups);
        const int seglen = base[s + 1] - base[s];
        const int nu = seglen - a.seg_extra;  // real units; the rest only balance the split
        const int64_t sbase = (int64_t)base[s] * groups;
        const int grp = (int)((i - sbase) / seglen);
        const int64_t seg0 = sbase + (int64_t)grp * seglen;
        const int64_t pe = min(hi, seg0 + seglen);
        const int g = grp * kWavesPerWG + wave;  // this wave's KV head
        const int u0 = (int)(i - seg0), u1 = (int)min(pe - seg0, (int64_t)nu);
        if (g < a.num_kv_heads && u0 < nu) {
          const int ctx = a.context_lens[s];
          // keys [0, sk) come from the shared-prefix partials (np of them): the units start
          // past them
          const int sk = a.skip ? a.skip[s] : 0;
          const int us = sk / kMfmaUnit;
          const int np = sk > 0 ? (sk + a.pre_tokens - 1) / a.pre_tokens : 0;
          const int row = a.qsl ? a.qsl[s] : s;
          const int nr = MULTI ? a.qsl[s + 1] - row : 1;
          const bool whole = u0 == 0 && u1 == nu;
          SplitSeg sg{};
          int32_t* cnt = nullptr;
          int seen = 0;
          if (!whole) {
            sg = split_seg(part, seg0, seg0 + nu - 1, wave);
            cnt = a.counters + kWavesPerWG * sg.k0 + wave;
            seen = counter_peek(cnt);  // consumed after the units
          }
          MfmaState<DT, D> st;
          mfma_attend<DT, D, MULTI, LEAN, B8>(a, s, g, u0 + us, u1 + us, ctx, nr, st);
          // the segment's first column in `out`; column c is row + c / G, head g * G + c % G
          const int64_t ob = ((int64_t)row * a.num_q_heads + (int64_t)g * G) * D;
          if (whole && np > 0)
            m_prefix_emit<DT, D, MULTI>(a, st, nr * G, row, g, np, ob);
          else if (whole)
            mfma_emit<DT, D>(st, nr * G, nullptr, nullptr, nullptr, D, a.out, ob, MULTI ? G : 16,
                             (int64_t)a.num_q_heads * D, D, a.out_f32);
          else
            m_split_finish<DT, D, MULTI, LEAN ? 1 : 2>(a, st, nr * G, sg, o, cnt, seen, ob, row, g, np);
        }
        i = pe;
      }
    });
  } else {
    // fixed partitions of the sequences with one query row (with query_start_loc, the
    // others are the chunk kernel's)
    const int PU = a.partition_units;  // 32-token units per partition
    const int P = a.max_partitions;
    PlanIn pin{a.context_lens, a.qsl, S, PU * kMfmaUnit, 0, 1};
    build_plan(base, pin);
    fill_past_partitions(a.context_lens, a.qsl, S, a.qsl ? a.qsl[S] : S, a.num_q_heads, P,
                         PU * kMfmaUnit, a.part_m, a.part_l, w, W);
    const int64_t total = (int64_t)base[S] * segs;
    for (int64_t i = w; i < total; i += W) {
      const int s = find_seq(base, S, i, segs);
      const int np = base[s + 1] - base[s];
      const int64_t sbase = (int64_t)base[s] * segs;
      const int g = (int)((i - sbase) / np);
      const int p = (int)(i - sbase - (int64_t)g * np);
      const int ctx = a.context_lens[s];
      const int nu = (ctx + kMfmaUnit - 1) / kMfmaUnit;
      const int u0 = p * PU, u1 = min(nu, u0 + PU);
      MfmaState<DT, D> st;
      mfma_attend<DT, D, false, false, B8>(a, s, g, u0, u1, ctx, 1, st);
      // tmp_out [row][h][P][D]: consecutive heads are P * D apart
      const int64_t row = a.qsl ? a.qsl[s] : s;
      const int64_t e0 = (row * a.num_q_heads + (int64_t)g * G) * P + p;
      mfma_emit<DT, D>(st, G, a.part_o + e0 * D, a.part_m + e0, a.part_l + e0, (int64_t)P * D,
                       nullptr, 0, 16, 0, 0, false);
    }
  }
  (void)lane;
}

template <int DT, int MODE, bool MULTI, bool LEAN, bool B8>
static void launch_b(const DecodeArgs& a, int grid, size_t lds, hipStream_t st) {
  if (a.head_dim == 64)
    hipLaunchKernelGGL((mfma_decode_kernel<DT, 64, MODE, MULTI, LEAN, B8>), dim3(grid), dim3(kWG), lds, st, a);
  else
    hipLaunchKernelGGL((mfma_decode_kernel<DT, 128, MODE, MULTI, LEAN, B8>), dim3(grid), dim3(kWG), lds, st, a);
}

template <int DT, int MODE, bool MULTI, bool LEAN = false>
static hipError_t launch_d(const DecodeArgs& a, int grid, hipStream_t st) {
  const size_t lds = (size_t)(a.num_seqs + 1) * sizeof(int32_t);
  if (a.b8)
    launch_b<DT, MODE, MULTI, LEAN, true>(a, grid, lds, st);
  else
    launch_b<DT, MODE, MULTI, LEAN, false>(a, grid, lds, st);
  return hipGetLastError();
}

// MODE_EVEN with a.max_rows > 1 runs the multi-row (verify) columns, with a.lean the lean
// stream (when the chunk kernel runs beside it)
hipError_t launch_mfma_decode(int dt, int mode, const DecodeArgs& a, int grid, hipStream_t st) {
  const bool f16 = dt == DT_F16;
  if (dt == DT_FP8) {
    if (mode == MODE_PARTITION) return launch_d<DT_FP8, MODE_PARTITION, false>(a, grid, st);
    if (a.max_rows > 1 && a.lean) return launch_d<DT_FP8, MODE_EVEN, true, true>(a, grid, st);
    return a.max_rows > 1 ? launch_d<DT_FP8, MODE_EVEN, true>(a, grid, st)
                          : launch_d<DT_FP8, MODE_EVEN, false>(a, grid, st);
  }
  if (dt == DT_FP8B) {
    if (mode == MODE_PARTITION) return launch_d<DT_FP8B, MODE_PARTITION, false>(a, grid, st);
    if (a.max_rows > 1 && a.lean) return launch_d<DT_FP8B, MODE_EVEN, true, true>(a, grid, st);
    return a.max_rows > 1 ? launch_d<DT_FP8B, MODE_EVEN, true>(a, grid, st)
                          : launch_d<DT_FP8B, MODE_EVEN, false>(a, grid, st);
  }
  if (mode == MODE_EVEN) {
    if (a.max_rows > 1 && a.lean)
      return f16 ? launch_d<DT_F16, MODE_EVEN, true, true>(a, grid, st)
                 : launch_d<DT_BF16, MODE_EVEN, true, true>(a, grid, st);
    if (a.max_rows > 1)
      return f16 ? launch_d<DT_F16, MODE_EVEN, true>(a, grid, st)
                 : launch_d<DT_BF16, MODE_EVEN, true>(a, grid, st);
    return f16 ? launch_d<DT_F16, MODE_EVEN, false>(a, grid, st)
               : launch_d<DT_BF16, MODE_EVEN, false>(a, grid, st);
  }
  return f16 ? launch_d<DT_F16, MODE_PARTITION, false>(a, grid, st)
             : launch_d<DT_BF16, MODE_PARTITION, false>(a, grid, st);
}

template <int DT, int MODE>
static int occ(int head_dim, int lds) {
  int nb = 0;
  hipError_t e;
  if (head_dim == 64)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, mfma_decode_kernel<DT, 64, MODE, false, false, false>, kWG, lds);
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, mfma_decode_kernel<DT, 128, MODE, false, false, false>, kWG, lds);
  return e == hipSuccess && nb > 0 ? nb : 1;
}

int mfma_decode_max_blocks_per_cu(int dt, int head_dim, int mode, int lds_bytes) {
  if (dt == DT_FP8)
    return mode == MODE_EVEN ? occ<DT_FP8, MODE_EVEN>(head_dim, lds_bytes)
                             : occ<DT_FP8, MODE_PARTITION>(head_dim, lds_bytes);
  if (dt == DT_FP8B)
    return mode == MODE_EVEN ? occ<DT_FP8B, MODE_EVEN>(head_dim, lds_bytes)
                             : occ<DT_FP8B, MODE_PARTITION>(head_dim, lds_bytes);
  if (mode == MODE_EVEN)
    return dt == DT_F16 ? occ<DT_F16, MODE_EVEN>(head_dim, lds_bytes)
                        : occ<DT_BF16, MODE_EVEN>(head_dim, lds_bytes);
  return dt == DT_F16 ? occ<DT_F16, MODE_PARTITION>(head_dim, lds_bytes)
                      : occ<DT_BF16, MODE_PARTITION>(head_dim, lds_bytes);
}

}  // namespace pa
