// chunk.hip — multi-row (chunked-prefill) attention over the paged cache.
//
// "vLLM 架构源码解析 第1篇" §1.1 runs a long prompt as 512-token chunks in the same step as
// other requests' decode rows, and §3.3.2 marks each request's rows with query_start_loc.
// A sequence s with n > 1 rows has its context_lens entry counting those rows (they were
// written by reshape_and_cache first, §3.3.3); row j sits at position ctx - n + j and attends
// keys [0, ctx - n + j] (causal).  Sequences with few rows (a decode row, or on the
// matrix-core path up to 16 / G rows, as in a speculative verify step) are left to the decode
// kernels of pa_decode; pa_decode_partitioned sends every sequence of several rows here.
//
// Work item = (sequence, KV head g, block of 128 query columns[, key partition]), a column
// being one (row, head) pair: 128 / G consecutive rows x the G query heads of g.  The
// workgroup stages each 32-token K/V unit in LDS once and its four waves each run 32
// columns over it on the matrix cores (S^T = K . Q^T, then O^T += V^T . P^T, operand layouts
// as in pa_mfma.h), so one unit read from memory serves 128 columns.
//
// The softmax between the two products is streamed with a lazy reference: a column's
// weights are exp2(score - m) against a reference m that moves only when the column's
// running max exceeds it by more than kLazy (2^8 in weight), so the rescale of the outputs
// is rare after a column's first keys; weights then lie in [0, 2^8], well inside fp32 and
// the 16-bit operand types.  The weight sum l comes out of the matrix core as well (P
// multiplied by a block of ones), from the same 16-bit weights as the outputs, so every
// column's output is a weighted mean whose weights sum to one up to fp32 rounding.  Feeding
// P as one 16-bit operand rounds each weight by a relative d_t, |d_t| <= 2^-9 (bf16) or
// 2^-11 (fp16); the output then errs by sum_t d_t w_t (v_t - o), w_t the final softmax
// weights.  A single heavy key makes that error large (w = 0.35, |v - o| = 3: 2e-3 in
// bf16), so a unit whose largest weight in some column of the block exceeds kHeavy of that
// column's running sum including it feeds P as hi + lo 16-bit parts (two products, ~2^-17
// relative).  Every weight fed as one part is then at most kHeavy of its column's final sum:
// each key adds at most 2^-9 kHeavy |v_t - o| and the independent roundings add up to a
// standard deviation of at most 2^-9 / sqrt(3) * sqrt(kHeavy) * rms_w(v - o).  The hi + lo
// units are the first few of every column (while its sum is small) and units with a new
// dominant key.
//
// FP8 pools ("vLLM 深度拆解" §10.1) take the same path: each 8-byte half of an E4M3 chunk is
// widened to the query's 16-bit type (exact for every E4M3 value) on its way into LDS, where
// the unit then has the 16-bit layout; k_scale is in the score factor and v_scale multiplies
// the output.
#include <algorithm>

#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma.h"

namespace pa {

constexpr int kChunkBlocks = 2;                       // 16-column MFMA blocks per wave
constexpr int kWaveCols = 16 * kChunkBlocks;          // query columns per wave
constexpr int kItemCols = kWaveCols * kWavesPerWG;    // query columns per workgroup
constexpr float kLazy = 8.f;                          // reference slack, base-2 exponent
constexpr float kHeavy = 1.f / 64;                    // heavier weights: hi + lo parts

constexpr int kCuLdsBytes = 160 * 1024;               // LDS of one CU

typedef __attribute__((address_space(1))) void gbl_void_t;
typedef __attribute__((address_space(3))) void lds_void_t;

template <int D>
struct ChunkTile {
  static constexpr int TILE = 16 * D * 2;                  // one block of one KV head, bytes
  static constexpr int UNIT = 4 * TILE;                    // K and V of a 32-token unit
  static constexpr int LOADS = UNIT / (kWG * 16);          // 16-byte loads per thread per unit
  static constexpr int CPT = TILE / 16;                    // 16-byte chunks per tile
};

// The staged unit in LDS is the 16-token layout (K tiles [D/8][16][8], V tiles [D][16]) with
// its 16-byte pieces permuted inside each 256-byte row, so that the operand reads of a wave
// hit distinct LDS banks in every group of 8 and of 16 lanes: K token tok of staged tile kt
// sits at slot swz_k(kt, tok) of its chunk row (lanes n and n + 8 read tokens 16 apart,
// which would share banks), and V's two 16-byte halves of dimension d are swapped when
// swz_v(d) (lanes n and n + 4, n + 8 read rows 128 and 256 bytes apart).
__device__ __forceinline__ int swz_k(int kt, int tok) {
  return tok ^ ((((tok >> 3) ^ kt) & 1) << 2);
}
__device__ __forceinline__ int swz_v(int d) { return ((d >> 2) ^ (d >> 3)) & 1; }

struct ChunkPlanIn {
  const int32_t* qsl;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t rows_per_item;
  int32_t min_rows;   // sequences with fewer rows are the decode kernel's
  int32_t part_tokens;  // > 0: one item per key partition of this many tokens as well
};

// work items per sequence: ceil(n / rows_per_item) column blocks (times the key partitions
// of its context with part_tokens) for sequences of at least min_rows rows, else 0
__device__ inline void build_chunk_plan(int32_t* base, const ChunkPlanIn& p) {
  wave_plan(base, p.num_seqs, [&](int s) {
    const int32_t n = p.qsl[s + 1] - p.qsl[s];
    if (n < p.min_rows) return 0;
    const int32_t cbs = (n + p.rows_per_item - 1) / p.rows_per_item;
    if (p.part_tokens <= 0) return cbs;
    const int32_t ctx = p.context_lens[s];
    return cbs * ((ctx + p.part_tokens - 1) / p.part_tokens);
  });
}

// What a chunk-kernel launch computes.
enum ChunkMode : int {
  CM_ROWS = 0,    // pa_decode: every row of the multi-row sequences, causal, to `out`
  CM_PART = 1,    // pa_decode_partitioned: per key partition, partials
  CM_PREFIX = 2,  // shared prefixes: every row of a group over the group's shared keys,
                  // per key partition, partials
};

// Group i of a shared-prefix call: its sequences [gs, ge) (clamped to the batch), their rows
// [r0, r1), and `keys`: the keys of the group's claimed leading blocks (grp_blocks[i], at
// most max_prefix_blocks) in whole 32-token units, 0 when the group is empty or when its
// first sequence has a row that does not see all of them (then no table entry of the group
// is ever used).
struct PrefixGroup {
  int gs, ge, r0, r1, keys;
};

__device__ inline PrefixGroup prefix_group(const DecodeArgs& a, int i) {
  PrefixGroup p;
  p.gs = min(max(a.grp_start[i], 0), a.num_seqs);
  p.ge = min(max(a.grp_start[i + 1], p.gs), a.num_seqs);
  p.r0 = a.qsl ? a.qsl[p.gs] : p.gs;
  p.r1 = a.qsl ? a.qsl[p.ge] : p.ge;
  const int blocks = min(a.grp_blocks[i], a.max_prefix_blocks);
  const int64_t keys = blocks > 0 ? (int64_t)blocks * a.block_size / kMfmaUnit * kMfmaUnit : 0;
  p.keys = (int)min(keys, (int64_t)0x7fffffe0);
  if (p.ge > p.gs) {
    const int rows = (a.qsl ? a.qsl[p.gs + 1] : p.gs + 1) - p.r0;
    if (rows < 1 || p.keys > a.context_lens[p.gs] - rows) p.keys = 0;
  } else {
    p.keys = 0;
  }
  return p;
}

// skip_out[s] for every sequence s (prefix mode, waves w, w + W, ...): the keys of its
// group's shared prefix when s is a sequence the decode kernel takes (1 .. max_rows rows),
// each of its rows sees every key of the prefix and its table entries over the prefix are
// those of the group's first sequence; else 0 (the decode or chunk kernel attends all its
// keys).  With grp_start not non-decreasing, groups could overlap (a row with two prefixes):
// then every skip is 0.
__device__ inline void write_skips(const DecodeArgs& a, int64_t w, int64_t W) {
  const int lane = lane_id();
  if (w >= a.num_seqs) return;
  bool ordered = true;
  for (int i = lane; i < a.num_groups; i += kWave)
    ordered &= a.grp_start[i] <= a.grp_start[i + 1];
  ordered = __builtin_amdgcn_ballot_w64(!ordered) == 0;
  for (int64_t s = w; s < a.num_seqs; s += W) {
    int sk = 0;
    if (!ordered) {
      if (lane == 0) a.skip_out[s] = 0;
      continue;
    }
    // the group of s: the largest i with grp_start[i] <= s
    int lo = 0, hi = a.num_groups - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.grp_start[mid] <= s)
        lo = mid;
      else
        hi = mid - 1;
    }
    const PrefixGroup pg = prefix_group(a, lo);
    if (pg.keys > 0 && s >= pg.gs && s < pg.ge) {
      const int row = a.qsl ? a.qsl[s] : (int)s;
      const int rows = (a.qsl ? a.qsl[s + 1] : (int)s + 1) - row;
      if (rows >= 1 && rows <= a.max_rows && pg.keys <= a.context_lens[s] - rows) {
        const int nb = (pg.keys + a.block_size - 1) / a.block_size;
        const int32_t* mine = a.block_tables + s * a.max_blocks_per_seq;
        const int32_t* lead = a.block_tables + (int64_t)pg.gs * a.max_blocks_per_seq;
        bool differ = false;
        for (int j = lane; j < nb; j += kWave) differ |= mine[j] != lead[j];
        if (!__builtin_amdgcn_ballot_w64(differ)) sk = pg.keys;
      }
    }
    if (lane == 0) a.skip_out[s] = sk;
  }
}

// Per-lane state of one 16-column block: outputs O[column n][dims 16 j + 4 r ..], the
// weight sum (all four entries equal), the weights' reference and the true running max
// (both base 2, scaled scores).
template <int D>
struct ChunkCol {
  f32x4_t acc[D / 16];
  f32x4_t lsum;
  float m;
  float mx;
};

template <int DT>
struct ChunkP {
  op8_t<DT> hi, lo;
  bool split;  // uniform: the weights are fed as hi + lo
};

// Eight fp32 weights as one 16-bit MFMA operand, converted in pairs (round to nearest even).
template <int DT>
__device__ __forceinline__ op8_t<DT> pack8(const float (&p)[8]) {
  using E = typename std::conditional<bf16_core<DT>(), __bf16, _Float16>::type;
  typedef __attribute__((ext_vector_type(2))) E e2_t;
  op8_t<DT> o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const e2_t v = __builtin_convertvector((f32x2_t){p[2 * j], p[2 * j + 1]}, e2_t);
    o[2 * j] = v[0];
    o[2 * j + 1] = v[1];
  }
  return o;
}

// The lazy softmax update of one column block over a unit and the block's weights, from its
// raw scores q . k (s0, s1: the two S-blocks of the unit from the matrix core; lane (r, n)
// holds unit tokens 8 r .. 8 r + 7 of column n).  sl > 0 is the score factor in the base-2
// domain.  masked (uniform): unit token 8 r + k exists for this lane's column only if
// 8 r + k <= lim.  The low parts of the weights are formed when some column's largest
// weight is heavy (kHeavy).
template <int DT, int D>
__device__ __forceinline__ ChunkP<DT> chunk_softmax(ChunkCol<D>& st, const f32x4_t& s0,
                                                    const f32x4_t& s1, float sl, int lim,
                                                    bool masked) {
  using C = MfmaCfg<DT, D>;
  const int r = lane_id() >> 4;
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = s0[i];
    x[4 + i] = s1[i];
  }
  if (masked) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (8 * r + k > lim) x[k] = -INFINITY;
  }
  float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                   fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
  mx = cross_rows_max(mx);
  const float ms = mx * sl;  // -inf when the column sees no key of the unit
  st.mx = fmaxf(st.mx, ms);
  // move the reference only when the max outgrows it by more than kLazy (and on a
  // column's first visible keys, whose reference is -inf)
  if (__builtin_amdgcn_ballot_w64(ms > st.m + kLazy)) {
    const bool up = ms > st.m + kLazy;
    const float mnew = up ? ms : st.m;
    const float alpha = up ? __builtin_amdgcn_exp2f(st.m - mnew) : 1.f;
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) st.acc[j] *= alpha;
    st.lsum *= alpha;
    st.m = mnew;
  }
  // a column with no visible key so far keeps the reference -inf: its weights are 0
  const float mref = st.m == -INFINITY ? 0.f : st.m;
  // the column's largest weight of the unit, p, against its sum so far l: heavy when
  // p > kHeavy (l + p)
  const float pmax = __builtin_amdgcn_exp2f(fmaf(mx, sl, -mref));
  ChunkP<DT> out;
  out.split = __builtin_amdgcn_ballot_w64(pmax * (1.f / kHeavy - 1.f) > st.lsum[0]) != 0;
  float p[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) p[k] = __builtin_amdgcn_exp2f(fmaf(x[k], sl, -mref));
  out.hi = pack8<DT>(p);
  if (out.split) {
    const op8_t<DT> h = out.hi;
    float lo[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) lo[k] = p[k] - (float)h[k];
    out.lo = pack8<DT>(lo);
  }
  return out;
}

// O^T += V^T . P^T for one column block, and the weight sum from the same 16-bit weights.
template <int DT, int D>
__device__ __forceinline__ void chunk_pv(ChunkCol<D>& st, const op8_t<DT> (&vo)[D / 16],
                                         const ChunkP<DT>& p, const op8_t<DT>& ones) {
  using C = MfmaCfg<DT, D>;
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) st.acc[j] = mfma<DT>(vo[j], p.hi, st.acc[j]);
  st.lsum = mfma<DT>(ones, p.hi, st.lsum);
  if (p.split) {
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) st.acc[j] = mfma<DT>(vo[j], p.lo, st.acc[j]);
    st.lsum = mfma<DT>(ones, p.lo, st.lsum);
  }
}

// One work item: rows [j0, j0 + kItemCols / G) of multi-row sequence s for KV head g over the
// keys [kbeg, kend) (PART: one key partition; else every key the rows see).  The workgroup
// streams the keys in 32-token units: every unit (K and V of two blocks) is loaded once by
// the whole workgroup into LDS, and each wave then runs its 32 query columns (two 16-column
// MFMA blocks, per-column causal limits) over it.  16-bit pools of 16-token tiles go straight
// from memory into LDS, US units per barrier; FP8 pools (widened on the way) and 8-token
// blocks (two blocks per staged tile) go through registers, one unit per barrier.  DT is the
// 16-bit type of the queries and of the staged unit; F8: the pools hold E4M3 bytes.  PART:
// the item writes the partition's partials (normalised output, max, sum) instead of the
// output.
template <int DT, int D, bool F8, int CM, bool B8, int US>
__device__ void chunk_item(const DecodeArgs& a, int s, int g, int cb, int part,
                           char* lds_units) {
  constexpr bool DMA = !F8 && !B8;  // 16-bit pools of 16-token tiles: direct staging
  constexpr bool PART = CM != CM_ROWS;
  constexpr bool PRE = CM == CM_PREFIX;
  using C = MfmaCfg<DT, D>;
  using CT = ChunkTile<D>;
  using T = op8_t<DT>;
  using E = typename std::conditional<bf16_core<DT>(), __bf16, _Float16>::type;
  constexpr int NCB = kChunkBlocks;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int r = lane >> 4, n = lane & 15;
  const int G = a.num_q_heads / a.num_kv_heads;
  // the item's rows [q0, q0 + nrows), its keys [0, ctx) and the sequence whose table holds
  // them: a sequence, or (PRE) group s, whose rows all see every shared key
  int q0, nrows, ctx, bts;
  if constexpr (PRE) {
    const PrefixGroup pg = prefix_group(a, s);
    q0 = pg.r0;
    nrows = pg.r1 - pg.r0;
    ctx = pg.keys;
    bts = pg.gs;
  } else {
    q0 = a.qsl[s];
    nrows = a.qsl[s + 1] - q0;
    ctx = a.context_lens[s];
    bts = s;
  }
  q0 = __builtin_amdgcn_readfirstlane(q0);
  nrows = __builtin_amdgcn_readfirstlane(nrows);
  ctx = __builtin_amdgcn_readfirstlane(ctx);
  bts = __builtin_amdgcn_readfirstlane(bts);
  // the last key row j sees: causal (position ctx - nrows + j), or every key (PRE)
  auto vis = [&](int j) { return PRE ? ctx - 1 : ctx - nrows + j; };
  const int RW = kWaveCols / G;                    // rows per wave
  const int j0g = cb * (kItemCols / G);            // first row of the workgroup
  const int jendg = min(nrows, j0g + kItemCols / G);
  const int j0 = j0g + wave * RW;                  // first row of this wave
  const int jend = min(jendg, j0 + RW);
  // keys [kbeg, kend) any column of the item may see; this wave's columns see keys below
  // kend_w
  const int kbeg = PART ? part * a.part_tokens : 0;
  int kend = vis(jendg - 1) + 1;
  int kend_w = jend > j0 ? vis(jend - 1) + 1 : 0;
  if (PART) {
    kend = min(kend, kbeg + a.part_tokens);
    kend_w = min(kend_w, kbeg + a.part_tokens);
  }

  // Scores are formed with the factor sl > 0: a negative factor is folded into q (sign
  // flips are exact) and a zero factor makes every score 0 (q = 0, factor 1).
  float sl = a.scale_log2;
  const uint32_t qflip = sl < 0.f ? 0x80008000u : 0u;
  const bool qzero = sl == 0.f;
  sl = qzero ? 1.f : fabsf(sl);

  T qb[NCB][C::NKK];
  int pos[NCB];     // this lane's column's last visible key (-1: column past the rows)
  int first[NCB];   // smallest last-visible key over the block's columns (uniform)
  bool full[NCB];   // every column of the block is a real row (uniform)
  bool live[NCB];   // the block has a real row (uniform)
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    const int col = 16 * c + n;
    const int jc = j0 + col / G, hc = col % G;
    const bool ok = jc < jend;
    pos[c] = ok ? vis(jc) : -1;
    first[c] = vis(j0 + (16 * c) / G);
    full[c] = j0 + (16 * c + 15) / G < jend;
    live[c] = j0 + (16 * c) / G < jend;
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     ((int64_t)(q0 + jc) * a.num_q_heads + (int64_t)g * G + hc) * D * C::E;
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
      uint4 v = ok && !qzero ? ld16(qp + (4 * kk + r) * 16) : make_uint4(0, 0, 0, 0);
      v.x ^= qflip;
      v.y ^= qflip;
      v.z ^= qflip;
      v.w ^= qflip;
      qb[c][kk] = __builtin_bit_cast(T, v);
    }
  }
  ChunkCol<D> st[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    st[c].m = -INFINITY;
    st[c].mx = -INFINITY;
    st[c].lsum = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) st[c].acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  T ones;
#pragma unroll
  for (int k = 0; k < 8; ++k) ones[k] = (E)1.f;

  // a pool tile of one KV head: 16 tokens (8 with 8-token blocks), 16-bit or E4M3 elements
  constexpr int64_t PTILE = (F8 ? C::TILE / 2 : C::TILE) / (B8 ? 2 : 1);
  const int64_t blk_stride = (int64_t)a.num_kv_heads * PTILE;
  const char* kc = reinterpret_cast<const char*>(a.k_cache) + (int64_t)g * PTILE;
  const char* vc = reinterpret_cast<const char*>(a.v_cache) + (int64_t)g * PTILE;
  const int32_t* bt_row = a.block_tables + (int64_t)bts * a.max_blocks_per_seq;
  constexpr int TT = B8 ? 8 : kBlock;                    // tokens of one pool tile
  constexpr int PER_UNIT = kMfmaUnit / TT;               // pool tiles per unit
  const int nblk = (kend + TT - 1) / TT;
  const int ubeg = kbeg / kMfmaUnit;                     // partitions are whole units
  const int uend = (kend + kMfmaUnit - 1) / kMfmaUnit;

  // this lane's operand offsets in the staged unit (swizzled as staged; see swz_k, swz_v):
  // K of S-block b at lk[b] + 1 KiB per kk, V at lv + 512 bytes per j
  int lk[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int t = 8 * (n >> 2) + 4 * b + (n & 3);  // unit token of S-block row n
    lk[b] = (t >> 4) * CT::TILE + r * 256 + swz_k(t >> 4, t & 15) * 16;
  }
  const int lv = (2 + (r >> 1)) * CT::TILE + n * 32 + (((r & 1) ^ swz_v(n)) * 16);

  // (ub is restrict-qualified: LDS reads through it then carry alias information, which
  // keeps the compiler from waiting for the direct loads of the other buffer before them)
  auto compute = [&](int u, const char* __restrict__ ub) {
    const int t0 = u * kMfmaUnit;
    if (u < uend && t0 < kend_w) {  // uniform: this wave's columns see keys of this unit
      // scores of both column blocks from K (their MFMA chains interleaved), the softmax of
      // each, then P . V from V: K and V are never live together
      uint4 kb[2][C::NKK];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk)
          kb[b][kk] = *reinterpret_cast<const uint4*>(ub + lk[b] + 1024 * kk);
      f32x4_t s0[NCB], s1[NCB];
#pragma unroll
      for (int c = 0; c < NCB; ++c) s0[c] = s1[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // (a block with no real row has q = 0: its scores are computed and never used)
#pragma unroll
      for (int kk = 0; kk < C::NKK; ++kk)
#pragma unroll
        for (int c = 0; c < NCB; ++c) {
          s0[c] = mfma<DT>(__builtin_bit_cast(T, kb[0][kk]), qb[c][kk], s0[c]);
          s1[c] = mfma<DT>(__builtin_bit_cast(T, kb[1][kk]), qb[c][kk], s1[c]);
        }
      // The softmax (vector ALU, mostly exponentials) runs at raised wave priority and the
      // matrix products at the normal one: of the two waves on a SIMD, the one in its softmax
      // issues first while the other's queued products keep the matrix core busy (chunk rows
      // 438 -> 411 us; the placement of the switch back, before V's reads or before P . V,
      // made no difference).
      __builtin_amdgcn_s_setprio(1);
      ChunkP<DT> pp[NCB];
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        if (!live[c]) continue;
        const bool masked = !(t0 + kMfmaUnit - 1 <= first[c] && full[c]);
        pp[c] = chunk_softmax<DT, D>(st[c], s0[c], s1[c], sl, pos[c] - t0, masked);
      }
      T vo[C::NJ];
#pragma unroll
      for (int j = 0; j < C::NJ; ++j)
        vo[j] = __builtin_bit_cast(T, *reinterpret_cast<const uint4*>(ub + lv + 512 * j));
      if (t0 + kMfmaUnit > kend) {
        // zero the V elements of tokens past the item's keys (0 * NaN is NaN); their
        // weights are 0 in every column
        const int kv = min(8, max(0, kend - t0 - 8 * r));
        uint32_t mk[4];
#pragma unroll
        for (int w = 0; w < 4; ++w)
          mk[w] = (2 * w < kv ? 0xffffu : 0u) | (2 * w + 1 < kv ? 0xffff0000u : 0u);
#pragma unroll
        for (int j = 0; j < C::NJ; ++j) {
          uint4 w = __builtin_bit_cast(uint4, vo[j]);
          w.x &= mk[0];
          w.y &= mk[1];
          w.z &= mk[2];
          w.w &= mk[3];
          vo[j] = __builtin_bit_cast(T, w);
        }
      }
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int c = 0; c < NCB; ++c)
        if (live[c]) chunk_pv<DT, D>(st[c], vo, pp[c], ones);
    }
  };

  // block-table windows of 64 entries, [wbase, wbase + 128): pool tiles (16-token tiles of
  // the table, or 8-token blocks); entries past the item's last tile hold 0 (masked tokens)
  int win0 = 0, win1 = 0, wbase = -1;
  // the pool tiles of unit u (uniform); 16-token tiles: a second tile past the keys is
  // replaced by the first (its tokens are masked)
  auto unit_tiles = [&](int u, int64_t (&bt)[PER_UNIT]) {
    const int e = PER_UNIT * u;
    if (wbase < 0 || e >= wbase + 128) {  // uniform; happens every 128 / PER_UNIT units
      wbase = e;
      if constexpr (B8) {
        win0 = (e + lane < nblk) ? bt_row[e + lane] : 0;
        win1 = (e + 64 + lane < nblk) ? bt_row[e + 64 + lane] : 0;
      } else {
        win0 = (e + lane < nblk) ? tile_block(bt_row, e + lane, a.blk_shift) : 0;
        win1 = (e + 64 + lane < nblk) ? tile_block(bt_row, e + 64 + lane, a.blk_shift) : 0;
      }
    }
    const int ia = e - wbase;  // the unit's PER_UNIT entries share one register
#pragma unroll
    for (int i = 0; i < PER_UNIT; ++i)
      bt[i] = ia < 64 ? readlane(win0, ia + i) : readlane(win1, ia + i - 64);
    if (!B8 && e + 1 >= nblk) bt[PER_UNIT - 1] = bt[0];
  };
  if constexpr (DMA) {
    // Direct staging: wave w moves staged tile w of every unit [K tokens 0-15, K tokens
    // 16-31, V tokens 0-15, V tokens 16-31] from the pool into LDS with global_load_lds (one
    // KiB per instruction, lane i filling bytes 16 i .. 16 i + 15 of it), each lane reading
    // the 16 pool bytes that the swizzle places at its slot (swz_k and the V swap are
    // involutions): K slot (row, slot) holds token swz_k(kt, slot) of that row, V slot
    // (d, half) the half (half ^ swz_v(d)) of dimension d.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int soff = wave_u < 2
                         ? (lane >> 4) * 256 + swz_k(wave_u & 1, lane & 15) * 16
                         : (lane >> 1) * 32 + ((lane & 1) ^ swz_v(lane >> 1)) * 16;
    // Step pipeline, US units per step in one of two LDS buffers: the loads of step
    // k + 1 go out before step k is computed, each wave waits for its own loads at the end of
    // the step, and the barrier then publishes the next step and frees the buffer just read.
    auto issue = [&](int u0, char* buf) {
#pragma unroll
      for (int i = 0; i < US; ++i) {
        if (u0 + i >= uend) break;  // uniform
        int64_t bt[PER_UNIT];
        unit_tiles(u0 + i, bt);
        const char* src = (wave_u & 2 ? vc : kc) + (wave_u & 1 ? bt[1] : bt[0]) * blk_stride;
        char* dst = buf + i * CT::UNIT + wave_u * CT::TILE;
#pragma unroll
        for (int pt = 0; pt < CT::TILE / 1024; ++pt)
          __builtin_amdgcn_global_load_lds((gbl_void_t*)(src + soff + 1024 * pt),
                                           (lds_void_t*)(dst + 1024 * pt), 16, 0, 0);
      }
    };
    if (uend > ubeg) {  // uniform; PART: the item's rows may all lie before the partition
      const int steps = (uend - ubeg + US - 1) / US;
      issue(ubeg, lds_units);
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      for (int k = 0; k < steps; ++k) {
        const int u0 = ubeg + US * k;
        const char* cur = lds_units + (k & 1) * US * CT::UNIT;
        if (k + 1 < steps) issue(u0 + US, lds_units + ((k + 1) & 1) * US * CT::UNIT);
#pragma unroll
        for (int i = 0; i < US; ++i) compute(u0 + i, cur + i * CT::UNIT);
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      }
    }
  } else {
    // Register staging: this thread's share of a unit is chunk k * kWG + threadIdx.x of the
    // four tiles of the staged unit, read from pool tile ld_blk of the unit at byte src_off:
    //  - 16-token tiles: 16-bit chunk c of the tile; FP8: its 8 source bytes, half of E4M3 K
    //    chunk (c / 32) * 16 + c % 16, or bytes 8c.. of the V tile;
    //  - 8-token blocks: K chunk c = (8-element chunk c / 16, token c % 16) comes from block
    //    (c / 8) % 2 of the 16-token pair, V chunk c = (dimension c / 2, tokens 8 (c % 2) ..)
    //    from block c % 2, in the 8-token layouts K [D/X][8][X], V [D][8].
    int ld_tile[CT::LOADS], ld_off[CT::LOADS], src_off[CT::LOADS], ld_blk[CT::LOADS];
#pragma unroll
    for (int k = 0; k < CT::LOADS; ++k) {
      const int c = k * kWG + threadIdx.x;
      ld_tile[k] = c / CT::CPT;
      const int cc = c % CT::CPT;
      const bool vt = ld_tile[k] & 2;
      ld_off[k] = vt ? ((cc >> 1) * 2 + ((cc & 1) ^ swz_v(cc >> 1))) * 16
                     : ((cc >> 4) * 16 + swz_k(ld_tile[k] & 1, cc & 15)) * 16;
      if constexpr (B8) {
        const int half = vt ? cc & 1 : (cc >> 3) & 1;
        ld_blk[k] = 2 * (ld_tile[k] & 1) + half;
        const int ch = cc >> 4, tok = cc & 7;
        if constexpr (F8)
          src_off[k] = vt ? (cc >> 1) * 8 : (((ch >> 1) << 3) + tok) * 16 + 8 * (ch & 1);
        else
          src_off[k] = vt ? (cc >> 1) * 16 : ((ch << 3) + tok) * 16;
      } else {
        ld_blk[k] = ld_tile[k] & 1;
        if constexpr (F8)
          src_off[k] = vt ? cc * 8 : (((cc >> 5) << 4) + (cc & 15)) * 16 + 8 * ((cc >> 4) & 1);
        else
          src_off[k] = cc * 16;
      }
    }
    using Raw = typename std::conditional<F8, uint2, uint4>::type;
    constexpr int WDT = DT == DT_BF16 ? DT_FP8B : DT_FP8;  // widening of FP8 staged bytes
    auto load_unit = [&](Raw* regs, int u) {
      int64_t bt[PER_UNIT];
      unit_tiles(u, bt);
#pragma unroll
      for (int k = 0; k < CT::LOADS; ++k) {
        if constexpr (B8) {
          int64_t b = bt[0];
#pragma unroll
          for (int i = 1; i < PER_UNIT; ++i) b = ld_blk[k] == i ? bt[i] : b;
          const char* base = (ld_tile[k] & 2 ? vc : kc) + b * blk_stride;
          regs[k] = *reinterpret_cast<const Raw*>(base + src_off[k]);
        } else {
          // a whole wave loads from one tile (256 or 128 threads per tile): a scalar base
          const int t = __builtin_amdgcn_readfirstlane(ld_tile[k]);
          const char* base = (t & 2 ? vc : kc) + (t & 1 ? bt[1] : bt[0]) * blk_stride;
          regs[k] = *reinterpret_cast<const Raw*>(base + src_off[k]);
        }
      }
    };
    auto store_unit = [&](const Raw* regs, int buf) {
#pragma unroll
      for (int k = 0; k < CT::LOADS; ++k) {
        uint4 v;
        if constexpr (F8)
          v = __builtin_bit_cast(uint4, operand<WDT>(regs[k]));
        else
          v = regs[k];
        *reinterpret_cast<uint4*>(lds_units + buf * CT::UNIT + ld_tile[k] * CT::TILE + ld_off[k]) = v;
      }
    };
    // Unit pipeline: the loads of unit u + 2 go out at the start of step u, unit u is
    // computed from LDS buffer u % 2, and unit u + 1 (loaded since the start of step u - 1,
    // so two compute phases ago) is stored into the other buffer at the end of the step.  Even
    // steps stage in ra, odd ones in rb.  Loads and stores run on every step (past the last
    // unit they repeat it and the result is never read), and the barrier between steps does
    // not wait for outstanding loads, so the compiler's wait before each store covers only
    // that unit.
    auto barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
    const int ulast = uend - 1;
    if (uend > ubeg) {  // uniform; PART: the item's rows may all lie before the partition
      Raw ra[CT::LOADS], rb[CT::LOADS];
      load_unit(ra, ubeg);
      load_unit(rb, min(ubeg + 1, ulast));
      store_unit(ra, 0);
      barrier();
      for (int u = ubeg; u < uend; u += 2) {
        load_unit(ra, min(u + 2, ulast));
        compute(u, lds_units);
        store_unit(rb, 1);
        barrier();
        load_unit(rb, min(u + 3, ulast));
        compute(u + 1, lds_units + CT::UNIT);
        store_unit(ra, 0);
        barrier();
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the repeated loads past the last unit
    }
  }

  // emit: lane (r, n) holds dimensions 16 j + 4 r + i of column 16 c + n, which is
  // (row j0 + col / G, head col % G)
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    const float l = st[c].lsum[0];
    // FP8: a stored V value stands for its E4M3 value times v_scale
    const float inv = l > 0.f ? (F8 ? a.v_factor : 1.f) / l : 0.f;
    const int col = 16 * c + n;
    const int jr = j0 + col / G, hr = col % G;
    if (jr >= jend) continue;
    const int64_t rowh = (int64_t)(q0 + jr) * a.num_q_heads + (int64_t)g * G + hr;
    if constexpr (PART) {
      // partials of partition `part`: normalised output, max (natural log) and sum taken
      // against the true max; a column with no key in the partition: max -inf, sum 0,
      // output not written
      const int64_t e = rowh * a.max_partitions + part;
      if (l > 0.f) {
        float* po = a.part_o + e * D;
#pragma unroll
        for (int j = 0; j < C::NJ; ++j)
          *reinterpret_cast<f32x4_t*>(po + 16 * j + 4 * r) = st[c].acc[j] * inv;
      }
      if (r == 0) {
        a.part_m[e] = l > 0.f ? st[c].mx * 0.69314718055994531f : -INFINITY;
        a.part_l[e] = l > 0.f ? l * __builtin_amdgcn_exp2f(st[c].m - st[c].mx) : 0.f;
      }
    } else {
      const int64_t ob = rowh * D;
#pragma unroll
      for (int j = 0; j < C::NJ; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          store_out<DT>(a.out, ob + 16 * j + 4 * r + i, st[c].acc[j][i] * inv, a.out_f32);
    }
  }
}

// Most multi-row sequences whose items are ordered longest first (see chunk_kernel).
constexpr int kMaxOrdered = 256;

// LDS of the staged units: two buffers of US units (direct staging) or of one unit
template <int D, bool F8, bool B8, int US>
constexpr int chunk_stage_bytes() {
  return 2 * (!F8 && !B8 ? US : 1) * ChunkTile<D>::UNIT;
}

// Work items, one per workgroup.  Items differ in length by up to the longest context over
// the shortest, and workgroups start in index order as earlier ones finish, so the items are
// numbered longest first: multi-row sequences by decreasing number of prior keys, within a
// sequence column blocks last to first (the longest causal ranges first), and the KV heads
// of one (sequence, column block) consecutively.  With more than kMaxOrdered multi-row
// sequences the items keep the sequence order instead, KV head slowest, numbered XCD-locally
// so that each XCD works through mostly one KV head.  CM_PART: items are (sequence, column
// block, partition) of at most one partition each, in sequence order, KV head slowest;
// CM_PREFIX the same over the groups' shared keys, and then the skips of every sequence.
template <int DT, int D, bool F8, int CM, bool B8, int US>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(2))) void chunk_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) char lds_raw[];
  char* lds_units = lds_raw;  // the unit buffers
  int32_t* base = reinterpret_cast<int32_t*>(lds_raw + chunk_stage_bytes<D, F8, B8, US>());
  const int G = a.num_q_heads / a.num_kv_heads;
  const int S = a.num_seqs;
  const int Hkv = a.num_kv_heads;

  if constexpr (CM == CM_PREFIX) {
    // items per group: column blocks x key partitions of its shared keys
    const int NG = a.num_groups;
    const int rpi = kItemCols / G;
    wave_plan(base, NG, [&](int i) {
      const PrefixGroup pg = prefix_group(a, i);
      if (pg.keys <= 0 || pg.r1 <= pg.r0) return 0;
      return (pg.r1 - pg.r0 + rpi - 1) / rpi * ((pg.keys + a.part_tokens - 1) / a.part_tokens);
    });
    const int64_t per_head = base[NG];
    const int64_t total = per_head * Hkv;
    for (int64_t i = xcd_local_block(blockIdx.x, gridDim.x); i < total; i += gridDim.x) {
      const int gh = (int)(i / per_head);
      const int64_t k = i - (int64_t)gh * per_head;
      const int grp = find_seq(base, NG, k, 1);
      const int np = (prefix_group(a, grp).keys + a.part_tokens - 1) / a.part_tokens;
      const int idx = (int)(k - base[grp]);
      chunk_item<DT, D, F8, CM_PREFIX, B8, US>(a, grp, gh, idx / np, idx % np, lds_units);
      __syncthreads();  // the unit buffers are reused by the next item
    }
    // the skips last, off the items' path (the decode kernel that reads them runs after this
    // kernel); the workgroups without items take them first
    const int64_t items_wg = min(total, (int64_t)gridDim.x);
    const int64_t rank = (xcd_local_block(blockIdx.x, gridDim.x) - items_wg + gridDim.x) %
                         gridDim.x;
    write_skips(a, rank * kWavesPerWG + threadIdx.x / kWave, (int64_t)gridDim.x * kWavesPerWG);
    return;
  }

  int32_t* order = base + a.num_seqs + 1;  // [kMaxOrdered] multi-row sequences, longest first
  int32_t* rbase = order + kMaxOrdered;    // [kMaxOrdered + 1] item prefix in that order
  int32_t* pkeys = rbase + kMaxOrdered + 1;  // [kMaxOrdered] prior keys of order[] entries
  int32_t* count = pkeys + kMaxOrdered;
  constexpr bool PART = CM == CM_PART;
  ChunkPlanIn pin{a.qsl, a.context_lens, S, kItemCols / G, a.max_rows + 1,
                  PART ? a.part_tokens : 0};
  build_chunk_plan(base, pin);
  const int64_t per_head = base[S];
  const int64_t total = per_head * Hkv;

  if constexpr (PART) {
    for (int64_t i = xcd_local_block(blockIdx.x, gridDim.x); i < total; i += gridDim.x) {
      const int gh = (int)(i / per_head);
      const int64_t k = i - (int64_t)gh * per_head;
      const int s = find_seq(base, S, k, 1);
      const int np = (a.context_lens[s] + a.part_tokens - 1) / a.part_tokens;
      const int idx = (int)(k - base[s]);
      chunk_item<DT, D, F8, CM_PART, B8, US>(a, s, gh, idx / np, idx % np, lds_units);
      __syncthreads();  // the unit buffers are reused by the next item
    }
    return;
  }

  // collect the multi-row sequences (any order), then rank them by prior keys (ties: index)
  if (threadIdx.x == 0) *count = 0;
  __syncthreads();
  for (int t = threadIdx.x; t < S; t += kWG) {
    if (base[t + 1] > base[t]) {
      const int slot = atomicAdd(count, 1);
      if (slot < kMaxOrdered) {
        order[slot] = t;
        pkeys[slot] = a.context_lens[t] - (a.qsl[t + 1] - a.qsl[t]);
      }
    }
  }
  __syncthreads();
  const int M = *count;
  const bool ordered = M <= kMaxOrdered;
  if (ordered) {
    int mine = -1, rank = 0;
    if (threadIdx.x < M) {
      mine = order[threadIdx.x];
      const int pm = pkeys[threadIdx.x];
      for (int k = 0; k < M; ++k) {
        const int o = order[k], po = pkeys[k];
        rank += (po > pm || (po == pm && o < mine)) ? 1 : 0;
      }
    }
    __syncthreads();
    if (mine >= 0) order[rank] = mine;
    __syncthreads();
    wave_plan(rbase, M, [&](int r) { return (base[order[r] + 1] - base[order[r]]) * Hkv; });
  }

  for (int64_t i = ordered ? (int64_t)blockIdx.x : xcd_local_block(blockIdx.x, gridDim.x);
       i < total; i += gridDim.x) {
    int s, g, cb;
    if (ordered) {
      const int rk = find_seq(rbase, M, i, 1);
      s = order[rk];
      const int k = (int)(i - rbase[rk]);
      const int nb = base[s + 1] - base[s];
      cb = nb - 1 - k / Hkv;
      g = k % Hkv;
    } else {
      g = (int)(i / per_head);
      const int64_t k = i - (int64_t)g * per_head;
      s = find_seq(base, S, k, 1);
      const int nb = base[s + 1] - base[s];
      cb = nb - 1 - (int)(k - base[s]);
    }
    chunk_item<DT, D, F8, CM_ROWS, B8, US>(a, s, g, cb, 0, lds_units);
    __syncthreads();  // the unit buffers are reused by the next item
  }
}

int max_lds_per_block() {
  static int v = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
      n = 65536;
    return n;
  }();
  return v;
}

// plan_lds: the plan arrays behind the unit buffers.  Direct staging takes two units per
// barrier where two workgroups of that size still fit a CU's LDS (the chunk kernel runs two
// per CU), else one.
template <int DT, int D, bool F8, int CM, bool B8>
static hipError_t launch_us(const DecodeArgs& a, int grid, size_t plan_lds, hipStream_t st) {
  constexpr int one = chunk_stage_bytes<D, F8, B8, 1>();
  if constexpr (!F8 && !B8) {
    constexpr int two = chunk_stage_bytes<D, F8, B8, 2>();
    if (2 * (two + plan_lds) <= (size_t)kCuLdsBytes && two + plan_lds <= (size_t)max_lds_per_block()) {
      hipLaunchKernelGGL((chunk_kernel<DT, D, F8, CM, B8, 2>), dim3(grid), dim3(kWG),
                         two + plan_lds, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((chunk_kernel<DT, D, F8, CM, B8, 1>), dim3(grid), dim3(kWG), one + plan_lds,
                     st, a);
  return hipGetLastError();
}

template <int DT, bool F8, int CM, bool B8>
static hipError_t launch_cb(const DecodeArgs& a, int grid, size_t plan_lds, hipStream_t st) {
  if (a.head_dim == 64) return launch_us<DT, 64, F8, CM, B8>(a, grid, plan_lds, st);
  return launch_us<DT, 128, F8, CM, B8>(a, grid, plan_lds, st);
}

template <int DT, bool F8, int CM>
static hipError_t launch_c(const DecodeArgs& a, int grid, size_t plan_lds, hipStream_t st) {
  if (a.b8) return launch_cb<DT, F8, CM, true>(a, grid, plan_lds, st);
  return launch_cb<DT, F8, CM, false>(a, grid, plan_lds, st);
}

template <int CM>
static hipError_t launch_dt(int dt, const DecodeArgs& a, int grid, size_t plan_lds,
                            hipStream_t st) {
  if (dt == DT_F16) return launch_c<DT_F16, false, CM>(a, grid, plan_lds, st);
  if (dt == DT_BF16) return launch_c<DT_BF16, false, CM>(a, grid, plan_lds, st);
  if (dt == DT_FP8) return launch_c<DT_F16, true, CM>(a, grid, plan_lds, st);
  return launch_c<DT_BF16, true, CM>(a, grid, plan_lds, st);
}

static size_t plan_bytes(int entries) {
  return (size_t)(entries + 1 + 3 * kMaxOrdered + 2) * sizeof(int32_t);
}

// dt: DT_F16 / DT_BF16 pools, or DT_FP8 / DT_FP8B (FP8 pools behind fp16 / bf16 queries).
// a.part_tokens > 0: the partition mode of pa_decode_partitioned (every sequence with more
// than a.max_rows rows, one item per key partition).
hipError_t launch_chunk(int dt, const DecodeArgs& a, int num_q_rows, hipStream_t st) {
  const int rpi = kItemCols / (a.num_q_heads / a.num_kv_heads);
  const size_t plan_lds = plan_bytes(a.num_seqs);
  if (a.part_tokens > 0) {
    // at most (ceil(rows / rows_per_item) + num_seqs) column blocks x max_partitions items per
    // KV head, walked with a grid stride by a grid of up to 4096 workgroups
    const int64_t items = ((int64_t)(num_q_rows + rpi - 1) / rpi + a.num_seqs) *
                          a.max_partitions * a.num_kv_heads;
    const int64_t wgs = (std::min<int64_t>(items, 4096) + kXcds - 1) / kXcds * kXcds;
    return launch_dt<CM_PART>(dt, a, (int)wgs, plan_lds, st);
  }
  // one workgroup per work item: at most ceil(rows / rows_per_item) + num_seqs items per KV
  // head; a multiple of the XCD count keeps the XCD-local numbering on
  const int64_t items = ((int64_t)(num_q_rows + rpi - 1) / rpi + a.num_seqs) * a.num_kv_heads;
  const int64_t wgs = (items + kXcds - 1) / kXcds * kXcds;
  const int grid = (int)(wgs < (1 << 20) ? wgs : (1 << 20) / kXcds * kXcds);
  if (grid <= 0) return hipSuccess;
  return launch_dt<CM_ROWS>(dt, a, grid, plan_lds, st);
}

// The shared-prefix kernel: every group's rows over its shared keys, a.part_tokens keys per
// partial (a.part_o / part_m / part_l with a.max_partitions slots per row and head), and
// a.skip_out for every sequence.  At most (ceil(rows / rows_per_item) + num_groups) column
// blocks x max_partitions items per KV head, walked with a grid stride by up to 4096
// workgroups (at least one per XCD, which also write the skips).
hipError_t launch_prefix(int dt, const DecodeArgs& a, int num_q_rows, hipStream_t st) {
  const int rpi = kItemCols / (a.num_q_heads / a.num_kv_heads);
  const int64_t items = ((int64_t)(num_q_rows + rpi - 1) / rpi + a.num_groups) *
                        a.max_partitions * a.num_kv_heads;
  const int64_t wgs = (std::max<int64_t>(std::min<int64_t>(items, 4096), 1) + kXcds - 1) /
                      kXcds * kXcds;
  return launch_dt<CM_PREFIX>(dt, a, (int)wgs, plan_bytes(std::max(a.num_seqs, a.num_groups)),
                              st);
}

}  // namespace pa
