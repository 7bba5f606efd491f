// pa_mfma.h — matrix-core building blocks of the decode and chunk kernels (gfx950).
//
// One 32-token unit (two 16-token blocks of one KV head) against 16 query columns:
//   S^T = K . Q^T    as 2 x (D/32) MFMA 16x16x32  (M = 16 tokens, N = 16 query columns)
//   O^T += V^T . P^T as (D/16) MFMA 16x16x32     (M = 16 dims, N = 16 query columns, K = 32 tokens)
// with a streamed (online) softmax per query column in between.  Both products keep the
// query column in N, so every lane's scores, running max / sum and output accumulators
// belong to its own column l%16: the softmax rescale needs no cross-lane traffic.
//
// Operand layouts (gfx950 v_mfma_f32_16x16x32_{bf16,f16}): lane l supplies A[l%16][8(l/16)..+8]
// and B[8(l/16)..+8][l%16] and receives D[4(l/16)+i][l%16], i < 4.
//   * The M row m of S-block b is unit token 8(m/4) + 4b + m%4, so lane l (r = l/16) ends up
//     with the scores of tokens 8r..8r+7 for column l%16 — exactly the P^T operand slots it
//     supplies to the V^T.P^T product (B[8r..8r+7][column]).  No score moves between lanes.
//   * V tiles are [D][16 tokens] in the pool, so the A operand of the V^T.P^T product
//     (tokens 8r..8r+7 of one dimension) is one 16-byte load.  The lane receives dimensions
//     16j + 4r + i (i < 4) of its column.
//   * K tiles are [D/8][16][8]: a token's 8-element chunk, the A operand of S^T, is one
//     16-byte load.
//   * FP8 pools (tiles of bytes, K [D/16][16][16]): the same operands are 8-byte loads (half a
//     K chunk; 8 tokens of a V row), widened to f16 in registers, which holds every E4M3
//     value exactly; the matrix cores then run in f16 with fp16 queries.
// P is fed to the matrix core as hi + lo 16-bit parts (two products), which keeps the
// rounding of the weights near 2^-16 relative instead of 2^-8 (bf16) or 2^-11 (fp16).
#pragma once

#include <math.h>

#include <type_traits>

#include "pa_device.h"

namespace pa {

template <int DT, int D>
struct MfmaCfg {
  static constexpr int E = is_fp8(DT) ? 1 : 2;  // pool element bytes (queries: 2)
  static constexpr int NKK = D / 32;  // MFMAs over the head dimension per S-block
  static constexpr int NJ = D / 16;   // MFMAs over output dims per unit
  static constexpr int64_t TILE = 16LL * D * E;
  static constexpr int DEPTH = 2;
};

// matrix-core operand type: bf16 or f16 (FP8 pools are widened to the query type, f16 or bf16,
// either of which holds every E4M3 value exactly)
template <int DT>
constexpr bool bf16_core() {
  return DT == DT_BF16 || DT == DT_FP8B;
}
template <int DT>
using op8_t = typename std::conditional<bf16_core<DT>(), bf16x8_t, f16x8_t>::type;

// What an operand load brings in: the 8-element operand itself (16-bit pools), or 8 E4M3
// bytes (FP8 pools), widened when the operand is used.
template <int DT>
struct MfmaRaw {
  using type = uint4;
};
template <>
struct MfmaRaw<DT_FP8> {
  using type = uint2;
};
template <>
struct MfmaRaw<DT_FP8B> {
  using type = uint2;
};

// an operand's raw bytes, loaded with the streaming (non-temporal) policy: the decode reads
// every K and V tile once per call
template <int DT>
__device__ __forceinline__ typename MfmaRaw<DT>::type ld_raw(const char* p) {
  using R = typename MfmaRaw<DT>::type;
  if constexpr (sizeof(R) == 16) {
    return ld16_nt(p);
  } else {
    typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_nt;
    const u32x2_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_nt*>(p));
    return R{v[0], v[1]};
  }
}

template <int DT>
__device__ __forceinline__ op8_t<DT> operand(const typename MfmaRaw<DT>::type& r) {
  if constexpr (is_fp8(DT)) {
    constexpr bool BF = bf16_core<DT>();
    const uint4 o = {fp8x2_to_16<BF, false>(r.x), fp8x2_to_16<BF, true>(r.x),
                     fp8x2_to_16<BF, false>(r.y), fp8x2_to_16<BF, true>(r.y)};
    return __builtin_bit_cast(op8_t<DT>, o);
  } else {
    return __builtin_bit_cast(op8_t<DT>, r);
  }
}

template <int DT>
__device__ __forceinline__ f32x4_t mfma(const op8_t<DT>& a, const op8_t<DT>& b, f32x4_t c) {
  if constexpr (bf16_core<DT>())
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int DT, int D>
struct MfmaState {
  float m;  // running max of head lane%16 (base-2 domain)
  float l;  // this lane's share of the running sum of head lane%16
  f32x4_t acc[MfmaCfg<DT, D>::NJ];  // O[column l%16][dim 16 j + 4(l/16) + i]
};

template <int DT, int D>
using MfmaK = typename MfmaRaw<DT>::type[2][MfmaCfg<DT, D>::NKK];
template <int DT, int D>
using MfmaV = typename MfmaRaw<DT>::type[MfmaCfg<DT, D>::NJ];
template <int DT, int D>
using MfmaQ = op8_t<DT>[MfmaCfg<DT, D>::NKK];

// Per-lane byte offsets of the unit operands.  Inside a tile the offsets of the other
// 16-byte pieces differ from these by compile-time steps (kk: 1 KiB, j: 256 elements), so
// they become immediate offsets of the loads instead of registers.
template <int DT, int D>
struct MfmaLaneOffsets {
  int k[2];   // offset inside the K tile of S-block b's piece kk = 0
  int kt[2];  // which tile of the unit (0 / 1) S-block b's token is in
  int v;      // offset inside the V tile of piece j = 0
  int vt;     // which tile of the unit this lane's V tokens are in
  __device__ __forceinline__ int koff(int b, int kk) const {
    return k[b] + 512 * MfmaCfg<DT, D>::E * kk;
  }
  __device__ __forceinline__ int voff(int j) const { return v + 256 * MfmaCfg<DT, D>::E * j; }
};

// The two halves of one unit for one 16-column block.  mfma_scores computes S^T = K . Q^T,
// masks tokens 8r + k > lim (MASK; lim: last visible unit token of this lane's query column,
// may differ per column), updates the running max and sum and returns the block's weights P
// (as hi + lo 16-bit parts) and the rescale factor of its outputs.  mfma_pv zeroes the V
// elements of tokens >= vvalid (MASK; uniform: tokens of the unit that hold written data, so
// poison never reaches the sums) and adds V^T . P^T to the rescaled outputs.  SAFE: a column
// may have seen no key yet (its running max is still -inf).
template <int DT>
struct MfmaP {
  op8_t<DT> hi, lo;
  float alpha;
};

template <int DT, int D, bool MASK, bool SAFE>
__device__ __forceinline__ MfmaP<DT> mfma_scores(MfmaState<DT, D>& st, const MfmaK<DT, D>& kb,
                                                 const MfmaQ<DT, D>& qb, float scale_log2,
                                                 int lim) {
  using C = MfmaCfg<DT, D>;
  using T = op8_t<DT>;
  const int lane = lane_id();
  const int r = lane >> 4;
  f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < C::NKK; ++kk) {
    s0 = mfma<DT>(operand<DT>(kb[0][kk]), qb[kk], s0);
    s1 = mfma<DT>(operand<DT>(kb[1][kk]), qb[kk], s1);
  }
  // raw scores q . k; the scale (> 0: a negative or zero one is folded into q by the caller)
  // enters through the exponent's fma, and the largest scaled score is the scale times the
  // largest raw score
  float s[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s[i] = s0[i];
    s[4 + i] = s1[i];
  }
  if (MASK) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (8 * r + k > lim) s[k] = -INFINITY;  // weight 0
  }
  float ext = s[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) ext = fmaxf(ext, s[k]);
  const float mx = cross_rows_max(ext) * scale_log2;
  const float mnew = fmaxf(st.m, mx);
  // SAFE: a column with no visible key so far keeps m = -inf, weight 0, and alpha 1
  const float mref = (SAFE && mnew == -INFINITY) ? 0.f : mnew;
  MfmaP<DT> p;
  p.alpha = __builtin_amdgcn_exp2f(st.m - mref);
  float psum = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float w = __builtin_amdgcn_exp2f(fmaf(s[k], scale_log2, -mref));
    psum += w;
    if constexpr (bf16_core<DT>()) {
      const __bf16 h = (__bf16)w;
      p.hi[k] = h;
      p.lo[k] = (__bf16)(w - (float)h);
    } else {
      const _Float16 h = (_Float16)w;
      p.hi[k] = h;
      p.lo[k] = (_Float16)(w - (float)h);
    }
  }
  st.l = st.l * p.alpha + psum;
  st.m = mnew;
  return p;
}

template <int DT, int D, bool MASK>
__device__ __forceinline__ void mfma_pv(MfmaState<DT, D>& st, MfmaV<DT, D>& vb,
                                        const MfmaP<DT>& p, int vvalid) {
  using C = MfmaCfg<DT, D>;
  using T = op8_t<DT>;
  T vo[C::NJ];
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) vo[j] = operand<DT>(vb[j]);
  if (MASK) {
    // zero the V elements of tokens past the written context (0 * NaN is NaN)
    const int r = lane_id() >> 4;
    const int kv = min(8, max(0, vvalid - 8 * r));
    const uint32_t m0 = (0 < kv ? 0xffffu : 0u) | (1 < kv ? 0xffff0000u : 0u);
    const uint32_t m1 = (2 < kv ? 0xffffu : 0u) | (3 < kv ? 0xffff0000u : 0u);
    const uint32_t m2 = (4 < kv ? 0xffffu : 0u) | (5 < kv ? 0xffff0000u : 0u);
    const uint32_t m3 = (6 < kv ? 0xffffu : 0u) | (7 < kv ? 0xffff0000u : 0u);
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
      uint4 w = __builtin_bit_cast(uint4, vo[j]);
      w.x &= m0;
      w.y &= m1;
      w.z &= m2;
      w.w &= m3;
      vo[j] = __builtin_bit_cast(T, w);
    }
  }
  // rescale this column's outputs by its own alpha (skipped when no column's max moved, as
  // is usual once a column has seen a few hundred keys: multiplying by 1 changes nothing),
  // then add V^T . P^T
  if (__builtin_amdgcn_ballot_w64(p.alpha != 1.f)) {
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.acc[j][i] *= p.alpha;
  }
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) {
    st.acc[j] = mfma<DT>(vo[j], p.hi, st.acc[j]);
    st.acc[j] = mfma<DT>(vo[j], p.lo, st.acc[j]);
  }
}
// One unit: scores, softmax update and P . V for one 16-column block.
template <int DT, int D, bool MASK, bool SAFE>
__device__ __forceinline__ void mfma_unit(MfmaState<DT, D>& st, const MfmaK<DT, D>& kb,
                                          MfmaV<DT, D>& vb, const MfmaQ<DT, D>& qb,
                                          float scale_log2, int lim, int vvalid) {
  const MfmaP<DT> p = mfma_scores<DT, D, MASK, SAFE>(st, kb, qb, scale_log2, lim);
  mfma_pv<DT, D, MASK>(st, vb, p, vvalid);
}

// Lane offsets of the unit operands (see the layout notes at the top of this file).
template <int DT, int D>
__device__ __forceinline__ MfmaLaneOffsets<DT, D> mfma_offsets() {
  using C = MfmaCfg<DT, D>;
  const int lane = lane_id();
  const int r = lane >> 4, n = lane & 15;
  MfmaLaneOffsets<DT, D> o;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int t = 8 * (n >> 2) + 4 * b + (n & 3);  // unit token of S-block row n
    o.kt[b] = t >> 4;
    if constexpr (C::E == 2)
      o.k[b] = (r * 16 + (t & 15)) * 16;  // chunk 4 kk + r of token t: + 1 KiB per kk
    else  // 16-element chunks: dims 8 r .. of block kk are half r & 1 of chunk 2 kk + r / 2
      o.k[b] = ((r >> 1) * 16 + (t & 15)) * 16 + 8 * (r & 1);
  }
  o.vt = r >> 1;
  o.v = (n * 16 + 8 * (r & 1)) * C::E;  // dimension 16 j + n: + 256 elements per j
  return o;
}

// Addressing of the 32-token units of KV head g of sequence s (context ctx): the block-table
// window of a chunk of units and the operand loads of one unit (see the layout notes at the
// top of this file).
//  - 16-token tiles: a unit is tiles 2 u and 2 u + 1; the window holds one tile per lane
//    (chunks of 64 units) and every lane reads its operands from one of the two tiles, whose
//    ids reach the scalar unit by readlane.  A unit whose second tile lies past the context
//    reads its first tile again (all of its tokens are masked).
//  - 8-token blocks (B8): a unit is blocks 4 u .. 4 u + 3; the window holds one block per
//    lane (chunks of 32 units).  Lane (r, n) reads its K operand (unit token
//    8 (n / 4) + 4 b + n % 4) from block n / 4 and its V operand (tokens 8 r .. 8 r + 7) from
//    block r, each lane fetching its block id from the window with a lane shuffle.  Entries
//    past the context's last block hold block 0 (masked).
template <int DT, int D, bool B8>
struct MfmaUnits {
  using C = MfmaCfg<DT, D>;
  static constexpr int CHUNK = B8 ? 32 : 64;              // units per window
  static constexpr int64_t PTILE = B8 ? C::TILE / 2 : C::TILE;  // one pool tile of a KV head
  const char* kc;
  const char* vc;
  const int32_t* bt_row;
  int64_t blk_stride;
  int ctx, nblk, shift;
  MfmaLaneOffsets<DT, D> o;
  int k8[2], v8;  // B8: this lane's offsets inside an 8-token tile (piece kk = 0, j = 0)
  int c0 = 0;
  int win0 = 0, win1 = 0;

  __device__ __forceinline__ MfmaUnits(const DecodeArgs& a, int s, int g, int ctx_) {
    kc = reinterpret_cast<const char*>(a.k_cache) + (int64_t)g * PTILE;
    vc = reinterpret_cast<const char*>(a.v_cache) + (int64_t)g * PTILE;
    bt_row = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    blk_stride = (int64_t)a.num_kv_heads * PTILE;
    ctx = ctx_;
    shift = a.blk_shift;
    nblk = B8 ? (ctx + 7) >> 3 : (ctx + kBlock - 1) / kBlock;
    o = mfma_offsets<DT, D>();
    const int lane = lane_id();
    const int r = lane >> 4, n = lane & 15;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int t8 = 4 * b + (n & 3);  // token inside block n / 4
      k8[b] = C::E == 2 ? 128 * r + 16 * t8 : 128 * (r >> 1) + 16 * t8 + 8 * (r & 1);
    }
    v8 = C::E == 2 ? 16 * n : 8 * n;
  }
  // the window of units [c0_, c1)
  __device__ __forceinline__ void window(int c0_, int c1) {
    c0 = c0_;
    const int lane = lane_id();
    if constexpr (B8) {
      const int e0 = 4 * c0, eend = min(nblk, 4 * c1);
      win0 = e0 + lane < eend ? bt_row[e0 + lane] : 0;
      win1 = e0 + 64 + lane < eend ? bt_row[e0 + 64 + lane] : 0;
    } else {
      const int b0 = 2 * c0, bend = min(nblk, 2 * c1);
      win0 = (b0 + lane < bend) ? tile_block(bt_row, b0 + lane, shift) : 0;
      win1 = (b0 + 64 + lane < bend) ? tile_block(bt_row, b0 + 64 + lane, shift) : 0;
    }
  }
  // B8: window entry e (per lane, e < 128)
  __device__ __forceinline__ int64_t entry(int e) const {
    const int x = __shfl(win0, e & 63, kWave), y = __shfl(win1, e & 63, kWave);
    return e < 64 ? x : y;
  }
  // 16-token tiles: the tile ids of unit u (uniform)
  __device__ __forceinline__ void tiles(int u, int64_t& ba, int64_t& bb) const {
    const int e = 2 * (u - c0);
    ba = e < 64 ? readlane(win0, e) : readlane(win1, e - 64);
    bb = (2 * u + 1 < nblk) ? (e + 1 < 64 ? readlane(win0, e + 1) : readlane(win1, e + 1 - 64)) : ba;
  }
  __device__ __forceinline__ void issue_k(MfmaK<DT, D>& kb, int u) const {
    if constexpr (B8) {
      const int n = lane_id() & 15;
      const char* kt = kc + entry(4 * (u - c0) + (n >> 2)) * blk_stride;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk) kb[b][kk] = ld_raw<DT>(kt + k8[b] + 256 * C::E * kk);
    } else {
      int64_t ba, bb;
      tiles(u, ba, bb);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const char* kt = kc + (o.kt[b] ? bb : ba) * blk_stride;
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk) kb[b][kk] = ld_raw<DT>(kt + o.koff(b, kk));
      }
    }
  }
  __device__ __forceinline__ void issue_v(MfmaV<DT, D>& vb, int u) const {
    if constexpr (B8) {
      const int r = lane_id() >> 4;
      const char* vt = vc + entry(4 * (u - c0) + r) * blk_stride;
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) vb[j] = ld_raw<DT>(vt + v8 + 128 * C::E * j);
    } else {
      int64_t ba, bb;
      tiles(u, ba, bb);
      const char* vt = vc + (o.vt ? bb : ba) * blk_stride;
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) vb[j] = ld_raw<DT>(vt + o.voff(j));
    }
  }
};

// Stream the 32-token units [u0, u1) of KV head g of sequence s (context ctx) through
// unit(kb, vb, u).  Units are walked in chunks (one block-table window each, loaded before
// the chunk's loop), and the loop is a two-stage software pipeline (the loads of unit u + 1
// are in flight while unit u is computed) in which every path into a unit has the same loads
// outstanding, so its wait covers only that unit.  All arguments must be wave-uniform.
template <int DT, int D, bool B8, class F>
__device__ __forceinline__ void mfma_stream(const DecodeArgs& a, int s, int g, int u0, int u1,
                                            int ctx, F&& unit) {
  MfmaUnits<DT, D, B8> U(a, s, g, ctx);
  for (int c0 = u0; c0 < u1; c0 += U.CHUNK) {
    const int c1 = min(u1, c0 + U.CHUNK);
    U.window(c0, c1);
    auto issue = [&](MfmaK<DT, D>& kb, MfmaV<DT, D>& vb, int u) {
      U.issue_k(kb, u);
      U.issue_v(vb, u);
    };
    MfmaK<DT, D> ka, kb;
    MfmaV<DT, D> va, vb;
    issue(ka, va, c0);
    int u = c0;
    for (; u + 2 < c1; u += 2) {
      issue(kb, vb, u + 1);
      unit(ka, va, u);
      issue(ka, va, u + 2);
      unit(kb, vb, u + 1);
    }
    if (u + 1 < c1) {
      issue(kb, vb, u + 1);
      unit(ka, va, u);
      unit(kb, vb, u + 1);
    } else {
      unit(ka, va, u);
    }
  }
}

// The lean form of mfma_stream: one K and one V operand buffer instead of two of each, so a
// wave needs about half the operand registers and two waves fit on a SIMD.  Unit u + 1's K
// loads go out as soon as unit u's scores have read K, its V loads as soon as unit u's P . V
// has read V; the in-order load counter then lets each wait cover only the operand it needs.
// scores(kb, u) returns the unit's weights, pv(vb, p, u) adds P . V.  All arguments must be
// wave-uniform.
template <int DT, int D, bool B8, class S, class PV>
__device__ __forceinline__ void mfma_stream_lean(const DecodeArgs& a, int s, int g, int u0,
                                                 int u1, int ctx, S&& scores, PV&& pv) {
  MfmaUnits<DT, D, B8> U(a, s, g, ctx);
  for (int c0 = u0; c0 < u1; c0 += U.CHUNK) {
    const int c1 = min(u1, c0 + U.CHUNK);
    U.window(c0, c1);
    MfmaK<DT, D> kb;
    MfmaV<DT, D> vb;
    U.issue_k(kb, c0);
    U.issue_v(vb, c0);
    for (int u = c0; u < c1; ++u) {
      const MfmaP<DT> p = scores(kb, u);
      if (u + 1 < c1) U.issue_k(kb, u + 1);
      pv(vb, p, u);
      if (u + 1 < c1) U.issue_v(vb, u + 1);
    }
  }
}

// Write the first ncols query columns of a finished piece: the normalised output (to `out`,
// column c at out_base + (c / group) * out_row_stride + (c % group) * out_col_stride, or to a
// partial slot, column c at po + c * po_col_stride), plus each column's max / sum for partial
// slots.  A column that saw no key writes 0.  (group = 16: column c at out_base + c * stride.)
template <int DT, int D>
__device__ __forceinline__ void mfma_emit(const MfmaState<DT, D>& st, int ncols, float* po,
                                          float* pm, float* pl, int64_t po_col_stride, void* out,
                                          int64_t out_base, int group, int64_t out_row_stride,
                                          int64_t out_col_stride, bool out_f32) {
  using C = MfmaCfg<DT, D>;
  const int lane = lane_id();
  const int r = lane >> 4, n = lane & 15;
  const float ltot = cross_rows_sum(st.l);  // sum of column n over the four lane rows
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (n < ncols) {
    const int64_t ocol = out_base + (int64_t)(n / group) * out_row_stride +
                         (int64_t)(n % group) * out_col_stride;
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
      const int d = 16 * j + 4 * r;  // this lane's four consecutive dimensions
      const f32x4_t v = st.acc[j] * inv;
      if (po) {
        *reinterpret_cast<f32x4_t*>(po + n * po_col_stride + d) = v;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) store_out<DT>(out, ocol + d + i, v[i], out_f32);
      }
    }
  }
  if (pm && r == 0 && n < ncols) {
    pm[n * (po_col_stride / D)] = st.m * 0.69314718055994531f;
    pl[n * (po_col_stride / D)] = ltot;
  }
}
}  // namespace pa
