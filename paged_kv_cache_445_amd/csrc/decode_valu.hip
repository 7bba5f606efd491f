// decode_valu.hip — paged-attention decode on the vector ALUs for multi-head attention (and
// the generic path for fp32): every wave runs HPW query heads of a work segment.
//
// The method ("vLLM 深度拆解：当 KV Cache 学会「分页」" §3.3 and §6.2): for every block of the
// sequence, look up its physical id in the block table, read the block's K and V, score
// each token with scale * q . k while the token index is below context_len, and finish
// with softmax(scores) . V (§2.2).  Here the softmax is streamed (running max m and sum l,
// rescaled when m grows), so each K/V tile is read exactly once.
//
// Both tiles of a block are read linearly: load i of a lane covers bytes
// [1024 i + 16 lane, +16) of the tile, so every load instruction is one contiguous KiB and
// the per-lane address is the same 32-bit offset for every tile (the tile base is a scalar).
// With the pool layout of include/pa.h (E-byte elements, X = 16 / E):
//   K tile [D/X chunks][16 tokens][X]: load i gives lane chunk 4i + lane/16 of token
//     lane%16.  The lane's partial dot product over its chunks is summed across the four
//     16-lane rows (gfx950 lane swaps), leaving token lane%16's score in every row.
//   V tile [D dims][16 tokens]: a dimension's 16 tokens are LPD = 16 E / 16 consecutive
//     16-byte pieces, so load j gives lane X tokens (group lane % LPD) of dimension
//     j * 64 / LPD + lane / LPD.  The lane accumulates those dimensions over its token group;
//     the LPD lanes of a dimension are summed once per piece of work.
//   The 16 softmax weights of a tile go through a 64-byte LDS slot of the wave; each lane
//   reads back the X weights of its token group.
//   Block-table entries sit one per lane in a 64-tile window and reach the scalar unit by
//   readlane.
// A wave runs the heads h0 + 4 j (j < HPW) of a segment tile by tile, head after head, so the
// four waves of a workgroup read 4 HPW adjacent heads of one block (16 KiB per head quartet
// for 16-bit K and as much for V) back to back before they move to the next block.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

template <int DT, int D>
struct VCfg {
  static constexpr int E = DtInfo<DT>::bytes;
  static constexpr int X = DtInfo<DT>::x;
  static constexpr int QE = DtInfo<DT>::qbytes;  // query element bytes
  static constexpr int TILE = 16 * D * E;  // bytes of one K or V tile
  static constexpr int NK = TILE / 1024;   // K loads per lane per tile
  static constexpr int NV = TILE / 1024;   // V loads per lane per tile
  static constexpr int LPD = 16 * E / 16;  // lanes sharing one V dimension row (>= 1)
  static constexpr int DPL = 64 / LPD;     // dimensions covered by one V load
  static constexpr int NQC = X * QE / 16;  // 16-byte query pieces per K chunk
  static constexpr int NQ = NK * NQC;      // 16-byte query pieces per head and lane
};

template <int DT, int D>
struct VTile {
  uint4 k[VCfg<DT, D>::NK];
  uint4 v[VCfg<DT, D>::NV];
};

template <int DT, int D>
struct VState {
  float m;                     // running max (base-2 domain), uniform
  float l;                     // running sum of token lane%16's weights
  float acc[VCfg<DT, D>::NV];  // unnormalised output over this lane's token group
};

template <int DT, int D>
__device__ __forceinline__ void v_issue(VTile<DT, D>& t, const char* kt, const char* vt, int off) {
  using C = VCfg<DT, D>;
#pragma unroll
  for (int i = 0; i < C::NK; ++i) t.k[i] = ld16_nt(kt + off + 1024 * i);
#pragma unroll
  for (int j = 0; j < C::NV; ++j) t.v[j] = ld16_nt(vt + off + 1024 * j);
}

// 8-token blocks: tokens 0-7 of a 16-token tile come from block tile (ka, va), tokens 8-15
// from (kb, vb), each an 8-token pool tile (K [D/X][8][X], V [D][8]).  Every lane loads the
// same pieces as from a 16-token tile, from its own block: K load i, lane l: chunk
// 4 i + l / 16 of token l % 16 (block (l / 8) % 2); V load j: the lane's dimension and token
// group of the 16-token layout (FP8: a dimension's 8 bytes from each block).
template <int DT, int D>
__device__ __forceinline__ void v_issue_b8(VTile<DT, D>& t, const char* ka, const char* kb,
                                           const char* va, const char* vb) {
  using C = VCfg<DT, D>;
  const int lane = lane_id();
  const char* kt = (lane & 8) ? kb : ka;
  const int koff = (lane >> 4) * 128 + (lane & 7) * 16;
#pragma unroll
  for (int i = 0; i < C::NK; ++i) t.k[i] = ld16_nt(kt + koff + 512 * i);
  if constexpr (C::E == 1) {
#pragma unroll
    for (int j = 0; j < C::NV; ++j) {
      const uint2 x = *reinterpret_cast<const uint2*>(va + 512 * j + 8 * lane);
      const uint2 y = *reinterpret_cast<const uint2*>(vb + 512 * j + 8 * lane);
      t.v[j] = make_uint4(x.x, x.y, y.x, y.y);
    }
  } else if constexpr (C::E == 2) {
    const char* vt = (lane & 1) ? vb : va;
#pragma unroll
    for (int j = 0; j < C::NV; ++j) t.v[j] = ld16_nt(vt + 512 * j + (lane >> 1) * 16);
  } else {
    const char* vt = ((lane >> 1) & 1) ? vb : va;
#pragma unroll
    for (int j = 0; j < C::NV; ++j)
      t.v[j] = ld16_nt(vt + 512 * j + (lane >> 2) * 32 + (lane & 1) * 16);
  }
}

// element k of a 16-byte V piece as float
template <int DT>
__device__ __forceinline__ float v_elem(const uint4& v, int k) {
  if constexpr (DT == DT_F32) {
    const uint32_t w = k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
    return __uint_as_float(w);
  } else {
    return elem16<DT>(v, k);
  }
}

// zero the elements of tokens >= valid (their slots may hold poison, and 0 * NaN is NaN)
template <int DT>
__device__ __forceinline__ void mask_piece(uint4& v, int first_token, int valid) {
  constexpr int X = DtInfo<DT>::x;
  const int n = min(X, max(0, valid - first_token));  // leading elements kept
  uint32_t m[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if constexpr (X == 4) {
      m[w] = w < n ? 0xffffffffu : 0u;
    } else {
      m[w] = (2 * w < n ? 0xffffu : 0u) | (2 * w + 1 < n ? 0xffff0000u : 0u);
    }
  }
  v.x &= m[0];
  v.y &= m[1];
  v.z &= m[2];
  v.w &= m[3];
}

// FP8: q . k over a 16-byte K chunk of 16 E4M3 values, each pair widened to the query's
// 16-bit type (fp16 for DT_FP8, bf16 for DT_FP8B; exact) and dotted with its two query
// elements (q0: elements 0-7, q1: 8-15) into the fp32 sum.
template <int DT>
__device__ __forceinline__ float dot_fp8(const uint4& k, const uint4& q0, const uint4& q1,
                                         float acc) {
  constexpr bool BF = DT == DT_FP8B;
  auto dot2 = [](uint32_t a, uint32_t b, float c) {
    if constexpr (BF)
      return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a),
                                             __builtin_bit_cast(bf162_t, b), c, false);
    else
      return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a),
                                    __builtin_bit_cast(half2_t, b), c, false);
  };
  const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
  const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    acc = dot2(fp8x2_to_16<BF, false>(kw[m]), qw[2 * m], acc);
    acc = dot2(fp8x2_to_16<BF, true>(kw[m]), qw[2 * m + 1], acc);
  }
  return acc;
}

// One 16-token tile.  MASK: only tokens < valid exist.
template <int DT, int D, bool MASK>
__device__ __forceinline__ void v_tile(VState<DT, D>& st, VTile<DT, D>& t, const uint4* qv,
                                       float scale_log2, int valid, float* pw) {
  using C = VCfg<DT, D>;
  const int lane = lane_id();
  float part = 0.f;
  if constexpr (is_fp8(DT)) {
    // each 16-byte K chunk is 16 E4M3 values, dotted with the chunk's 16 query elements
    // (k_scale is in the score factor)
#pragma unroll
    for (int i = 0; i < C::NK; ++i) part = dot_fp8<DT>(t.k[i], qv[2 * i], qv[2 * i + 1], part);
  } else {
#pragma unroll
    for (int i = 0; i < C::NK; ++i) part = dot16<DT>(t.k[i], qv[i], part);
  }
  float sc = cross_rows_sum(part) * scale_log2;
  if (MASK && (lane & 15) >= valid) sc = -INFINITY;
  const float mnew = fmaxf(st.m, row16_max(sc));
  const float alpha = __builtin_amdgcn_exp2f(st.m - mnew);
  const float p = __builtin_amdgcn_exp2f(sc - mnew);
  st.l = st.l * alpha + p;
  st.m = mnew;
  if (lane < 16) pw[lane] = p;
  __builtin_amdgcn_wave_barrier();
  const int g = lane % C::LPD;  // token group: tokens X g .. X g + X - 1
  float w[C::X];
#pragma unroll
  for (int k = 0; k < C::X; k += 4) {
    const float4 f = *reinterpret_cast<const float4*>(pw + C::X * g + k);
    w[k] = f.x;
    w[k + 1] = f.y;
    w[k + 2] = f.z;
    w[k + 3] = f.w;
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < C::NV; ++j) {
    float a = st.acc[j] * alpha;
    if constexpr (is_fp8(DT)) {
      // the 16 tokens of one dimension row; tokens >= valid are zeroed (MASK)
      const uint32_t vw[4] = {t.v[j].x, t.v[j].y, t.v[j].z, t.v[j].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        float f[4];
        fp8x4_to_f32(vw[m], f);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (MASK && 4 * m + k >= valid) f[k] = 0.f;
          a = fmaf(w[4 * m + k], f[k], a);
        }
      }
    } else {
      if (MASK) mask_piece<DT>(t.v[j], C::X * g, valid);
#pragma unroll
      for (int k = 0; k < C::X; ++k) a = fmaf(w[k], v_elem<DT>(t.v[j], k), a);
    }
    st.acc[j] = a;
  }
}

// A piece: query heads h0 + 4 j (j < HPW) of sequence s over its tiles [t0, t1).  Every
// field is wave-uniform.
struct VPiece {
  int s, h0, t0, t1, ctx;
};

// The loads a piece needs before its tile loop: the block-table window of its first chunk,
// the query of its heads and its first step (tile t0 of head h0).  They are issued while
// the previous piece ends, so a wave moves from piece to piece without draining its loads.
template <int DT, int D, int HPW>
struct VStart {
  int win0, win1;  // entries t0 + lane and t0 + 64 + lane of the block table
  uint4 q[HPW][VCfg<DT, D>::NQ];
  VTile<DT, D> first;
};

// tiles per block-table window chunk
template <bool B8>
constexpr int kValuChunk = B8 ? 64 : 128;

// Block-table window of the first chunk of p (tiles t0 .. t0 + 127, or 63 with 8-token blocks).
template <bool B8>
__device__ __forceinline__ void v_window(const DecodeArgs& a, const VPiece& p, int& win0,
                                         int& win1) {
  const int32_t* bt_row = a.block_tables + (int64_t)p.s * a.max_blocks_per_seq;
  load_window<B8>(bt_row, p.t0, min(p.t1, p.t0 + kValuChunk<B8>), p.ctx, a.blk_shift, win0, win1);
}

// a pool tile of one KV head: 16 tokens, or 8 with 8-token blocks
template <int DT, int D, bool B8>
constexpr int64_t kPoolTile = B8 ? VCfg<DT, D>::TILE / 2 : VCfg<DT, D>::TILE;

template <int DT, int D, bool B8>
__device__ __forceinline__ const char* v_head_base(const void* pool, const DecodeArgs& a, int h) {
  const int64_t kvh = h / (a.num_q_heads / a.num_kv_heads);
  return reinterpret_cast<const char*>(pool) + kvh * kPoolTile<DT, D, B8>;
}

// Issue the query and first-step loads of p (vs.win0 / win1 already hold its window).
template <int DT, int D, int HPW, bool B8>
__device__ __forceinline__ void v_start(const DecodeArgs& a, const VPiece& p,
                                        VStart<DT, D, HPW>& vs) {
  using C = VCfg<DT, D>;
  const int lane = lane_id();
  const int row = a.qsl ? a.qsl[p.s] : p.s;
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     ((int64_t)row * a.num_q_heads + p.h0 + 4 * j) * D * C::QE;
    // the query elements of this lane's K chunks 4 i + lane / 16 (X elements each)
#pragma unroll
    for (int i = 0; i < C::NK; ++i)
#pragma unroll
      for (int c = 0; c < C::NQC; ++c)
        vs.q[j][C::NQC * i + c] = ld16(qp + C::X * C::QE * (4 * i + (lane >> 4)) + 16 * c);
  }
  const int64_t stride = a.num_kv_heads * kPoolTile<DT, D, B8>;
  const char* kh = v_head_base<DT, D, B8>(a.k_cache, a, p.h0);
  const char* vh = v_head_base<DT, D, B8>(a.v_cache, a, p.h0);
  if constexpr (B8) {
    const int64_t ba = readlane(vs.win0, 0), bb = readlane(vs.win0, 1);
    v_issue_b8<DT, D>(vs.first, kh + ba * stride, kh + bb * stride, vh + ba * stride,
                      vh + bb * stride);
  } else {
    const int64_t off = readlane(vs.win0, 0) * stride;
    v_issue<DT, D>(vs.first, kh + off, vh + off, 16 * lane);
  }
}

// Attention of piece p, whose start loads vs are in flight.  The tiles are walked in chunks
// of 128, each with its 64-entry block-table windows in registers before its pipelined
// loop (the first chunk's come with vs), so the loop itself only waits for tile loads.  A
// step is one tile of one head; the loads of the next step are in flight while a step is
// computed.
template <int DT, int D, int HPW, bool B8>
__device__ void valu_run(const DecodeArgs& a, VPiece p, VStart<DT, D, HPW>& vs,
                         VState<DT, D> (&st)[HPW], float* pw) {
  using C = VCfg<DT, D>;
  const int lane = lane_id();
  // every per-piece value is wave-uniform: keep it in scalar registers
  p.s = __builtin_amdgcn_readfirstlane(p.s);
  p.h0 = __builtin_amdgcn_readfirstlane(p.h0);
  p.t0 = __builtin_amdgcn_readfirstlane(p.t0);
  p.t1 = __builtin_amdgcn_readfirstlane(p.t1);
  p.ctx = __builtin_amdgcn_readfirstlane(p.ctx);
  const int off = 16 * lane;
  const char* kc[HPW];
  const char* vc[HPW];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    kc[j] = v_head_base<DT, D, B8>(a.k_cache, a, p.h0 + 4 * j);
    vc[j] = v_head_base<DT, D, B8>(a.v_cache, a, p.h0 + 4 * j);
    st[j].m = -INFINITY;
    st[j].l = 0.f;
#pragma unroll
    for (int e = 0; e < C::NV; ++e) st[j].acc[e] = 0.f;
  }
  const int64_t blk_stride = (int64_t)a.num_kv_heads * kPoolTile<DT, D, B8>;
  const int32_t* bt_row = a.block_tables + (int64_t)p.s * a.max_blocks_per_seq;
  constexpr int CH = kValuChunk<B8>;

  // one chunk [c0, c1); FIRST: its first step is already in flight in vs.first
  auto chunk = [&](int c0, int c1, int win0, int win1, auto first) {
    auto issue = [&](VTile<DT, D>& t, int tt, int j) {
      const int idx = tt - c0;
      if constexpr (B8) {
        const int e = 2 * idx;  // blocks e and e + 1 (e even: both in one register)
        const int64_t ba = e < 64 ? readlane(win0, e) : readlane(win1, e - 64);
        const int64_t bb = e < 64 ? readlane(win0, e + 1) : readlane(win1, e - 63);
        v_issue_b8<DT, D>(t, kc[j] + ba * blk_stride, kc[j] + bb * blk_stride,
                          vc[j] + ba * blk_stride, vc[j] + bb * blk_stride);
      } else {
        const int64_t blk = idx < 64 ? readlane(win0, idx) : readlane(win1, idx - 64);
        v_issue<DT, D>(t, kc[j] + blk * blk_stride, vc[j] + blk * blk_stride, off);
      }
    };
    auto step = [&](VTile<DT, D>& t, int tt, int j) {
      const int valid = p.ctx - tt * kBlock;
      if (valid >= kBlock)
        v_tile<DT, D, false>(st[j], t, vs.q[j], a.scale_log2, kBlock, pw);
      else
        v_tile<DT, D, true>(st[j], t, vs.q[j], a.scale_log2, valid, pw);
    };
    // Two-stage software pipeline over steps.  The steady-state loop always issues, so
    // every path into a step has the same loads outstanding and the wait before it covers
    // only that step; the last tiles of the chunk are peeled.
    VTile<DT, D>& ta = vs.first;
    VTile<DT, D> tb;
    if constexpr (!decltype(first)::value) issue(ta, c0, 0);
    int tt = c0;
    if constexpr (HPW == 1) {
      for (; tt + 2 < c1; tt += 2) {
        issue(tb, tt + 1, 0);
        step(ta, tt, 0);
        issue(ta, tt + 2, 0);
        step(tb, tt + 1, 0);
      }
      if (tt + 1 < c1) {
        issue(tb, tt + 1, 0);
        step(ta, tt, 0);
        step(tb, tt + 1, 0);
      } else {
        step(ta, tt, 0);
      }
    } else {
      static_assert(HPW % 2 == 0, "steps alternate between two tile buffers");
      for (; tt + 1 < c1; ++tt) {
        static_for<0, HPW>([&](auto J) {
          constexpr int j = decltype(J)::value;
          VTile<DT, D>& cur = (j % 2 == 0) ? ta : tb;
          VTile<DT, D>& nxt = (j % 2 == 0) ? tb : ta;
          if constexpr (j + 1 < HPW)
            issue(nxt, tt, j + 1);
          else
            issue(nxt, tt + 1, 0);
          step(cur, tt, j);
        });
      }
      static_for<0, HPW>([&](auto J) {
        constexpr int j = decltype(J)::value;
        VTile<DT, D>& cur = (j % 2 == 0) ? ta : tb;
        VTile<DT, D>& nxt = (j % 2 == 0) ? tb : ta;
        if constexpr (j + 1 < HPW) issue(nxt, tt, j + 1);
        step(cur, tt, j);
      });
    }
  };
  chunk(p.t0, min(p.t1, p.t0 + CH), vs.win0, vs.win1, std::true_type{});
  for (int c0 = p.t0 + CH; c0 < p.t1; c0 += CH) {
    const int c1 = min(p.t1, c0 + CH);
    int win0, win1;
    load_window<B8>(bt_row, c0, c1, p.ctx, a.blk_shift, win0, win1);
    chunk(c0, c1, win0, win1, std::false_type{});
  }
  (void)lane;
}

// Finish a piece: combine the lanes of each dimension row and the per-token sums; returns
// the total l (every lane).  Afterwards every lane holds full sums for its dimensions.  FP8
// pools: the sums are also multiplied by vfac (v_scale: a stored V value stands for its E4M3
// value times v_scale).
template <int DT, int D>
__device__ __forceinline__ float v_finish(VState<DT, D>& st, float vfac) {
  using C = VCfg<DT, D>;
#pragma unroll
  for (int j = 0; j < C::NV; ++j) {
    if constexpr (C::LPD >= 2) st.acc[j] += dpp_mov<0xB1>(st.acc[j]);  // [1,0,3,2]: lane ^ 1
    if constexpr (C::LPD == 4) st.acc[j] += dpp_mov<0x4E>(st.acc[j]);  // [2,3,0,1]: ^ 2
    if constexpr (is_fp8(DT)) st.acc[j] *= vfac;
  }
  return row16_sum(st.l);
}

// Store a finished head's output scaled by inv: dimension j * DPL + lane / LPD of each load j.
template <int DT, int D>
__device__ __forceinline__ void v_store(const float (&acc)[VCfg<DT, D>::NV], float inv,
                                        void* out, int64_t base, bool out_f32) {
  using C = VCfg<DT, D>;
  const int lane = lane_id();
  if (lane % C::LPD == 0) {
#pragma unroll
    for (int j = 0; j < C::NV; ++j)
      store_out<DT>(out, base + j * C::DPL + lane / C::LPD, acc[j] * inv, out_f32);
  }
}

template <int DT, int D>
__device__ __forceinline__ void v_store_f32(const VState<DT, D>& st, float inv, float* po) {
  using C = VCfg<DT, D>;
  const int lane = lane_id();
  if (lane % C::LPD == 0) {
#pragma unroll
    for (int j = 0; j < C::NV; ++j) po[j * C::DPL + lane / C::LPD] = st.acc[j] * inv;
  }
}

// Folds the np shared-prefix partials of (row, query head h) into a merged head held as
// (M, L, U): U[e] is this lane's dimension e * DPL + lane / LPD.
template <int DT, int D>
__device__ __forceinline__ void v_fold(const DecodeArgs& a, float& M, float& L,
                                       float (&U)[VCfg<DT, D>::NV], int64_t row, int h, int np) {
  using C = VCfg<DT, D>;
  const int dim0 = lane_id() / C::LPD;
  const int64_t e = (row * a.num_q_heads + h) * a.pre_parts;
  fold_prefix<C::NV, 4>(M, L, U, a.pre_m + e, a.pre_l + e, a.pre_o + e * D, D, np,
                        [&](int k) { return k * C::DPL + dim0; });
}

// A finished head of a whole segment of a sequence with a shared prefix (row, query head h,
// output at ob): its keys past the prefix folded with the np prefix partials.
template <int DT, int D>
__device__ __forceinline__ void v_prefix_store(const DecodeArgs& a, const VState<DT, D>& st,
                                               float l, int64_t row, int h, int np,
                                               int64_t ob) {
  using C = VCfg<DT, D>;
  float M = st.m * 0.69314718055994531f, L = l, U[C::NV];
#pragma unroll
  for (int e = 0; e < C::NV; ++e) U[e] = st.acc[e];
  v_fold<DT, D>(a, M, L, U, row, h, np);
  v_store<DT, D>(U, 1.f / L, a.out, ob, a.out_f32);
}

// A piece of a split segment (heads h0 + 4 j of row `row`): publish it, or (if it is the
// segment's last arrival) merge every piece, fold in the np shared-prefix partials of each
// head (np > 0) and write the output; `between` (the next piece's start loads) runs once, as
// early as the arrival protocol allows.  Every lane holds full sums for its dimensions after
// v_finish, so each lane reads and merges its own dimensions of every head.  Slot rows: head
// j of a piece is row (slot HPW + j) of the partial arrays.
template <int DT, int D, int HPW, class Between>
__device__ void v_split_finish(const DecodeArgs& a, const VState<DT, D> (&st)[HPW],
                               const float (&l)[HPW], const SplitSeg& sg, int64_t self,
                               int32_t* cnt, int seen, int64_t ob0, int64_t row, int h0, int np,
                               Between&& between) {
  using C = VCfg<DT, D>;
  const int lane = lane_id();
  const int dim0 = lane / C::LPD;  // dimension e * DPL + dim0 of load e
  // this piece's partial as published: normalised output, max (natural log), sum
  float mine_m[HPW], mine_o[HPW][C::NV];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const float inv = 1.f / l[j];
    mine_m[j] = st[j].m * 0.69314718055994531f;
#pragma unroll
    for (int e = 0; e < C::NV; ++e) mine_o[j][e] = st[j].acc[e] * inv;
  }
  const bool last = split_arrive(cnt, (int)(sg.k1 - sg.k0), seen, [&] {
    const int64_t row0 = piece_slot(sg, self) * HPW;
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      if (lane % C::LPD == 0) {
#pragma unroll
        for (int e = 0; e < C::NV; ++e)
          coh_store(a.part_o + (row0 + j) * D + e * C::DPL + dim0, mine_o[j][e]);
      }
      if (lane == 0) {
        coh_store(a.part_m + row0 + j, mine_m[j]);
        coh_store(a.part_l + row0 + j, l[j]);
      }
    }
  }, between);
  if (!last) return;
  float M[HPW], L[HPW], U[HPW][C::NV];
  merge_ordered<HPW, C::NV, (HPW > 2 ? 1 : 2)>(
      M, L, U, sg.k0, sg.k1,
      [&](int64_t k, float (&m)[HPW], float (&lk)[HPW], float (&ov)[HPW][C::NV]) {
        if (k == self) {
#pragma unroll
          for (int j = 0; j < HPW; ++j) {
            m[j] = mine_m[j];
            lk[j] = l[j];
#pragma unroll
            for (int e = 0; e < C::NV; ++e) ov[j][e] = mine_o[j][e];
          }
          return;
        }
        const int64_t row0 = piece_slot(sg, k) * HPW;
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
          m[j] = coh_load(a.part_m + row0 + j);
          lk[j] = coh_load(a.part_l + row0 + j);
#pragma unroll
          for (int e = 0; e < C::NV; ++e)
            ov[j][e] = coh_load(a.part_o + (row0 + j) * D + e * C::DPL + dim0);
        }
      });
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    if (np > 0) v_fold<DT, D>(a, M[j], L[j], U[j], row, h0 + 4 * j, np);
    v_store<DT, D>(U[j], 1.f / L[j], a.out, ob0 + 4 * j * D, a.out_f32);
  }
  counter_reset(cnt);
}

template <int DT, int D, int MODE, int HPW, bool B8>
__global__ __launch_bounds__(kWG) void valu_decode_kernel(DecodeArgs a) {
  // LDS: one 16-float weight slot per wave (first, for 16-byte alignment), then the plan
  // (S + 1 ints)
  extern __shared__ __align__(16) int32_t lds[];
  const int S = a.num_seqs;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  float* pw = reinterpret_cast<float*>(lds) + 16 * wave;
  int32_t* base = lds + 16 * kWavesPerWG;
  const int64_t W = (int64_t)gridDim.x * kWavesPerWG;
  const int64_t w = (int64_t)blockIdx.x * kWavesPerWG + wave;

  if constexpr (MODE == MODE_EVEN) {
    PlanIn pin{a.context_lens, a.qsl, S, kValuUnit, a.seg_extra, 1, a.skip};
    build_plan(base, pin);
    zero_empty_rows<DT>(pin, a.out, a.num_q_heads, D, w, W, a.out_f32, a.nan_rows);
    // units: (sequence, group of 4 HPW heads, tile); wave i runs heads i + 4 j of each group
    constexpr int GH = kWavesPerWG * HPW;
    const int groups = (a.num_q_heads + GH - 1) / GH;
    // the list is (sequence, head group, tile), or with xcd_major (head group, sequence,
    // tile) split over XCD-major owners, so that each XCD works through a few head groups of
    // every sequence and keeps the blocks several sequences share in its own L2
    const Part part = make_part((int64_t)base[S] * groups, gridDim.x, a.odd_skew, a.xcd_major);
    const int64_t per_group = base[S];
    even_split_drive(part, [&](int64_t o, int64_t lo, int64_t hi) {
      // this wave's piece of the segment that unit i of the range belongs to
      struct Unit {
        VPiece p;           // tiles [p.t0, p.t1) of the sequence
        int nt;             // real tiles of the segment
        int sk;             // keys [0, sk) come from the shared-prefix partials
        int64_t seg0, end;  // the segment's first unit, the piece's end in the range
        bool run;           // real heads and real tiles
        bool whole;         // the piece is the whole segment
      };
      auto at = [&](int64_t i) {
        Unit u;
        int grp, seglen;
        if (part.xcd) {
          grp = (int)(i / per_group);
          u.p.s = find_seq(base, S, i - grp * per_group, 1);
          seglen = base[u.p.s + 1] - base[u.p.s];
          u.seg0 = grp * per_group + base[u.p.s];
        } else {
          u.p.s = find_seq(base, S, i, groups);
          seglen = base[u.p.s + 1] - base[u.p.s];
          const int64_t sbase = (int64_t)base[u.p.s] * groups;
          grp = (int)((i - sbase) / seglen);
          u.seg0 = sbase + (int64_t)grp * seglen;
        }
        u.nt = seglen - a.seg_extra;  // real tiles; the rest only balance the split
        u.end = min(hi, u.seg0 + seglen);
        u.p.h0 = grp * GH + wave;  // this wave's first head (HPW > 1: all exist)
        const int t0 = (int)(i - u.seg0);  // the segment's tiles start past a shared prefix
        const int t1 = (int)min(u.end - u.seg0, (int64_t)u.nt);
        u.run = u.p.h0 < a.num_q_heads && t0 < u.nt;
        u.whole = t0 == 0 && t1 == u.nt;
        u.p.ctx = u.run ? a.context_lens[u.p.s] : 0;
        u.sk = u.run && a.skip ? a.skip[u.p.s] : 0;
        u.p.t0 = t0 + u.sk / kValuUnit;
        u.p.t1 = t1 + u.sk / kValuUnit;
        return u;
      };
      VStart<DT, D, HPW> vs;
      Unit cur = at(lo);
      if (cur.run) {
        v_window<B8>(a, cur.p, vs.win0, vs.win1);
        v_start<DT, D, HPW, B8>(a, cur.p, vs);
      }
      for (;;) {
        const bool more = cur.end < hi;
        Unit nxt{};
        if (more) nxt = at(cur.end);
        const bool nrun = more && nxt.run;
        int nw0 = 0, nw1 = 0;  // the next piece's window, read before this piece's tiles
        if (nrun) v_window<B8>(a, nxt.p, nw0, nw1);
        auto start_next = [&] {
          if (nrun) {
            vs.win0 = nw0;
            vs.win1 = nw1;
            v_start<DT, D, HPW, B8>(a, nxt.p, vs);
          }
        };
        if (cur.run) {
          const int row = a.qsl ? a.qsl[cur.p.s] : cur.p.s;
          const int64_t ob0 = ((int64_t)row * a.num_q_heads + cur.p.h0) * D;
          const bool whole = cur.whole;
          const int np = cur.sk > 0 ? (cur.sk + a.pre_tokens - 1) / a.pre_tokens : 0;
          SplitSeg sg{};
          int32_t* cnt = nullptr;
          int seen = 0;
          if (!whole) {
            sg = split_seg(part, cur.seg0, cur.seg0 + cur.nt - 1, wave);
            cnt = a.counters + kWavesPerWG * sg.k0 + wave;
            seen = counter_peek(cnt);  // consumed after the tiles
          }
          VState<DT, D> st[HPW];
          valu_run<DT, D, HPW, B8>(a, cur.p, vs, st, pw);
          float l[HPW];
#pragma unroll
          for (int j = 0; j < HPW; ++j) l[j] = v_finish<DT, D>(st[j], a.v_factor);
          if (whole) {
#pragma unroll
            for (int j = 0; j < HPW; ++j) {
              if (np > 0)
                v_prefix_store<DT, D>(a, st[j], l[j], row, cur.p.h0 + 4 * j, np, ob0 + 4 * j * D);
              else
                v_store<DT, D>(st[j].acc, 1.f / l[j], a.out, ob0 + 4 * j * D, a.out_f32);
            }
            start_next();
          } else if constexpr (HPW <= 2) {
            v_split_finish<DT, D, HPW>(a, st, l, sg, o, cnt, seen, ob0, row, cur.p.h0, np,
                                       start_next);
          } else {
            // with four or more heads the next piece's queries and a merge do not fit in
            // the registers together: start it once this piece is done
            v_split_finish<DT, D, HPW>(a, st, l, sg, o, cnt, seen, ob0, row, cur.p.h0, np,
                                       [] {});
            start_next();
          }
        } else {
          start_next();
        }
        if (!more) break;
        cur = nxt;
      }
    });
  } else {
    // fixed partitions of the sequences with one query row (with query_start_loc, the
    // others are the chunk kernel's)
    const int PU = a.partition_units;  // tiles per partition
    const int P = a.max_partitions;
    PlanIn pin{a.context_lens, a.qsl, S, PU * kBlock, 0, 1};
    build_plan(base, pin);
    fill_past_partitions(a.context_lens, a.qsl, S, a.qsl ? a.qsl[S] : S, a.num_q_heads, P,
                         PU * kBlock, a.part_m, a.part_l, w, W);
    const int segs = a.num_q_heads;
    const int64_t total = (int64_t)base[S] * segs;
    for (int64_t i = w; i < total; i += W) {
      const int s = find_seq(base, S, i, segs);
      const int np = base[s + 1] - base[s];
      const int64_t sbase = (int64_t)base[s] * segs;
      const int h = (int)((i - sbase) / np);
      const int p = (int)(i - sbase - (int64_t)h * np);
      const int ctx = a.context_lens[s];
      const int nt = (ctx + kBlock - 1) / kBlock;
      const int t0 = p * PU, t1 = min(nt, t0 + PU);
      VState<DT, D> st[1];
      const VPiece pc{s, h, t0, t1, ctx};
      VStart<DT, D, 1> vs;
      v_window<B8>(a, pc, vs.win0, vs.win1);
      v_start<DT, D, 1, B8>(a, pc, vs);
      valu_run<DT, D, 1, B8>(a, pc, vs, st, pw);
      const float l = v_finish<DT, D>(st[0], a.v_factor);
      const float inv = 1.f / l;
      const int64_t row = a.qsl ? a.qsl[s] : s;
      const int64_t e = (row * a.num_q_heads + h) * P + p;
      v_store_f32<DT, D>(st[0], inv, a.part_o + e * D);
      if (lane == 0) {
        a.part_m[e] = st[0].m * 0.69314718055994531f;
        a.part_l[e] = l;
      }
    }
  }
}

static size_t valu_lds_bytes(int num_seqs) {
  return (size_t)(num_seqs + 1) * sizeof(int32_t) + kWavesPerWG * 16 * sizeof(float);
}

template <int DT, int D, int MODE, int HPW, bool B8 = false>
static void launch_k(const DecodeArgs& a, int grid, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((valu_decode_kernel<DT, D, MODE, HPW, B8>), dim3(grid), dim3(kWG), lds, st, a);
}

template <int DT, int D, int MODE>
static void launch_hpw(const DecodeArgs& a, int grid, size_t lds, hipStream_t st) {
  // 8-token blocks: one head per wave
  if (a.b8) return launch_k<DT, D, MODE, 1, true>(a, grid, lds, st);
  if constexpr (MODE == MODE_EVEN) {
    // fp32 queries fill twice the registers: at most two heads per wave; FP8 widens to
    // fp32 in registers: at most four
    if constexpr (DT != DT_F32 && !is_fp8(DT)) {
      if (a.heads_per_wave == 8) return launch_k<DT, D, MODE, 8>(a, grid, lds, st);
    }
    if constexpr (DT != DT_F32) {
      if (a.heads_per_wave == 4) return launch_k<DT, D, MODE, 4>(a, grid, lds, st);
    }
    if (a.heads_per_wave == 2) return launch_k<DT, D, MODE, 2>(a, grid, lds, st);
  }
  launch_k<DT, D, MODE, 1>(a, grid, lds, st);
}

template <int DT, int MODE>
static hipError_t launch_d(const DecodeArgs& a, int grid, hipStream_t st) {
  const size_t lds = valu_lds_bytes(a.num_seqs);
  if (a.head_dim == 64)
    launch_hpw<DT, 64, MODE>(a, grid, lds, st);
  else
    launch_hpw<DT, 128, MODE>(a, grid, lds, st);
  return hipGetLastError();
}

hipError_t launch_valu_decode(int dt, int mode, const DecodeArgs& a, int grid, hipStream_t st) {
  if (mode == MODE_EVEN) {
    if (dt == DT_F32) return launch_d<DT_F32, MODE_EVEN>(a, grid, st);
    if (dt == DT_F16) return launch_d<DT_F16, MODE_EVEN>(a, grid, st);
    if (dt == DT_FP8) return launch_d<DT_FP8, MODE_EVEN>(a, grid, st);
    if (dt == DT_FP8B) return launch_d<DT_FP8B, MODE_EVEN>(a, grid, st);
    return launch_d<DT_BF16, MODE_EVEN>(a, grid, st);
  }
  if (dt == DT_F32) return launch_d<DT_F32, MODE_PARTITION>(a, grid, st);
  if (dt == DT_F16) return launch_d<DT_F16, MODE_PARTITION>(a, grid, st);
  if (dt == DT_FP8) return launch_d<DT_FP8, MODE_PARTITION>(a, grid, st);
  if (dt == DT_FP8B) return launch_d<DT_FP8B, MODE_PARTITION>(a, grid, st);
  return launch_d<DT_BF16, MODE_PARTITION>(a, grid, st);
}

// resident workgroups per CU of the kernel that `hpw` selects (the 8-token-block variants
// are built for the same occupancy)
template <int DT, int MODE, int HPW>
static int occ_k(int head_dim, int lds) {
  int n = 0;
  hipError_t e;
  if (head_dim == 64)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, valu_decode_kernel<DT, 64, MODE, HPW, false>, kWG, lds);
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, valu_decode_kernel<DT, 128, MODE, HPW, false>, kWG, lds);
  return e == hipSuccess && n > 0 ? n : 1;
}

template <int DT, int MODE>
static int occ(int head_dim, int hpw, int lds) {
  if constexpr (MODE == MODE_EVEN) {
    if constexpr (DT != DT_F32 && !is_fp8(DT)) {
      if (hpw == 8) return occ_k<DT, MODE, 8>(head_dim, lds);
    }
    if constexpr (DT != DT_F32) {
      if (hpw == 4) return occ_k<DT, MODE, 4>(head_dim, lds);
    }
    if (hpw == 2) return occ_k<DT, MODE, 2>(head_dim, lds);
  }
  return occ_k<DT, MODE, 1>(head_dim, lds);
}

int valu_decode_max_blocks_per_cu(int dt, int head_dim, int hpw, int mode, int lds_bytes) {
  const int lds = lds_bytes + kWavesPerWG * 16 * (int)sizeof(float);
  if (mode == MODE_EVEN) {
    if (dt == DT_F32) return occ<DT_F32, MODE_EVEN>(head_dim, hpw, lds);
    if (dt == DT_F16) return occ<DT_F16, MODE_EVEN>(head_dim, hpw, lds);
    if (dt == DT_FP8) return occ<DT_FP8, MODE_EVEN>(head_dim, hpw, lds);
    if (dt == DT_FP8B) return occ<DT_FP8B, MODE_EVEN>(head_dim, hpw, lds);
    return occ<DT_BF16, MODE_EVEN>(head_dim, hpw, lds);
  }
  if (dt == DT_F32) return occ<DT_F32, MODE_PARTITION>(head_dim, 1, lds);
  if (dt == DT_F16) return occ<DT_F16, MODE_PARTITION>(head_dim, 1, lds);
  if (dt == DT_FP8) return occ<DT_FP8, MODE_PARTITION>(head_dim, 1, lds);
  if (dt == DT_FP8B) return occ<DT_FP8B, MODE_PARTITION>(head_dim, 1, lds);
  return occ<DT_BF16, MODE_PARTITION>(head_dim, 1, lds);
}

}  // namespace pa
