// decode_valu.hip — paged-attention decode on the vector ALUs, one query head per work
// segment (multi-head attention; also the generic path for fp32).
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
//   Block-table entries sit one per lane in a 64-tile window (the next window is loaded
//   ahead) and reach the scalar unit by readlane.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

template <int DT, int D>
struct VCfg {
  static constexpr int E = DtInfo<DT>::bytes;
  static constexpr int X = DtInfo<DT>::x;
  static constexpr int TILE = 16 * D * E;  // bytes of one K or V tile
  static constexpr int NK = TILE / 1024;   // K loads per lane per tile
  static constexpr int NV = TILE / 1024;   // V loads per lane per tile
  static constexpr int LPD = 16 * E / 16;  // lanes sharing one V dimension row
  static constexpr int DPL = 64 / LPD;     // dimensions covered by one V load
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
  for (int i = 0; i < C::NK; ++i) t.k[i] = ld16(kt + off + 1024 * i);
#pragma unroll
  for (int j = 0; j < C::NV; ++j) t.v[j] = ld16(vt + off + 1024 * j);
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

// One 16-token tile.  MASK: only tokens < valid exist.
template <int DT, int D, bool MASK>
__device__ __forceinline__ void v_tile(VState<DT, D>& st, VTile<DT, D>& t, const uint4* qv,
                                       float scale_log2, int valid, float* pw) {
  using C = VCfg<DT, D>;
  const int lane = lane_id();
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < C::NK; ++i) part = dot16<DT>(t.k[i], qv[i], part);
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
    if (MASK) mask_piece<DT>(t.v[j], C::X * g, valid);
    float a = st.acc[j] * alpha;
#pragma unroll
    for (int k = 0; k < C::X; ++k) a = fmaf(w[k], v_elem<DT>(t.v[j], k), a);
    st.acc[j] = a;
  }
}

// Attention of query head h of sequence s over its tiles [t0, t1).  The tiles are walked in
// chunks of 128: both 64-entry block-table windows of a chunk are loaded before its
// pipelined tile loop, so the loop itself only waits for tile loads.
template <int DT, int D>
__device__ void valu_attend(const DecodeArgs& a, int s, int h, int t0, int t1, int ctx,
                            VState<DT, D>& st, float* pw) {
  using C = VCfg<DT, D>;
  const int lane = lane_id();
  // every per-piece value is wave-uniform: keep it in scalar registers
  s = __builtin_amdgcn_readfirstlane(s);
  h = __builtin_amdgcn_readfirstlane(h);
  t0 = __builtin_amdgcn_readfirstlane(t0);
  t1 = __builtin_amdgcn_readfirstlane(t1);
  ctx = __builtin_amdgcn_readfirstlane(ctx);
  const int G = a.num_q_heads / a.num_kv_heads;
  const int kvh = h / G;
  const int row = __builtin_amdgcn_readfirstlane(a.qsl ? a.qsl[s] : s);
  const int off = 16 * lane;
  uint4 qv[C::NK];
  {
    const char* qp = reinterpret_cast<const char*>(a.q) + ((int64_t)row * a.num_q_heads + h) * D * C::E;
#pragma unroll
    for (int i = 0; i < C::NK; ++i) qv[i] = ld16(qp + 16 * (4 * i + (lane >> 4)));
  }
  const int64_t blk_stride = (int64_t)a.num_kv_heads * C::TILE;
  const char* kc = reinterpret_cast<const char*>(a.k_cache) + (int64_t)kvh * C::TILE;
  const char* vc = reinterpret_cast<const char*>(a.v_cache) + (int64_t)kvh * C::TILE;
  const int32_t* bt_row = a.block_tables + (int64_t)s * a.max_blocks_per_seq;

  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int j = 0; j < C::NV; ++j) st.acc[j] = 0.f;

  for (int c0 = t0; c0 < t1; c0 += 128) {
    const int c1 = min(t1, c0 + 128);
    const int win0 = (c0 + lane < c1) ? bt_row[c0 + lane] : 0;
    const int win1 = (c0 + 64 + lane < c1) ? bt_row[c0 + 64 + lane] : 0;
    auto issue = [&](VTile<DT, D>& t, int tt) {
      const int idx = tt - c0;
      const int64_t blk = idx < 64 ? readlane(win0, idx) : readlane(win1, idx - 64);
      v_issue<DT, D>(t, kc + blk * blk_stride, vc + blk * blk_stride, off);
    };
    auto tile = [&](VTile<DT, D>& t, int tt) {
      const int valid = ctx - tt * kBlock;
      if (valid >= kBlock)
        v_tile<DT, D, false>(st, t, qv, a.scale_log2, kBlock, pw);
      else
        v_tile<DT, D, true>(st, t, qv, a.scale_log2, valid, pw);
    };
    // two-stage software pipeline: the loads of tile tt + 1 are in flight while tile tt is
    // computed.  The steady-state loop always issues, so every path into a tile has the
    // same loads outstanding and the wait before it covers only that tile.
    VTile<DT, D> ta, tb;
    issue(ta, c0);
    int tt = c0;
    for (; tt + 2 < c1; tt += 2) {
      issue(tb, tt + 1);
      tile(ta, tt);
      issue(ta, tt + 2);
      tile(tb, tt + 1);
    }
    if (tt + 1 < c1) {
      issue(tb, tt + 1);
      tile(ta, tt);
      tile(tb, tt + 1);
    } else {
      tile(ta, tt);
    }
  }
}

// Finish a piece: combine the lanes of each dimension row and the per-token sums; returns
// the total l (every lane).  Afterwards lanes with lane % LPD == 0 hold full dimension sums.
template <int DT, int D>
__device__ __forceinline__ float v_finish(VState<DT, D>& st) {
  using C = VCfg<DT, D>;
#pragma unroll
  for (int j = 0; j < C::NV; ++j) {
    st.acc[j] += dpp_mov<0xB1>(st.acc[j]);    // quad_perm [1,0,3,2]: partner lane ^ 1
    if constexpr (C::LPD == 4) st.acc[j] += dpp_mov<0x4E>(st.acc[j]);  // [2,3,0,1]: ^ 2
  }
  return row16_sum(st.l);
}

// Store a finished piece's normalised output: dimension j * DPL + lane / LPD of each load j.
template <int DT, int D>
__device__ __forceinline__ void v_store(const VState<DT, D>& st, float inv, void* out,
                                        int64_t base, bool out_f32) {
  using C = VCfg<DT, D>;
  const int lane = lane_id();
  if (lane % C::LPD == 0) {
#pragma unroll
    for (int j = 0; j < C::NV; ++j)
      store_out<DT>(out, base + j * C::DPL + lane / C::LPD, st.acc[j] * inv, out_f32);
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

// A piece of a split segment: publish it, or (if it is the segment's last arrival) merge
// every piece and write the output.  Lanes of a dimension row hold the same full sum after
// v_finish, so each lane reads and merges its own dimensions.
template <int DT, int D>
__device__ void v_split_finish(const DecodeArgs& a, VState<DT, D>& st, float l,
                               const SplitSeg& sg, int64_t self, int32_t* cnt, int seen,
                               int64_t ob) {
  using C = VCfg<DT, D>;
  const int lane = lane_id();
  const CohBuf bo = coh_buf(a.part_o), bm = coh_buf(a.part_m), bl = coh_buf(a.part_l);
  const int dim0 = lane / C::LPD;  // dimension j * DPL + dim0 of load j
  // this piece's partial as published: normalised output, max (natural log), sum
  const float inv = 1.f / l;
  const float mine_m = st.m * 0.69314718055994531f;
  float mine_o[C::NV];
#pragma unroll
  for (int j = 0; j < C::NV; ++j) mine_o[j] = st.acc[j] * inv;
  const bool last = split_arrive(cnt, (int)(sg.k1 - sg.k0), seen, [&] {
    const int64_t slot = piece_slot(sg, self);
    if (lane % C::LPD == 0) {
#pragma unroll
      for (int j = 0; j < C::NV; ++j) coh_store(bo, slot * D + j * C::DPL + dim0, mine_o[j]);
    }
    if (lane == 0) {
      coh_store(bm, slot, mine_m);
      coh_store(bl, slot, l);
    }
  });
  if (!last) return;
  float L, U[C::NV];
  merge_ordered<C::NV, 4>(L, U, sg.k0, sg.k1,
                          [&](int64_t k, float& m, float& lk, float (&ov)[C::NV]) {
    if (k == self) {
      m = mine_m;
      lk = l;
#pragma unroll
      for (int j = 0; j < C::NV; ++j) ov[j] = mine_o[j];
      return;
    }
    const int64_t slot = piece_slot(sg, k);
    m = coh_load(bm, slot);
    lk = coh_load(bl, slot);
#pragma unroll
    for (int j = 0; j < C::NV; ++j) ov[j] = coh_load(bo, slot * D + j * C::DPL + dim0);
  });
#pragma unroll
  for (int j = 0; j < C::NV; ++j) st.acc[j] = U[j];
  v_store<DT, D>(st, 1.f / L, a.out, ob, a.out_f32);
  counter_reset(cnt);
}

template <int DT, int D, int MODE>
__global__ __launch_bounds__(kWG) void valu_decode_kernel(DecodeArgs a) {
  // LDS: one 16-float weight slot per wave (first, for 16-byte alignment), then the plan
  // (S + 1 ints) and the scan buffer (kWG ints)
  extern __shared__ __align__(16) int32_t lds[];
  const int S = a.num_seqs;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  float* pw = reinterpret_cast<float*>(lds) + 16 * wave;
  int32_t* base = lds + 16 * kWavesPerWG;
  int32_t* tmp = base + S + 1;
  const int segs = a.num_q_heads;
  const int64_t W = (int64_t)gridDim.x * kWavesPerWG;
  const int64_t w = (int64_t)blockIdx.x * kWavesPerWG + wave;

  if constexpr (MODE == MODE_EVEN) {
    PlanIn pin{a.context_lens, a.qsl, S, kValuUnit, a.seg_extra};
    build_plan(base, tmp, pin);
    zero_empty_rows<DT>(pin, a.out, a.num_q_heads, D, w, W, a.out_f32);
    // units: (sequence, group of kWavesPerWG heads, tile); wave i runs head i of each group
    const int groups = (a.num_q_heads + kWavesPerWG - 1) / kWavesPerWG;
    const Part part = make_part((int64_t)base[S] * groups, gridDim.x);
    even_split_drive(part, [&](int64_t o, int64_t lo, int64_t hi) {
      for (int64_t i = lo; i < hi;) {
        const int s = find_seq(base, S, i, groups);
        const int seglen = base[s + 1] - base[s];
        const int nt = seglen - a.seg_extra;  // real tiles; the rest only balance the split
        const int64_t sbase = (int64_t)base[s] * groups;
        const int grp = (int)((i - sbase) / seglen);
        const int64_t seg0 = sbase + (int64_t)grp * seglen;
        const int64_t pe = min(hi, seg0 + seglen);
        const int h = grp * kWavesPerWG + wave;  // this wave's head
        const int t0 = (int)(i - seg0), t1 = (int)min(pe - seg0, (int64_t)nt);
        if (h < a.num_q_heads && t0 < nt) {
          const int ctx = a.context_lens[s];
          const int row = a.qsl ? a.qsl[s] : s;
          const int64_t ob = ((int64_t)row * a.num_q_heads + h) * D;
          const bool whole = t0 == 0 && t1 == nt;
          SplitSeg sg{};
          int32_t* cnt = nullptr;
          int seen = 0;
          if (!whole) {
            sg = split_seg(part, seg0, seg0 + nt - 1, wave);
            cnt = a.counters + kWavesPerWG * sg.k0 + wave;
            seen = counter_peek(cnt);  // consumed after the tiles
          }
          VState<DT, D> st;
          valu_attend<DT, D>(a, s, h, t0, t1, ctx, st, pw);
          const float l = v_finish<DT, D>(st);
          if (whole) {
            v_store<DT, D>(st, 1.f / l, a.out, ob, a.out_f32);
          } else {
            v_split_finish<DT, D>(a, st, l, sg, o, cnt, seen, ob);
          }
        }
        i = pe;
      }
    });
  } else {
    // fixed partitions; rows are sequences (no query_start_loc in this mode)
    const int PU = a.partition_units;  // tiles per partition
    const int P = a.max_partitions;
    PlanIn pin{a.context_lens, nullptr, S, PU * kBlock, 0};
    build_plan(base, tmp, pin);
    // partitions past the context: max_logits = -inf, exp_sums = 0
    const int64_t nent = (int64_t)S * a.num_q_heads * P;
    for (int64_t e = (int64_t)blockIdx.x * kWG + threadIdx.x; e < nent; e += (int64_t)gridDim.x * kWG) {
      const int p = (int)(e % P);
      const int s = (int)(e / ((int64_t)P * a.num_q_heads));
      if (p >= base[s + 1] - base[s]) {
        a.part_m[e] = -INFINITY;
        a.part_l[e] = 0.f;
      }
    }
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
      VState<DT, D> st;
      valu_attend<DT, D>(a, s, h, t0, t1, ctx, st, pw);
      const float l = v_finish<DT, D>(st);
      const float inv = 1.f / l;
      const int64_t e = ((int64_t)s * a.num_q_heads + h) * P + p;
      v_store_f32<DT, D>(st, inv, a.part_o + e * D);
      if (lane == 0) {
        a.part_m[e] = st.m * 0.69314718055994531f;
        a.part_l[e] = l;
      }
    }
  }
}

static size_t valu_lds_bytes(int num_seqs) {
  return (size_t)(num_seqs + 1 + kWG) * sizeof(int32_t) + kWavesPerWG * 16 * sizeof(float);
}

template <int DT, int MODE>
static hipError_t launch_d(const DecodeArgs& a, int grid, hipStream_t st) {
  const size_t lds = valu_lds_bytes(a.num_seqs);
  if (a.head_dim == 64)
    hipLaunchKernelGGL((valu_decode_kernel<DT, 64, MODE>), dim3(grid), dim3(kWG), lds, st, a);
  else
    hipLaunchKernelGGL((valu_decode_kernel<DT, 128, MODE>), dim3(grid), dim3(kWG), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_valu_decode(int dt, int mode, const DecodeArgs& a, int grid, hipStream_t st) {
  if (mode == MODE_EVEN) {
    if (dt == DT_F32) return launch_d<DT_F32, MODE_EVEN>(a, grid, st);
    if (dt == DT_F16) return launch_d<DT_F16, MODE_EVEN>(a, grid, st);
    return launch_d<DT_BF16, MODE_EVEN>(a, grid, st);
  }
  if (dt == DT_F32) return launch_d<DT_F32, MODE_PARTITION>(a, grid, st);
  if (dt == DT_F16) return launch_d<DT_F16, MODE_PARTITION>(a, grid, st);
  return launch_d<DT_BF16, MODE_PARTITION>(a, grid, st);
}

template <int DT, int MODE>
static int occ(int head_dim, int lds) {
  int n = 0;
  hipError_t e;
  if (head_dim == 64)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, valu_decode_kernel<DT, 64, MODE>, kWG, lds);
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, valu_decode_kernel<DT, 128, MODE>, kWG, lds);
  return e == hipSuccess && n > 0 ? n : 1;
}

int valu_decode_max_blocks_per_cu(int dt, int head_dim, int mode, int lds_bytes) {
  const int lds = lds_bytes + kWavesPerWG * 16 * (int)sizeof(float);
  if (mode == MODE_EVEN) {
    if (dt == DT_F32) return occ<DT_F32, MODE_EVEN>(head_dim, lds);
    if (dt == DT_F16) return occ<DT_F16, MODE_EVEN>(head_dim, lds);
    return occ<DT_BF16, MODE_EVEN>(head_dim, lds);
  }
  if (dt == DT_F32) return occ<DT_F32, MODE_PARTITION>(head_dim, lds);
  if (dt == DT_F16) return occ<DT_F16, MODE_PARTITION>(head_dim, lds);
  return occ<DT_BF16, MODE_PARTITION>(head_dim, lds);
}

}  // namespace pa
