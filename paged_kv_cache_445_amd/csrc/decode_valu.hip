// decode_valu.hip — paged-attention decode on the vector ALUs, one query head per wavefront
// work segment (multi-head attention; also the generic path for fp32).
//
// The method ("vLLM 深度拆解：当 KV Cache 学会「分页」" §3.3 and §6.2): for every block of the
// sequence, look up its physical id in the block table, read the block's K and V, score
// each token with scale * q . k while the token index is below context_len, and finish
// with softmax(scores) . V (§2.2).  Here the softmax is streamed (running max m and sum l,
// rescaled when m grows), so each K/V tile is read exactly once.
//
// Wavefront mapping of one 16-token tile (E-byte elements, X = 16 / E, D = head_dim):
//   K: load i (i < D/X/4): lane reads 16-byte chunk c = 4i + lane/16 of token lane%16, so
//      one load instruction covers 1 KiB of the tile contiguously.  The lane's partial
//      dot product over its chunks is summed across the four DPP rows, leaving the full
//      score of token lane%16 in every row.
//   V: load j (j < D/64 * 16/X): lane reads X consecutive tokens (group j / (D/64)) of
//      dimension 64 * (j % (D/64)) + lane.  The token group is uniform per instruction, so
//      the weights come from readlane of the score lanes (scalar operands), and each lane
//      accumulates the output dimensions it owns with no cross-lane reduction.
//   Block-table entries for up to 64 tiles sit one per lane and are broadcast by readlane.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

template <int DT, int D>
struct ValuCfg {
  static constexpr int E = DtInfo<DT>::bytes;
  static constexpr int X = DtInfo<DT>::x;
  static constexpr int NCH = D / X;  // 16-byte K chunks per token
  static constexpr int NK = NCH / 4; // K loads per lane per tile
  static constexpr int NVD = D / 64; // output dimensions owned by a lane
  static constexpr int TG = 16 / X;  // X-token groups in one V dimension row
  static constexpr int NV = NVD * TG;// V loads per lane per tile
  static constexpr int64_t TILE = 16LL * D * E;
  static constexpr int DEPTH = 2;    // tiles in flight per wavefront
};

template <int DT, int D>
using ValuK = uint4[ValuCfg<DT, D>::NK];
template <int DT, int D>
using ValuV = uint4[ValuCfg<DT, D>::NV];
template <int DT, int D>
using ValuKOff = int[ValuCfg<DT, D>::NK];
template <int DT, int D>
using ValuVOff = int[ValuCfg<DT, D>::NV];

template <int DT, int D>
struct ValuState {
  float m;                          // running max (base-2 domain)
  float l;                          // this lane's share of the running sum (token lane%16)
  float acc[ValuCfg<DT, D>::NVD];   // unnormalised output, dims 64*jd + lane
};

template <int DT, int D>
__device__ __forceinline__ void valu_load(ValuK<DT, D>& kb, ValuV<DT, D>& vb, const char* kblk,
                                          const char* vblk, const ValuKOff<DT, D>& koff,
                                          const ValuVOff<DT, D>& voff) {
  using C = ValuCfg<DT, D>;
#pragma unroll
  for (int i = 0; i < C::NK; ++i) kb[i] = ld16(kblk + koff[i]);
#pragma unroll
  for (int j = 0; j < C::NV; ++j) vb[j] = ld16(vblk + voff[j]);
}

template <int DT, int D, bool MASK>
__device__ __forceinline__ void valu_tile(ValuState<DT, D>& st, const ValuK<DT, D>& kb,
                                          const ValuV<DT, D>& vb, const ValuK<DT, D>& qv,
                                          float scale_log2,
                                          int valid /* tokens of this tile below context_len */) {
  using C = ValuCfg<DT, D>;
  const int lane = lane_id();
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < C::NK; ++i) part = dot16<DT>(kb[i], qv[i], part);
  part = cross_rows_sum(part);
  float sc = part * scale_log2;
  if (MASK && (lane & 15) >= valid) sc = -INFINITY;
  const float mnew = fmaxf(st.m, row16_max(sc));
  const float alpha = __builtin_amdgcn_exp2f(st.m - mnew);
  const float p = __builtin_amdgcn_exp2f(sc - mnew);
  st.l = st.l * alpha + p;
  st.m = mnew;
#pragma unroll
  for (int jd = 0; jd < C::NVD; ++jd) st.acc[jd] *= alpha;
#pragma unroll
  for (int j = 0; j < C::NV; ++j) {
    const int tg = j / C::NVD, jd = j % C::NVD;
#pragma unroll
    for (int k = 0; k < C::X; ++k) {
      const int tok = tg * C::X + k;
      if (MASK && tok >= valid) continue;  // uniform: never touch a V element past the context
      const float pk = readlane(p, tok);
      float v;
      if constexpr (DT == DT_F32) {
        const uint32_t w = k == 0 ? vb[j].x : k == 1 ? vb[j].y : k == 2 ? vb[j].z : vb[j].w;
        v = __uint_as_float(w);
      } else {
        v = elem16<DT>(vb[j], k);
      }
      st.acc[jd] = fmaf(pk, v, st.acc[jd]);
    }
  }
}

// Attention of query head h of sequence s over its tiles [t0, t1).
template <int DT, int D>
__device__ void valu_attend(const DecodeArgs& a, int s, int h, int t0, int t1, int ctx,
                            ValuState<DT, D>& st) {
  using C = ValuCfg<DT, D>;
  const int lane = lane_id();
  const int G = a.num_q_heads / a.num_kv_heads;
  const int kvh = h / G;
  const int row = a.qsl ? a.qsl[s] : s;
  const char* qp = reinterpret_cast<const char*>(a.q) + ((int64_t)row * a.num_q_heads + h) * D * C::E;
  uint4 qv[C::NK];
  int koff[C::NK], voff[C::NV];
#pragma unroll
  for (int i = 0; i < C::NK; ++i) {
    const int c = 4 * i + (lane >> 4);
    qv[i] = ld16(qp + c * 16);
    koff[i] = (c * 16 + (lane & 15)) * 16;
  }
#pragma unroll
  for (int j = 0; j < C::NV; ++j)
    voff[j] = ((64 * (j % C::NVD) + lane) * 16 + (j / C::NVD) * C::X) * C::E;

  const int64_t blk_stride = (int64_t)a.num_kv_heads * C::TILE;
  const char* kc = reinterpret_cast<const char*>(a.k_cache) + (int64_t)kvh * C::TILE;
  const char* vc = reinterpret_cast<const char*>(a.v_cache) + (int64_t)kvh * C::TILE;
  const int32_t* bt_row = a.block_tables + (int64_t)s * a.max_blocks_per_seq;

  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int jd = 0; jd < C::NVD; ++jd) st.acc[jd] = 0.f;

  for (int wb = t0; wb < t1; wb += kWave) {
    const int we = min(t1, wb + kWave);
    const int btv = (wb + lane < we) ? bt_row[wb + lane] : 0;
    uint4 kb[C::DEPTH][C::NK], vb[C::DEPTH][C::NV];
#pragma unroll
    for (int b = 0; b < C::DEPTH - 1; ++b) {
      if (wb + b < we) {
        const int64_t blk = readlane(btv, b);
        valu_load<DT, D>(kb[b], vb[b], kc + blk * blk_stride, vc + blk * blk_stride, koff, voff);
      }
    }
    for (int j = wb; j < we; j += C::DEPTH) {
#pragma unroll
      for (int b = 0; b < C::DEPTH; ++b) {
        const int jt = j + b;
        if (jt < we) {
          const int jn = jt + C::DEPTH - 1;
          if (jn < we) {
            const int64_t blk = readlane(btv, jn - wb);
            valu_load<DT, D>(kb[(b + C::DEPTH - 1) % C::DEPTH], vb[(b + C::DEPTH - 1) % C::DEPTH],
                             kc + blk * blk_stride, vc + blk * blk_stride, koff, voff);
          }
          const int valid = ctx - jt * kBlock;
          if (valid >= kBlock)
            valu_tile<DT, D, false>(st, kb[b], vb[b], qv, a.scale_log2, kBlock);
          else
            valu_tile<DT, D, true>(st, kb[b], vb[b], qv, a.scale_log2, valid);
        }
      }
    }
  }
}

template <int DT, int D, int MODE>
__global__ __launch_bounds__(kWG) void valu_decode_kernel(DecodeArgs a) {
  using C = ValuCfg<DT, D>;
  extern __shared__ int32_t lds[];
  int32_t* base = lds;
  int32_t* tmp = lds + a.num_seqs + 1;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int segs = a.num_q_heads;
  const int S = a.num_seqs;
  const int64_t W = (int64_t)gridDim.x * kWavesPerWG;
  const int64_t w = (int64_t)blockIdx.x * kWavesPerWG + wave;

  if constexpr (MODE == MODE_EVEN) {
    PlanIn pin{a.context_lens, a.qsl, S, kValuUnit};
    build_plan(base, tmp, pin);
    const int64_t total = (int64_t)base[S] * segs;
    const int64_t lo = range_lo(total, w, W), hi = range_lo(total, w + 1, W);
    for (int64_t i = lo; i < hi;) {
      const int s = find_seq(base, S, i, segs);
      const int nt = base[s + 1] - base[s];
      const int64_t sbase = (int64_t)base[s] * segs;
      const int h = (int)((i - sbase) / nt);
      const int64_t seg0 = sbase + (int64_t)h * nt;
      const int64_t pe = min(hi, seg0 + nt);
      const int t0 = (int)(i - seg0), t1 = (int)(pe - seg0);
      const int ctx = a.context_lens[s];
      ValuState<DT, D> st;
      valu_attend<DT, D>(a, s, h, t0, t1, ctx, st);
      const float l = row16_sum(st.l);
      const float inv = 1.f / l;
      if (t0 == 0 && t1 == nt) {
        const int row = a.qsl ? a.qsl[s] : s;
        const int64_t ob = ((int64_t)row * a.num_q_heads + h) * D;
#pragma unroll
        for (int jd = 0; jd < C::NVD; ++jd)
          store_out<DT>(a.out, ob + 64 * jd + lane, st.acc[jd] * inv, a.out_f32);
      } else {
        const int64_t slot = w * 2 + (i == lo ? 0 : 1);
#pragma unroll
        for (int jd = 0; jd < C::NVD; ++jd) a.part_o[slot * D + 64 * jd + lane] = st.acc[jd] * inv;
        if (lane == 0) {
          a.part_m[slot] = st.m * 0.69314718055994531f;  // natural-log domain
          a.part_l[slot] = l;
        }
      }
      i = pe;
    }
  } else {
    // fixed partitions; rows are sequences (no query_start_loc in this mode)
    const int PU = a.partition_units;  // tiles per partition
    const int P = a.max_partitions;
    PlanIn pin{a.context_lens, nullptr, S, PU * kBlock};
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
      ValuState<DT, D> st;
      valu_attend<DT, D>(a, s, h, t0, t1, ctx, st);
      const float l = row16_sum(st.l);
      const float inv = 1.f / l;
      const int64_t e = ((int64_t)s * a.num_q_heads + h) * P + p;
#pragma unroll
      for (int jd = 0; jd < C::NVD; ++jd) a.part_o[e * D + 64 * jd + lane] = st.acc[jd] * inv;
      if (lane == 0) {
        a.part_m[e] = st.m * 0.69314718055994531f;
        a.part_l[e] = l;
      }
    }
  }
}

template <int DT, int MODE>
static hipError_t launch_d(const DecodeArgs& a, int grid, hipStream_t st) {
  const size_t lds = (size_t)(a.num_seqs + 1 + kWG) * sizeof(int32_t);
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
  if (mode == MODE_EVEN) {
    if (dt == DT_F32) return occ<DT_F32, MODE_EVEN>(head_dim, lds_bytes);
    if (dt == DT_F16) return occ<DT_F16, MODE_EVEN>(head_dim, lds_bytes);
    return occ<DT_BF16, MODE_EVEN>(head_dim, lds_bytes);
  }
  if (dt == DT_F32) return occ<DT_F32, MODE_PARTITION>(head_dim, lds_bytes);
  if (dt == DT_F16) return occ<DT_F16, MODE_PARTITION>(head_dim, lds_bytes);
  return occ<DT_BF16, MODE_PARTITION>(head_dim, lds_bytes);
}

}  // namespace pa
