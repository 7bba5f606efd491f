// chunk.hip — multi-row (chunked-prefill) attention over the paged cache.
//
// "vLLM 架构源码解析 第1篇" §1.1 runs a long prompt as 512-token chunks in the same step as
// other requests' decode rows, and §3.3.2 marks each request's rows with query_start_loc.
// A sequence s with n > 1 rows has its context_lens entry counting those rows (they were
// written by reshape_and_cache first, §3.3.3); row j sits at position ctx - n + j and attends
// keys [0, ctx - n + j] (causal).  Decode rows (n = 1) are left to the decode kernels.
//
// Work item = (sequence, KV head g, block of 16 query columns), a column being one (row, head)
// pair: 16 / G consecutive rows x the G query heads of g.  A wavefront streams the item's
// keys in 32-token units through the matrix-core unit of pa_mfma.h with a per-column
// causal limit.
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma.h"

namespace pa {

struct ChunkPlanIn {
  const int32_t* qsl;
  int32_t num_seqs;
  int32_t rows_per_block;
};

// column blocks per sequence: ceil(n / rows_per_block) for multi-row sequences, else 0
__device__ inline void build_chunk_plan(int32_t* base, int32_t* tmp, const ChunkPlanIn& p) {
  const int t = threadIdx.x;
  const int S = p.num_seqs;
  const int per = (S + kWG - 1) / kWG;
  const int s0 = t * per, s1 = min(S, s0 + per);
  int32_t sum = 0;
  for (int s = s0; s < s1; ++s) {
    const int32_t n = p.qsl[s + 1] - p.qsl[s];
    const int32_t u = n > 1 ? (n + p.rows_per_block - 1) / p.rows_per_block : 0;
    base[s] = u;
    sum += u;
  }
  tmp[t] = sum;
  __syncthreads();
  for (int off = 1; off < kWG; off <<= 1) {
    const int32_t v = t >= off ? tmp[t - off] : 0;
    __syncthreads();
    tmp[t] += v;
    __syncthreads();
  }
  int32_t run = tmp[t] - sum;
  for (int s = s0; s < s1; ++s) {
    const int32_t u = base[s];
    base[s] = run;
    run += u;
  }
  if (t == kWG - 1) base[S] = tmp[kWG - 1];
  __syncthreads();
}

template <int DT, int D>
__device__ void chunk_item(const DecodeArgs& a, int s, int g, int cb) {
  using C = MfmaCfg<DT, D>;
  using T = op8_t<DT>;
  const int lane = lane_id();
  const int r = lane >> 4, n = lane & 15;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int RB = kWave / 4 / G;  // rows per 16-column block
  const int q0 = a.qsl[s], nrows = a.qsl[s + 1] - q0;
  const int ctx = a.context_lens[s];
  const int j0 = cb * RB;
  const int jend = min(nrows, j0 + RB);
  const int first_pos = ctx - nrows + j0;    // smallest last-visible key of the block
  const int last_pos = ctx - nrows + jend - 1;
  // this lane's query column
  const int jc = j0 + n / G, hc = n % G;
  const bool col_ok = jc < jend;
  const int pos_c = col_ok ? ctx - nrows + jc : -1;

  T qb[C::NKK];
  {
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     ((int64_t)(q0 + jc) * a.num_q_heads + (int64_t)g * G + hc) * D * C::E;
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
      const uint4 v = col_ok ? ld16(qp + (4 * kk + r) * 16) : make_uint4(0, 0, 0, 0);
      qb[kk] = __builtin_bit_cast(T, v);
    }
  }
  MfmaLaneOffsets<DT, D> o;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int t = 8 * (n >> 2) + 4 * b + (n & 3);
    o.kt[b] = t >> 4;
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) o.k[b][kk] = ((4 * kk + r) * 16 + (t & 15)) * 16;
  }
  o.vt = r >> 1;
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) o.v[j] = ((16 * j + n) * 16 + 8 * (r & 1)) * C::E;

  const int64_t blk_stride = (int64_t)a.num_kv_heads * C::TILE;
  const char* kc = reinterpret_cast<const char*>(a.k_cache) + (int64_t)g * C::TILE;
  const char* vc = reinterpret_cast<const char*>(a.v_cache) + (int64_t)g * C::TILE;
  const int32_t* bt_row = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int nkeys = last_pos + 1;            // keys any column of the block may see
  const int nblk = (nkeys + kBlock - 1) / kBlock;
  const int nu = (nkeys + kMfmaUnit - 1) / kMfmaUnit;

  MfmaState<DT, D> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) st.acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  constexpr int WU = kWave / 2;
  for (int wb = 0; wb < nu; wb += WU) {
    const int we = min(nu, wb + WU);
    const int e0 = 2 * wb;
    const int btv = (e0 + lane < min(nblk, 2 * we)) ? bt_row[e0 + lane] : 0;
    uint4 kb[C::DEPTH][2][C::NKK], vb[C::DEPTH][C::NJ];
    auto issue = [&](int slot, int u) {
      const int ia = 2 * (u - wb);
      const int64_t ba = readlane(btv, ia);
      const int64_t bb = (2 * u + 1 < nblk) ? (int64_t)readlane(btv, ia + 1) : ba;
      mfma_load<DT, D>(kb[slot], vb[slot], kc + ba * blk_stride, kc + bb * blk_stride,
                       vc + ba * blk_stride, vc + bb * blk_stride, o);
    };
#pragma unroll
    for (int b = 0; b < C::DEPTH - 1; ++b)
      if (wb + b < we) issue(b, wb + b);
    for (int u = wb; u < we; u += C::DEPTH) {
#pragma unroll
      for (int b = 0; b < C::DEPTH; ++b) {
        const int ut = u + b;
        if (ut < we) {
          const int un = ut + C::DEPTH - 1;
          if (un < we) issue((b + C::DEPTH - 1) % C::DEPTH, un);
          const int t0 = ut * kMfmaUnit;
          if (t0 + kMfmaUnit - 1 <= first_pos && jend - j0 == RB)
            mfma_unit<DT, D, false, true>(st, kb[b], vb[b], qb, a.scale_log2, kMfmaUnit - 1,
                                          kMfmaUnit);
          else
            mfma_unit<DT, D, true, true>(st, kb[b], vb[b], qb, a.scale_log2, pos_c - t0,
                                         nkeys - t0);
        }
      }
    }
  }

  // emit: output column c = 4r + i of the P.V tile is (row j0 + c / G, head c % G)
  const float ltot = cross_rows_sum(st.l);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 4 * r + i;
    const float inv_c = shfl(inv, c);
    const int jr = j0 + c / G, hr = c % G;
    if (jr < jend) {
      const int64_t ob = ((int64_t)(q0 + jr) * a.num_q_heads + (int64_t)g * G + hr) * D;
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) store_out<DT>(a.out, ob + 16 * j + n, st.acc[j][i] * inv_c, a.out_f32);
    }
  }
}

template <int DT, int D>
__global__ __launch_bounds__(kWG) void chunk_kernel(DecodeArgs a) {
  extern __shared__ int32_t lds[];
  int32_t* base = lds;
  int32_t* tmp = lds + a.num_seqs + 1;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int S = a.num_seqs;
  ChunkPlanIn pin{a.qsl, S, kWave / 4 / G};
  build_chunk_plan(base, tmp, pin);
  const int segs = a.num_kv_heads;
  const int64_t total = (int64_t)base[S] * segs;
  const int64_t W = (int64_t)gridDim.x * kWavesPerWG;
  const int64_t w = (int64_t)blockIdx.x * kWavesPerWG + threadIdx.x / kWave;
  for (int64_t i = w; i < total; i += W) {
    const int s = find_seq(base, S, i, segs);
    const int nb = base[s + 1] - base[s];
    const int64_t sbase = (int64_t)base[s] * segs;
    const int g = (int)((i - sbase) / nb);
    const int cb = (int)(i - sbase - (int64_t)g * nb);
    chunk_item<DT, D>(a, s, g, cb);
  }
}

hipError_t launch_chunk(int dt, const DecodeArgs& a, int grid, hipStream_t st) {
  const size_t lds = (size_t)(a.num_seqs + 1 + kWG) * sizeof(int32_t);
  if (grid <= 0) return hipSuccess;
  if (dt == DT_F16) {
    if (a.head_dim == 64)
      hipLaunchKernelGGL((chunk_kernel<DT_F16, 64>), dim3(grid), dim3(kWG), lds, st, a);
    else
      hipLaunchKernelGGL((chunk_kernel<DT_F16, 128>), dim3(grid), dim3(kWG), lds, st, a);
  } else {
    if (a.head_dim == 64)
      hipLaunchKernelGGL((chunk_kernel<DT_BF16, 64>), dim3(grid), dim3(kWG), lds, st, a);
    else
      hipLaunchKernelGGL((chunk_kernel<DT_BF16, 128>), dim3(grid), dim3(kWG), lds, st, a);
  }
  return hipGetLastError();
}

}  // namespace pa
