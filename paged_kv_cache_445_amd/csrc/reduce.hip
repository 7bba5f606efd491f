// reduce.hip — log-sum-exp merge of split-context partials.
//
// Partials of one query row / head over disjoint key ranges p carry their softmax-normalised
// output o_p, max score m_p and sum l_p = sum exp(score - m_p).  With M = max_p m_p and
// w_p = l_p * exp(m_p - M), the full result is sum_p w_p o_p / sum_p w_p: the softmax of
// "vLLM 深度拆解：当 KV Cache 学会「分页」" §2.2 evaluated over the union of the ranges.
#include <math.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// pa_decode_reduce: one wavefront per (row, head).  Lane p holds partition p's weight (64
// partitions at a time), so the max and the sum of weights are wave reductions; the outputs
// (lanes over the head dimension) then accumulate only the partitions with a key, four at a
// time with their loads in flight together.  Partitions without a key (exp_sums 0) are never
// read (their tmp_out entries are not written).
template <int DT, int D>
__global__ __launch_bounds__(kWG) void part_reduce_kernel(PartReduceArgs a) {
  constexpr int ND = D / kWave;  // output dimensions per lane
  const int lane = lane_id();
  const int64_t item = (int64_t)blockIdx.x * kWavesPerWG + threadIdx.x / kWave;
  if (item >= a.num_items) return;
  const int P = a.max_partitions;
  const float* m = a.max_logits + item * P;
  const float* l = a.exp_sums + item * P;
  const float* po = a.tmp_out + item * P * D + lane;
  float M = -INFINITY;
  for (int p = lane; p < P; p += kWave)
    if (l[p] > 0.f) M = fmaxf(M, m[p]);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) M = fmaxf(M, shfl_xor(M, d));
  float L = 0.f, acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = 0.f;
  if (M != -INFINITY) {
    for (int p0 = 0; p0 < P; p0 += kWave) {
      const int p = p0 + lane;
      const float lp = p < P ? l[p] : 0.f;
      const float w = lp > 0.f ? lp * __expf(m[p] - M) : 0.f;
      L += w;
      uint64_t live = __builtin_amdgcn_ballot_w64(lp > 0.f);
      while (live) {
        int q[4];
        float wq[4];
        float o[4][ND];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          q[b] = live ? __builtin_ctzll(live) : -1;
          live &= live ? live - 1 : 0;
          wq[b] = q[b] >= 0 ? readlane(w, q[b]) : 0.f;
#pragma unroll
          for (int i = 0; i < ND; ++i)
            o[b][i] = q[b] >= 0 ? po[(int64_t)(p0 + q[b]) * D + kWave * i] : 0.f;
        }
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int i = 0; i < ND; ++i) acc[i] = fmaf(wq[b], o[b][i], acc[i]);
      }
    }
  }
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) L += shfl_xor(L, d);
#pragma unroll
  for (int i = 0; i < ND; ++i)
    store_out<DT>(a.out, item * D + lane + kWave * i, L > 0.f ? acc[i] / L : 0.f, a.out_f32);
}

hipError_t launch_part_reduce(int dt, const PartReduceArgs& a, hipStream_t st) {
  const int64_t grid = (a.num_items + kWavesPerWG - 1) / kWavesPerWG;
  if (grid == 0) return hipSuccess;
  auto go = [&](auto dt_c) {
    constexpr int T = decltype(dt_c)::value;
    if (a.head_dim == 64)
      hipLaunchKernelGGL((part_reduce_kernel<T, 64>), dim3((unsigned)grid), dim3(kWG), 0, st, a);
    else
      hipLaunchKernelGGL((part_reduce_kernel<T, 128>), dim3((unsigned)grid), dim3(kWG), 0, st, a);
  };
  if (dt == DT_F32)
    go(std::integral_constant<int, DT_F32>{});
  else if (dt == DT_F16)
    go(std::integral_constant<int, DT_F16>{});
  else
    go(std::integral_constant<int, DT_BF16>{});
  return hipGetLastError();
}

}  // namespace pa
