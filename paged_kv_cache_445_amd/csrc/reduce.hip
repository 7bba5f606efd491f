// reduce.hip — log-sum-exp merge of split-context partials.
//
// Partials of one query row / head over disjoint key ranges p carry their softmax-normalised
// output o_p, max score m_p and sum l_p = sum exp(score - m_p).  With M = max_p m_p and
// w_p = l_p * exp(m_p - M), the full result is sum_p w_p o_p / sum_p w_p: the softmax of
// "vLLM 深度拆解：当 KV Cache 学会「分页」" §2.2 evaluated over the union of the ranges.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// pa_decode_reduce: one wavefront per (row, head), lanes over the head dimension.
template <int DT>
__global__ __launch_bounds__(kWG) void part_reduce_kernel(PartReduceArgs a) {
  const int lane = lane_id();
  const int64_t item = (int64_t)blockIdx.x * kWavesPerWG + threadIdx.x / kWave;
  if (item >= a.num_items) return;
  const int P = a.max_partitions, D = a.head_dim;
  const float* m = a.max_logits + item * P;
  const float* l = a.exp_sums + item * P;
  float M = -INFINITY;
  for (int p = 0; p < P; ++p)
    if (l[p] > 0.f) M = fmaxf(M, m[p]);
  for (int d = lane; d < D; d += kWave) {
    float L = 0.f, acc = 0.f;
    if (M != -INFINITY) {
      for (int p = 0; p < P; ++p) {
        if (!(l[p] > 0.f)) continue;
        const float wp = l[p] * __expf(m[p] - M);
        L += wp;
        acc += wp * a.tmp_out[(item * P + p) * D + d];
      }
    }
    store_out<DT>(a.out, item * D + d, L > 0.f ? acc / L : 0.f, a.out_f32);
  }
}

hipError_t launch_part_reduce(int dt, const PartReduceArgs& a, hipStream_t st) {
  const int64_t grid = (a.num_items + kWavesPerWG - 1) / kWavesPerWG;
  if (grid == 0) return hipSuccess;
  if (dt == DT_F32)
    hipLaunchKernelGGL(part_reduce_kernel<DT_F32>, dim3((unsigned)grid), dim3(kWG), 0, st, a);
  else if (dt == DT_F16)
    hipLaunchKernelGGL(part_reduce_kernel<DT_F16>, dim3((unsigned)grid), dim3(kWG), 0, st, a);
  else
    hipLaunchKernelGGL(part_reduce_kernel<DT_BF16>, dim3((unsigned)grid), dim3(kWG), 0, st, a);
  return hipGetLastError();
}

}  // namespace pa
