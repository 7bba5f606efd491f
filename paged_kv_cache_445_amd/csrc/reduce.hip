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

// Merge for pa_decode's even split.  For every decode sequence s and segment g: if the
// segment's units all fell inside one wavefront's share, that wave already wrote the
// output; otherwise each wave w0..w1 touching it left one partial in slot
// (w, first piece ? 0 : 1) and this kernel merges them.  Decode rows with no key get 0.
template <int DT>
__global__ __launch_bounds__(kWG) void even_reduce_kernel(EvenReduceArgs a) {
  extern __shared__ int32_t lds[];
  int32_t* base = lds;
  int32_t* tmp = lds + a.num_seqs + 1;
  const int S = a.num_seqs;
  PlanIn pin{a.context_lens, a.qsl, S, a.unit_tokens};
  build_plan(base, tmp, pin);
  const int64_t T = (int64_t)base[S] * a.segs;
  const int64_t W = a.num_waves;
  const int hp = a.heads_per_seg, D = a.head_dim;
  const int64_t items = (int64_t)S * a.segs;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int s = (int)(it / a.segs), g = (int)(it % a.segs);
    const int rows = a.qsl ? a.qsl[s + 1] - a.qsl[s] : 1;
    if (rows != 1) continue;  // multi-row sequences are written by the chunk kernel
    const int row = a.qsl ? a.qsl[s] : s;
    const int nu = base[s + 1] - base[s];
    const int64_t ob = ((int64_t)row * a.num_q_heads + (int64_t)g * hp) * D;
    if (nu == 0) {  // no visible key
      for (int e = threadIdx.x; e < hp * D; e += kWG) store_out<DT>(a.out, ob + e, 0.f, a.out_f32);
      continue;
    }
    const int64_t seg0 = (int64_t)base[s] * a.segs + (int64_t)g * nu;
    const int64_t seg1 = seg0 + nu - 1;
    // wave owning flattened unit i: largest w with floor(w T / W) <= i
    const int64_t w0 = ((seg0 + 1) * W - 1) / T;
    const int64_t w1 = ((seg1 + 1) * W - 1) / T;
    if (w0 == w1) continue;
    const bool w0_second = range_lo(T, w0, W) < seg0;
    // (when there are fewer units than waves, some waves own nothing and wrote no slot)
    for (int e = threadIdx.x; e < hp * D; e += kWG) {
      const int hh = e / D, d = e - hh * D;
      float M = -INFINITY;
      for (int64_t w = w0; w <= w1; ++w) {
        if (range_lo(T, w, W) == range_lo(T, w + 1, W)) continue;
        const int64_t slot = w * 2 + ((w == w0 && w0_second) ? 1 : 0);
        M = fmaxf(M, a.part_m[slot * hp + hh]);
      }
      float L = 0.f, acc = 0.f;
      for (int64_t w = w0; w <= w1; ++w) {
        if (range_lo(T, w, W) == range_lo(T, w + 1, W)) continue;
        const int64_t slot = w * 2 + ((w == w0 && w0_second) ? 1 : 0);
        const float wp = a.part_l[slot * hp + hh] * __expf(a.part_m[slot * hp + hh] - M);
        L += wp;
        acc += wp * a.part_o[(slot * hp + hh) * D + d];
      }
      store_out<DT>(a.out, ob + e, acc / L, a.out_f32);
    }
  }
}

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

hipError_t launch_even_reduce(int dt, const EvenReduceArgs& a, int grid, hipStream_t st) {
  const size_t lds = (size_t)(a.num_seqs + 1 + kWG) * sizeof(int32_t);
  if (grid <= 0) return hipSuccess;
  if (dt == DT_F32)
    hipLaunchKernelGGL(even_reduce_kernel<DT_F32>, dim3(grid), dim3(kWG), lds, st, a);
  else if (dt == DT_F16)
    hipLaunchKernelGGL(even_reduce_kernel<DT_F16>, dim3(grid), dim3(kWG), lds, st, a);
  else
    hipLaunchKernelGGL(even_reduce_kernel<DT_BF16>, dim3(grid), dim3(kWG), lds, st, a);
  return hipGetLastError();
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
