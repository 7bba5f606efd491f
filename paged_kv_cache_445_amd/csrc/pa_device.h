// pa_device.h — device-side helpers shared by the gfx950 kernels of libpa.so.
//
// Pool layout (the ABI of include/pa.h): elem E bytes, X = 16 / E elements per 16-byte chunk,
//   K tile of (block, kv_head): [D / X chunks][16 tokens][X]   = 16 * D * E bytes
//   V tile of (block, kv_head): [D dims][16 tokens]            = 16 * D * E bytes
// Tiles of consecutive kv heads of one block are adjacent.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {

template <int DT>
struct DtInfo {
  static constexpr int bytes = DT == DT_F32 ? 4 : 2;
  static constexpr int x = 16 / bytes;  // elements per 16-byte chunk
};

typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf162_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---------------------------------------------------------------- 16-byte global loads

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t u) {
  return (float)__builtin_bit_cast(half2_t, u)[0];
}
__device__ __forceinline__ float f16_hi(uint32_t u) {
  return (float)__builtin_bit_cast(half2_t, u)[1];
}

// element k (0..7) of a 16-byte chunk of 16-bit values, widened to float
template <int DT>
__device__ __forceinline__ float elem16(const uint4& v, int k) {
  const uint32_t w = k < 2 ? v.x : k < 4 ? v.y : k < 6 ? v.z : v.w;
  if constexpr (DT == DT_BF16)
    return (k & 1) ? bf16_hi(w) : bf16_lo(w);
  else
    return (k & 1) ? f16_hi(w) : f16_lo(w);
}

// dot of two 16-byte chunks (8 x 16-bit or 4 x fp32), accumulated in fp32
template <int DT>
__device__ __forceinline__ float dot16(const uint4& a, const uint4& b, float acc) {
  if constexpr (DT == DT_F32) {
    acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
    acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
    acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
    acc = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
  } else if constexpr (DT == DT_F16) {
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a.x), __builtin_bit_cast(half2_t, b.x), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a.y), __builtin_bit_cast(half2_t, b.y), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a.z), __builtin_bit_cast(half2_t, b.z), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a.w), __builtin_bit_cast(half2_t, b.w), acc, false);
  } else {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a.x), __builtin_bit_cast(bf162_t, b.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a.y), __builtin_bit_cast(bf162_t, b.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a.z), __builtin_bit_cast(bf162_t, b.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a.w), __builtin_bit_cast(bf162_t, b.w), acc, false);
  }
  return acc;
}

// store one output element in the output dtype (round to nearest even for 16-bit)
template <int DT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v, bool out_f32) {
  if (out_f32 || DT == DT_F32) {
    reinterpret_cast<float*>(out)[idx] = v;
  } else if constexpr (DT == DT_F16) {
    reinterpret_cast<_Float16*>(out)[idx] = (_Float16)v;
  } else {
    reinterpret_cast<__bf16*>(out)[idx] = (__bf16)v;
  }
}

// ---------------------------------------------------------------- cross-lane reductions

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// max / sum over the 16 lanes of a DPP row; every lane of the row receives the result
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_mov<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_mov<0x140>(v));  // row_mirror
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return v;
}

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, kWave); }
__device__ __forceinline__ float shfl(float v, int src) { return __shfl(v, src, kWave); }

// sum over lanes {l, l^16, l^32, l^48}: the four DPP rows
__device__ __forceinline__ float cross_rows_sum(float v) {
  v += shfl_xor(v, 16);
  v += shfl_xor(v, 32);
  return v;
}
__device__ __forceinline__ float cross_rows_max(float v) {
  v = fmaxf(v, shfl_xor(v, 16));
  v = fmaxf(v, shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ int readlane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float readlane(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// ---------------------------------------------------------------- work plan
//
// The split kernels walk a flattened list of work units: for every decode sequence s
// (exactly one query row) and every segment index g in [0, segs), the units
// [0, units(s)) of that sequence, units(s) = ceil(ctx_s / unit_tokens).  Flattened index:
//   i = base[s] * segs + g * units(s) + u,     base[s] = sum_{s' < s} units(s').
// Each workgroup rebuilds base[] in LDS from context_lens (one coalesced read + a scan).

struct PlanIn {
  const int32_t* context_lens;
  const int32_t* qsl;  // NULL: one row per sequence
  int32_t num_seqs;
  int32_t unit_tokens;
};

__device__ __forceinline__ int32_t seq_units(const PlanIn& p, int s) {
  const int32_t rows = p.qsl ? p.qsl[s + 1] - p.qsl[s] : 1;
  if (rows != 1) return 0;  // multi-row sequences are not split-context work
  const int32_t ctx = p.context_lens[s];
  return ctx > 0 ? (ctx + p.unit_tokens - 1) / p.unit_tokens : 0;
}

// base[0..S] in LDS; `tmp` is kWG ints of LDS.  Must be called by all threads of the WG.
__device__ inline void build_plan(int32_t* base, int32_t* tmp, const PlanIn& p) {
  const int t = threadIdx.x;
  const int S = p.num_seqs;
  const int per = (S + kWG - 1) / kWG;
  const int s0 = t * per, s1 = min(S, s0 + per);
  int32_t sum = 0;
  for (int s = s0; s < s1; ++s) {
    const int32_t u = seq_units(p, s);
    base[s] = u;  // units for now, prefix below
    sum += u;
  }
  tmp[t] = sum;
  __syncthreads();
  // inclusive Hillis-Steele scan of the kWG partial sums
  for (int off = 1; off < kWG; off <<= 1) {
    const int32_t v = t >= off ? tmp[t - off] : 0;
    __syncthreads();
    tmp[t] += v;
    __syncthreads();
  }
  int32_t run = tmp[t] - sum;  // exclusive prefix of this thread's range
  for (int s = s0; s < s1; ++s) {
    const int32_t u = base[s];
    base[s] = run;
    run += u;
  }
  if (t == kWG - 1) base[S] = tmp[kWG - 1];
  __syncthreads();
}

// largest s in [0, S) with base[s] * segs <= i  (requires i < base[S] * segs)
__device__ __forceinline__ int find_seq(const int32_t* base, int S, int64_t i, int segs) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)base[mid] * segs <= i)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// even split of [0, total) over W waves: wave w owns [range_lo(w), range_lo(w+1))
__device__ __forceinline__ int64_t range_lo(int64_t total, int64_t w, int64_t W) {
  return (total * w) / W;
}

}  // namespace pa
