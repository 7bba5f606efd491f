// reshape.hip — the paged KV-cache write ("vLLM 架构源码解析 第1篇" §3.3.3: reshape_and_cache
// scatters this step's K and V into the block pool at slot_mapping before attention; the
// block / offset split of a slot is §4.2's `//` and `%` by the block size).  The pools are
// addressed in tiles of T tokens: T = 8 for 8-token blocks, else 16 (a block of 32 or 64
// tokens is 2 or 4 consecutive 16-token tiles, so slot / 16 names a tile for every block
// size from 16 up).
//
// One thread per 16-byte K chunk, then one thread per V element.  Consecutive threads read
// consecutive input bytes (coalesced loads); K chunk stores are 16-byte stores into the
// token's row of each 256-byte chunk plane; V stores are single elements into the token's
// column of each dimension row.  The copy is a bit copy: no conversion.
//
// A single token touches many partly written lines of its tiles (16 K chunks and D V
// elements per head).  The stores are non-temporal: left dirty in L2, those lines were
// written back while the next decode streamed the pools and cost it ~5% on the LLaMA-7B
// batch; streamed stores leave nothing behind.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

template <int DT>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(ReshapeArgs a) {
  constexpr int E = DtInfo<DT>::bytes;
  constexpr int X = DtInfo<DT>::x;
  const int H = a.num_kv_heads, D = a.head_dim, NCH = D / X;
  const int64_t nk = a.num_tokens * H * NCH;
  const int64_t nv = a.num_tokens * H * D;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid < nk) {
    const int64_t t = tid / (H * NCH);
    const int rem = (int)(tid - t * H * NCH);
    const int g = rem / NCH, c = rem - g * NCH;
    const int64_t slot = a.slot_mapping[t];
    if (slot < 0) return;  // padding token
    const int64_t blk = slot >> a.tile_shift;  // tile of T = 2^tile_shift tokens
    const int off = (int)(slot & ((1 << a.tile_shift) - 1));
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
    const u32x4 v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(a.key) +
                                                     ((t * H + g) * D + c * X) * E);
    char* dst = reinterpret_cast<char*>(a.k_cache) +
                ((((blk * H + g) * NCH + c) << a.tile_shift) + off) * 16;
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
  } else if (tid < nk + nv) {
    const int64_t e = tid - nk;
    const int64_t t = e / (H * D);
    const int rem = (int)(e - t * H * D);
    const int g = rem / D, d = rem - g * D;
    const int64_t slot = a.slot_mapping[t];
    if (slot < 0) return;
    const int64_t blk = slot >> a.tile_shift;  // tile of T = 2^tile_shift tokens
    const int off = (int)(slot & ((1 << a.tile_shift) - 1));
    const int64_t dst = (((blk * H + g) * D + d) << a.tile_shift) + off;
    if constexpr (E == 4)
      __builtin_nontemporal_store(reinterpret_cast<const uint32_t*>(a.value)[e],
                                  reinterpret_cast<uint32_t*>(a.v_cache) + dst);
    else
      __builtin_nontemporal_store(reinterpret_cast<const uint16_t*>(a.value)[e],
                                  reinterpret_cast<uint16_t*>(a.v_cache) + dst);
  }
}

// FP8 pools ("vLLM 深度拆解" §10.1 names FP8 with calibrated scales): the fp16 or bf16 inputs are
// quantised on the way in, element x -> e4m3(fp32(x) / scale) with one scale per pool.  One
// thread per 16-byte K chunk (16 elements: two 16-byte input loads, one 16-byte store), then
// one thread per V element (a byte store into the token's column of its dimension row).
template <int DT>  // DT_FP8: fp16 inputs; DT_FP8B: bf16 inputs
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(ReshapeArgs a) {
  auto lo = [](uint32_t w) { return DT == DT_FP8B ? bf16_lo(w) : f16_lo(w); };
  auto hi = [](uint32_t w) { return DT == DT_FP8B ? bf16_hi(w) : f16_hi(w); };
  constexpr int X = 16;
  const int H = a.num_kv_heads, D = a.head_dim, NCH = D / X;
  const int64_t nk = a.num_tokens * H * NCH;
  const int64_t nv = a.num_tokens * H * D;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid < nk) {
    const int64_t t = tid / (H * NCH);
    const int rem = (int)(tid - t * H * NCH);
    const int g = rem / NCH, c = rem - g * NCH;
    const int64_t slot = a.slot_mapping[t];
    if (slot < 0) return;  // padding token
    const int64_t blk = slot >> a.tile_shift;  // tile of T = 2^tile_shift tokens
    const int off = (int)(slot & ((1 << a.tile_shift) - 1));
    const char* src = reinterpret_cast<const char*>(a.key) + ((t * H + g) * D + c * X) * 2;
    const uint4 h0 = ld16(src), h1 = ld16(src + 16);
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4& h = k < 2 ? h0 : h1;
      const uint32_t p0 = (k & 1) ? h.z : h.x, p1 = (k & 1) ? h.w : h.y;
      w[k] = f32_to_fp8(lo(p0) / a.k_scale) | (f32_to_fp8(hi(p0) / a.k_scale) << 8) |
             (f32_to_fp8(lo(p1) / a.k_scale) << 16) | (f32_to_fp8(hi(p1) / a.k_scale) << 24);
    }
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
    char* dst = reinterpret_cast<char*>(a.k_cache) + ((((blk * H + g) * NCH + c) << a.tile_shift) + off) * 16;
    __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4*>(dst));
  } else if (tid < nk + nv) {
    const int64_t e = tid - nk;
    const int64_t t = e / (H * D);
    const int rem = (int)(e - t * H * D);
    const int g = rem / D, d = rem - g * D;
    const int64_t slot = a.slot_mapping[t];
    if (slot < 0) return;
    const int64_t blk = slot >> a.tile_shift;  // tile of T = 2^tile_shift tokens
    const int off = (int)(slot & ((1 << a.tile_shift) - 1));
    const uint32_t xb = reinterpret_cast<const uint16_t*>(a.value)[e];
    const float x = DT == DT_FP8B ? bf16_lo(xb) : f16_lo(xb);
    __builtin_nontemporal_store((uint8_t)f32_to_fp8(x / a.v_scale),
                                reinterpret_cast<uint8_t*>(a.v_cache) + (((blk * H + g) * D + d) << a.tile_shift) + off);
  }
}

hipError_t launch_reshape(int dt, const ReshapeArgs& a, hipStream_t st) {
  if (is_fp8(dt)) {
    const int64_t threads = a.num_tokens * a.num_kv_heads * (a.head_dim / 16 + a.head_dim);
    const int64_t grid = (threads + 255) / 256;
    if (grid == 0) return hipSuccess;
    if (dt == DT_FP8B)
      hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<DT_FP8B>, dim3((unsigned)grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<DT_FP8>, dim3((unsigned)grid), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  const int X = dt == DT_F32 ? 4 : 8;
  const int64_t threads = a.num_tokens * a.num_kv_heads * (a.head_dim / X + a.head_dim);
  const int64_t grid = (threads + 255) / 256;
  if (grid == 0) return hipSuccess;
  switch (dt) {
    case DT_F32: hipLaunchKernelGGL(reshape_and_cache_kernel<DT_F32>, dim3((unsigned)grid), dim3(256), 0, st, a); break;
    case DT_F16: hipLaunchKernelGGL(reshape_and_cache_kernel<DT_F16>, dim3((unsigned)grid), dim3(256), 0, st, a); break;
    default:     hipLaunchKernelGGL(reshape_and_cache_kernel<DT_BF16>, dim3((unsigned)grid), dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace pa
