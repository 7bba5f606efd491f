// measure.hip — HBM read ceilings the benchmark compares the decode kernels with.  Not part
// of the attention path: two read-only kernels that fetch bytes and fold them into a sink
// so that the loads cannot be dropped.
//
//  - stream: one contiguous buffer read front to back, 16 bytes per lane and four loads in
//    flight per lane, workgroups striding over the buffer (the best case for HBM).
//  - tiles: a list of equal-size tiles at arbitrary byte offsets (e.g. every 4 KiB K and V
//    tile a decode batch reads, in the order the decode walks them), split evenly over the
//    waves of the grid as the decode's even split does: the attainable rate of that access
//    pattern with no attention arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"
#include "pa_measure.h"

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t fold(const uint4& v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* p, int64_t n16,
                                                               uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
  }
  for (; i < n16; i += stride) acc ^= fold(p[i]);
  // a store that practically never happens keeps every load alive
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

// wave w of W reads tiles [w * n / W, (w + 1) * n / W); a tile of B bytes is B / 1024 loads of
// one contiguous KiB per wave (16 bytes per lane), two tiles in flight
__global__ __launch_bounds__(kThreads) void tile_read_kernel(const char* base, const int64_t* off,
                                                             int64_t n, int tile_bytes,
                                                             uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t W = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t w = (int64_t)blockIdx.x * (kThreads / 64) + threadIdx.x / 64;
  const int64_t t0 = w * n / W, t1 = (w + 1) * n / W;
  const int loads = tile_bytes / 1024;
  uint32_t acc = 0;
  int64_t t = t0;
  for (; t + 1 < t1; t += 2) {
    const char* a = base + off[t] + 16 * lane;
    const char* b = base + off[t + 1] + 16 * lane;
    for (int k = 0; k < loads; ++k) {
      const uint4 x = *reinterpret_cast<const uint4*>(a + 1024 * k);
      const uint4 y = *reinterpret_cast<const uint4*>(b + 1024 * k);
      acc ^= fold(x) ^ fold(y);
    }
  }
  if (t < t1) {
    const char* a = base + off[t] + 16 * lane;
    for (int k = 0; k < loads; ++k) acc ^= fold(*reinterpret_cast<const uint4*>(a + 1024 * k));
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

int cu_count_now() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  return n;
}

}  // namespace

extern "C" {

pa_status pa_measure_stream_read(const void* buf, size_t bytes, uint32_t* sink,
                                 int32_t workgroups, void* stream) {
  if (bytes == 0) return PA_OK;
  if (!buf || !sink) return PA_ERR_NULL;
  if (bytes % 16 || workgroups < 0) return PA_ERR_SHAPE;
  const int grid = workgroups > 0 ? workgroups : cu_count_now() * 8;
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<const uint4*>(buf), (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_measure_tile_read(const void* base, const int64_t* tile_offsets, int64_t num_tiles,
                               int32_t tile_bytes, uint32_t* sink, int32_t workgroups,
                               void* stream) {
  if (num_tiles == 0) return PA_OK;
  if (!base || !tile_offsets || !sink) return PA_ERR_NULL;
  if (num_tiles < 0 || tile_bytes <= 0 || tile_bytes % 1024 || workgroups < 0) return PA_ERR_SHAPE;
  const int grid = workgroups > 0 ? workgroups : cu_count_now();
  hipLaunchKernelGGL(tile_read_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<const char*>(base), tile_offsets, num_tiles, (int)tile_bytes,
                     sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
