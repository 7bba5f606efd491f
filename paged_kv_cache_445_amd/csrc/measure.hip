// measure.hip — HBM read ceilings the benchmark compares the decode kernels with.  Not part
// of the attention path: two read-only kernels that fetch bytes and fold them into a sink
// so that the loads cannot be dropped.  Both load with the streaming (non-temporal) policy,
// as the decode kernels do.
//
//  - stream: one contiguous buffer read in 16 KiB pieces, one per wave at a time with all 16
//    of its one-KiB loads in flight, pieces striding over the buffer (the best case for HBM).
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

__device__ __forceinline__ uint4 ld_stream(const char* p) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Each wave reads a contiguous 16 KiB piece per iteration (16 loads of one KiB in flight),
// pieces handed out with a grid stride; the tail (bytes past the last whole piece) is read
// 16 bytes per lane.
constexpr int kPieceLoads = 16;
constexpr int64_t kPiece = kPieceLoads * 1024;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const char* p, int64_t bytes,
                                                               uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t W = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t w = (int64_t)blockIdx.x * (kThreads / 64) + threadIdx.x / 64;
  const int64_t pieces = bytes / kPiece;
  uint32_t acc = 0;
  for (int64_t k = w; k < pieces; k += W) {
    const char* q = p + k * kPiece + 16 * lane;
    uint4 v[kPieceLoads];
#pragma unroll
    for (int i = 0; i < kPieceLoads; ++i) v[i] = ld_stream(q + 1024 * i);
#pragma unroll
    for (int i = 0; i < kPieceLoads; ++i) acc ^= fold(v[i]);
  }
  for (int64_t e = pieces * kPiece + (w * 64 + lane) * 16; e < bytes; e += W * 64 * 16)
    acc ^= fold(ld_stream(p + e));
  // a store that practically never happens keeps every load alive
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

// wave w of W reads tiles [w * n / W, (w + 1) * n / W); a tile of B bytes is B / 1024 loads of
// one contiguous KiB per wave (16 bytes per lane); eight tiles of up to 4 KiB in flight
constexpr int kTilesInFlight = 8;

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
  if (loads == 4) {
    for (; t + kTilesInFlight <= t1; t += kTilesInFlight) {
      uint4 v[kTilesInFlight][4];
#pragma unroll
      for (int j = 0; j < kTilesInFlight; ++j) {
        const char* a = base + off[t + j] + 16 * lane;
#pragma unroll
        for (int k = 0; k < 4; ++k) v[j][k] = ld_stream(a + 1024 * k);
      }
#pragma unroll
      for (int j = 0; j < kTilesInFlight; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc ^= fold(v[j][k]);
    }
  }
  for (; t < t1; ++t) {
    const char* a = base + off[t] + 16 * lane;
    for (int k = 0; k < loads; ++k) acc ^= fold(ld_stream(a + 1024 * k));
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
  const int grid = workgroups > 0 ? workgroups : cu_count_now() * 2;
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<const char*>(buf), (int64_t)bytes, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_measure_tile_read(const void* base, const int64_t* tile_offsets, int64_t num_tiles,
                               int32_t tile_bytes, uint32_t* sink, int32_t workgroups,
                               void* stream) {
  if (num_tiles == 0) return PA_OK;
  if (!base || !tile_offsets || !sink) return PA_ERR_NULL;
  if (num_tiles < 0 || tile_bytes <= 0 || tile_bytes % 1024 || workgroups < 0) return PA_ERR_SHAPE;
  const int grid = workgroups > 0 ? workgroups : cu_count_now() * 2;
  hipLaunchKernelGGL(tile_read_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<const char*>(base), tile_offsets, num_tiles, (int)tile_bytes,
                     sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
