// copy_blocks.hip — whole-block copies inside the K and V pools.
//
// Copy-on-write ("vLLM 架构源码解析 第1篇" §4.3.2): samples forked from one prompt share its
// blocks; before a sample writes into a block that others still reference, the block
// manager gives it a fresh block holding a copy of the shared one.  This kernel makes those
// copies for a list of (source, destination) pairs.
//
// In both pools the tiles of all KV heads of one block are adjacent, so a block is one
// contiguous run of num_kv_heads * block_size * head_dim * elem bytes in each pool.  A
// workgroup copies one 16 KiB piece of one run: four 16-byte loads per thread, issued
// together, then four stores.  Consecutive threads move consecutive 16-byte chunks, so
// every load and store instruction of a wave covers one contiguous KiB.  The stores are
// streamed (non-temporal), like the cache write's, so the copies leave no dirty lines in L2
// behind them for the next decode to evict.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kCopyLoads = 4;                           // 16-byte chunks per thread
constexpr int kCopyPiece = kWG * kCopyLoads * 16;       // bytes per workgroup: 16 KiB

__global__ __launch_bounds__(kWG) void copy_blocks_kernel(CopyBlocksArgs a) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  // blockIdx.x = (pair * 2 + pool) * pieces + piece
  const int64_t pieces = (a.block_bytes + kCopyPiece - 1) / kCopyPiece;
  const int64_t w = blockIdx.x;
  const int64_t pair = w / (2 * pieces);
  const int pool = (int)(w / pieces) & 1;
  const int64_t piece = w % pieces;
  const int64_t src = a.block_mapping[2 * pair];
  const int64_t dst = a.block_mapping[2 * pair + 1];
  if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks) return;  // skipped pair
  char* base = reinterpret_cast<char*>(pool ? a.v_cache : a.k_cache);
  const char* s = base + src * a.block_bytes;
  char* d = base + dst * a.block_bytes;
  const int64_t off0 = piece * kCopyPiece + (int64_t)threadIdx.x * 16;
  u32x4 v[kCopyLoads];
#pragma unroll
  for (int k = 0; k < kCopyLoads; ++k) {
    const int64_t off = off0 + (int64_t)k * kWG * 16;
    if (off < a.block_bytes) v[k] = *reinterpret_cast<const u32x4*>(s + off);
  }
#pragma unroll
  for (int k = 0; k < kCopyLoads; ++k) {
    const int64_t off = off0 + (int64_t)k * kWG * 16;
    if (off < a.block_bytes) __builtin_nontemporal_store(v[k], reinterpret_cast<u32x4*>(d + off));
  }
}

// Swap ("vLLM 架构源码解析 第1篇" §1.1, preemption by swapping): the same pieces between a
// device pool and a pinned host pool mapped into the device's address space, so that one
// launch moves every pair over PCIe instead of one copy-engine transfer per block.
__global__ __launch_bounds__(kWG) void swap_blocks_kernel(SwapArgs a) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  const int64_t pieces = (a.block_bytes + kCopyPiece - 1) / kCopyPiece;
  const int64_t w = blockIdx.x;
  const int64_t pair = w / (2 * pieces);
  const int pool = (int)(w / pieces) & 1;
  const int64_t piece = w % pieces;
  if (pair >= a.num_pairs) return;
  const char* s = (pool ? a.src_v : a.src_k) + a.pairs[pair][0] * a.block_bytes;
  char* d = (pool ? a.dst_v : a.dst_k) + a.pairs[pair][1] * a.block_bytes;
  const int64_t off0 = piece * kCopyPiece + (int64_t)threadIdx.x * 16;
  u32x4 v[kCopyLoads];
#pragma unroll
  for (int k = 0; k < kCopyLoads; ++k) {
    const int64_t off = off0 + (int64_t)k * kWG * 16;
    if (off < a.block_bytes) v[k] = *reinterpret_cast<const u32x4*>(s + off);
  }
#pragma unroll
  for (int k = 0; k < kCopyLoads; ++k) {
    const int64_t off = off0 + (int64_t)k * kWG * 16;
    if (off < a.block_bytes) __builtin_nontemporal_store(v[k], reinterpret_cast<u32x4*>(d + off));
  }
}

hipError_t launch_swap_blocks(const SwapArgs& a, hipStream_t st) {
  const int64_t pieces = (a.block_bytes + kCopyPiece - 1) / kCopyPiece;
  const int64_t grid = (int64_t)a.num_pairs * 2 * pieces;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(swap_blocks_kernel, dim3((unsigned)grid), dim3(kWG), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t st) {
  const int64_t pieces = (a.block_bytes + kCopyPiece - 1) / kCopyPiece;
  const int64_t grid = a.num_pairs * 2 * pieces;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)grid), dim3(kWG), 0, st, a);
  return hipGetLastError();
}

}  // namespace pa
