// reshape.hip — the paged KV-cache write ("vLLM 架构源码解析 第1篇" §3.3.3: reshape_and_cache
// scatters this step's K and V into the block pool at slot_mapping before attention; the
// block / offset split of a slot is §4.2's `//` and `%` by the block size).  The pools are
// addressed in tiles of T tokens: T = 8 for 8-token blocks, else 16 (a block of 32 or 64
// tokens is 2 or 4 consecutive 16-token tiles, so slot / 16 names a tile for every block
// size from 16 up).
//
// Tokens are written in segments: a segment is a maximal run of consecutive tokens of
// slot_mapping whose slots are consecutive within one tile (at most T tokens; a prompt or
// prefill chunk is a chain of them, a decode token a segment of one).  Workgroup (k, head)
// writes the segments that start among tokens [kT, kT + T), each of which may reach up to
// T - 1 tokens past them.  Within the workgroup consecutive threads take consecutive tokens
// of a segment, so a wave's stores fill each row of a tile contiguously: 16-byte K chunks
// along a chunk plane's row, V elements along a dimension row.  16-bit and fp32 pools get a
// bit copy; FP8 pools ("vLLM 深度拆解" §10.1 names FP8 with calibrated scales) quantise each
// element on the way in, x -> e4m3(fp32(x) / scale), with one scale per pool.
//
// The stores are non-temporal: left dirty in L2, the partly written lines of a decode step
// were written back while the next decode streamed the pools and cost it ~5% on the LLaMA-7B
// batch; streamed stores leave nothing behind.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kReshapeThreads = 256;
constexpr int kMaxTile = 16;     // tokens of a pool tile

template <int DT>
struct RCfg {
  static constexpr bool F8 = is_fp8(DT);
  static constexpr int IE = F8 ? 2 : DtInfo<DT>::bytes;  // input element bytes
  static constexpr int OE = F8 ? 1 : DtInfo<DT>::bytes;  // pool element bytes
  static constexpr int X = 16 / OE;                      // elements per 16-byte pool chunk
};

// an FP8 pool's input element (fp16 or bf16 bits) as fp32
template <int DT>
__device__ __forceinline__ float f8_input(uint32_t bits) {
  return DT == DT_FP8B ? bf16_lo(bits) : f16_lo(bits);
}

// The 16-byte pool chunk of the X consecutive input elements at src.
template <int DT>
__device__ __forceinline__ uint4 pool_chunk(const char* src, float scale) {
  if constexpr (!RCfg<DT>::F8) {
    (void)scale;
    return ld16(src);
  } else {
    const uint4 h0 = ld16(src), h1 = ld16(src + 16);
    const uint32_t in[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t p0 = in[2 * k], p1 = in[2 * k + 1];
      w[k] = f32_to_fp8(f8_input<DT>(p0) / scale) |
             (f32_to_fp8(f8_input<DT>(p0 >> 16) / scale) << 8) |
             (f32_to_fp8(f8_input<DT>(p1) / scale) << 16) |
             (f32_to_fp8(f8_input<DT>(p1 >> 16) / scale) << 24);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// One V element's pool bits (input element bits: 16-bit, or fp32 for fp32 pools).
template <int DT>
__device__ __forceinline__ uint32_t pool_elem(uint32_t bits, float scale) {
  if constexpr (RCfg<DT>::F8) return f32_to_fp8(f8_input<DT>(bits) / scale);
  else return bits;
}

template <int DT>
__device__ __forceinline__ uint32_t load_elem(const char* p) {
  if constexpr (RCfg<DT>::IE == 4) return *reinterpret_cast<const uint32_t*>(p);
  else return *reinterpret_cast<const uint16_t*>(p);
}

template <int DT>
__device__ __forceinline__ void store_elem(char* p, uint32_t v) {
  if constexpr (RCfg<DT>::OE == 4)
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
  else if constexpr (RCfg<DT>::OE == 2)
    __builtin_nontemporal_store((uint16_t)v, reinterpret_cast<uint16_t*>(p));
  else
    __builtin_nontemporal_store((uint8_t)v, reinterpret_cast<uint8_t*>(p));
}

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

__device__ __forceinline__ void store16(char* p, const uint4& v) {
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
}

template <int DT>
__global__ __launch_bounds__(kReshapeThreads) void reshape_and_cache_kernel(ReshapeArgs a) {
  using R = RCfg<DT>;
  const int shift = a.tile_shift;
  const int T = 1 << shift;
  const int H = a.num_kv_heads, D = a.head_dim, NCH = D / R::X;
  const int g = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * T;
  const int tid = threadIdx.x;
  // slots of tokens t0 - 1 .. t0 + 2T - 2 (-1 outside the batch)
  __shared__ int64_t sl[2 * kMaxTile];
  __shared__ int seg_t[kMaxTile + 1];  // first token (offset from t0) of each segment
  __shared__ int seg_c[kMaxTile + 1];  // tokens of the segments before it
  __shared__ int nseg;
  __shared__ int in_order;  // the workgroup writes tokens t0, t0 + 1, .. t0 + Ms - 1 in order
  const char* key = static_cast<const char*>(a.key);
  const char* val = static_cast<const char*>(a.value);
  const int64_t row_in = (int64_t)D * R::IE;  // bytes of one (token, head) input row
  constexpr int KU = 2, VU = 8;

  // Loads issued before the slots are known: decode tokens (one-token segments) and chunks
  // whose segments start at t0 make the workgroup write tokens t0 .. t0 + Ms - 1 in order,
  // the j-th at offset j, so each thread loads its pieces of that order (K chunk c of token
  // j: piece c Ms + j; V dimension d: piece d Ms + j) beside the slot loads and keeps them
  // when the segment scan finds that order; otherwise the pieces are loaded again below.
  const int Ms = (int)min((int64_t)T, a.num_tokens - t0);
  uint4 kpre[KU];
  uint32_t vpre[VU];
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int i = u * kReshapeThreads + tid;
    if (i < NCH * Ms) {
      const int c = i / Ms, j = i - c * Ms;
      kpre[u] = pool_chunk<DT>(key + ((t0 + j) * H + g) * row_in + (int64_t)c * R::X * R::IE,
                               a.k_scale);
    }
  }
#pragma unroll
  for (int u = 0; u < VU; ++u) {
    const int i = u * kReshapeThreads + tid;
    if (i < D * Ms) {
      const int d = i / Ms, j = i - d * Ms;
      vpre[u] = load_elem<DT>(val + ((t0 + j) * H + g) * row_in + (int64_t)d * R::IE);
    }
  }
  if (tid < kWave) {
    const int64_t t = t0 - 1 + tid;
    const int64_t s = tid < 2 * T && t >= 0 && t < a.num_tokens ? a.slot_mapping[t] : -1;
    if (tid < 2 * T) sl[tid] = s;
    // token t continues the segment of t - 1: same tile, next slot
    const int64_t prev = ((int64_t)__shfl((int)(s >> 32), tid - 1) << 32) |
                         (uint32_t)__shfl((int)s, tid - 1);
    const bool cont = tid > 0 && s >= 0 && prev >= 0 && s == prev + 1 && (s >> shift) == (prev >> shift);
    // segments that start at tokens t0 .. t0 + T - 1 (lanes 1 .. T)
    const bool start = tid >= 1 && tid <= T && s >= 0 && !cont;
    const uint64_t starts = __builtin_amdgcn_ballot_w64(start);
    const uint64_t conts = __builtin_amdgcn_ballot_w64(cont);
    // a segment's length: its start and the run of continuing tokens after it
    const uint64_t after = ~conts >> (tid + 1);
    int len = start ? min(__builtin_ctzll(after | (1ull << 62)), T - 1) + 1 : 0;
    // tokens of the segments before each one: an exclusive scan over the lanes
    int incl = len;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int v = __shfl_up(incl, d, kWave);
      if (tid >= d) incl += v;
    }
    if (start) {
      const int k = __popcll(starts & ((1ull << tid) - 1));  // segments before this one
      seg_t[k] = tid - 1;
      seg_c[k] = incl - len;
    }
    // in order: every segment starts where the ones before it end, and they hold Ms tokens
    const uint64_t gaps = __builtin_amdgcn_ballot_w64(start && tid - 1 != incl - len);
    if (tid == kWave - 1) {
      nseg = __popcll(starts);
      seg_c[__popcll(starts)] = incl;  // every token of the workgroup
      in_order = gaps == 0 && incl == Ms;
    }
  }
  __syncthreads();
  const int ns = nseg;
  const int M = seg_c[ns];  // tokens this workgroup writes
  if (M == 0) return;
  char* kc = static_cast<char*>(a.k_cache);
  char* vc = static_cast<char*>(a.v_cache);
  if (in_order && NCH * M <= KU * kReshapeThreads && D * M <= VU * kReshapeThreads) {
    // token j at offset j: the pieces loaded above, stored at their slots
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int i = u * kReshapeThreads + tid;
      if (i < NCH * M) {
        const int c = i / M, j = i - c * M;
        const int64_t slot = sl[j + 1];
        const int64_t dst = ((((slot >> shift) * H + g) * NCH + c) << shift) + (slot & (T - 1));
        store16(kc + dst * 16, kpre[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int i = u * kReshapeThreads + tid;
      if (i < D * M) {
        const int d = i / M, j = i - d * M;
        const int64_t slot = sl[j + 1];
        const int64_t dst = ((((slot >> shift) * H + g) * D + d) << shift) + (slot & (T - 1));
        store_elem<DT>(vc + dst * R::OE, pool_elem<DT>(vpre[u], a.v_scale));
      }
    }
    return;
  }
  // j-th token of the workgroup (segments in order): its offset from t0 and its slot
  auto token = [&](int j, int& off, int64_t& slot) {
    int k = 0, hi = ns - 1;  // the last segment with seg_c[k] <= j
    while (k < hi) {
      const int mid = (k + hi + 1) >> 1;
      if (seg_c[mid] <= j)
        k = mid;
      else
        hi = mid - 1;
    }
    off = seg_t[k] + (j - seg_c[k]);
    slot = sl[off + 1];
  };
  // K: chunk c of token j is piece c * M + j
  for (int i0 = 0; i0 < NCH * M; i0 += KU * kReshapeThreads) {
    uint4 v[KU];
    int64_t dst[KU];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int i = i0 + u * kReshapeThreads + tid;
      dst[u] = -1;
      if (i < NCH * M) {
        const int c = i / M, j = i - c * M;
        int off;
        int64_t slot;
        token(j, off, slot);
        const int64_t blk = slot >> shift;
        dst[u] = ((((blk * H + g) * NCH + c) << shift) + (slot & (T - 1))) * 16;
        v[u] = pool_chunk<DT>(key + ((t0 + off) * H + g) * row_in + (int64_t)c * R::X * R::IE,
                              a.k_scale);
      }
    }
#pragma unroll
    for (int u = 0; u < KU; ++u)
      if (dst[u] >= 0) store16(kc + dst[u], v[u]);
  }
  // V: dimension d of token j is piece d * M + j
  for (int i0 = 0; i0 < D * M; i0 += VU * kReshapeThreads) {
    uint32_t v[VU];
    int64_t dst[VU];
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int i = i0 + u * kReshapeThreads + tid;
      dst[u] = -1;
      if (i < D * M) {
        const int d = i / M, j = i - d * M;
        int off;
        int64_t slot;
        token(j, off, slot);
        const int64_t blk = slot >> shift;
        dst[u] = ((((blk * H + g) * D + d) << shift) + (slot & (T - 1))) * R::OE;
        v[u] = load_elem<DT>(val + ((t0 + off) * H + g) * row_in + (int64_t)d * R::IE);
      }
    }
#pragma unroll
    for (int u = 0; u < VU; ++u)
      if (dst[u] >= 0) store_elem<DT>(vc + dst[u], pool_elem<DT>(v[u], a.v_scale));
  }
}

hipError_t launch_reshape(int dt, const ReshapeArgs& a, hipStream_t st) {
  const int64_t groups = (a.num_tokens + (1 << a.tile_shift) - 1) >> a.tile_shift;
  if (groups == 0) return hipSuccess;
  const dim3 grid((unsigned)groups, (unsigned)a.num_kv_heads);
  switch (dt) {
    case DT_F32: hipLaunchKernelGGL(reshape_and_cache_kernel<DT_F32>, grid, dim3(kReshapeThreads), 0, st, a); break;
    case DT_F16: hipLaunchKernelGGL(reshape_and_cache_kernel<DT_F16>, grid, dim3(kReshapeThreads), 0, st, a); break;
    case DT_BF16: hipLaunchKernelGGL(reshape_and_cache_kernel<DT_BF16>, grid, dim3(kReshapeThreads), 0, st, a); break;
    case DT_FP8: hipLaunchKernelGGL(reshape_and_cache_kernel<DT_FP8>, grid, dim3(kReshapeThreads), 0, st, a); break;
    default: hipLaunchKernelGGL(reshape_and_cache_kernel<DT_FP8B>, grid, dim3(kReshapeThreads), 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace pa
