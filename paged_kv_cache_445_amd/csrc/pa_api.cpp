// pa_api.cpp — the C entry points of libpa.so (include/pa.h): argument checks, kernel choice,
// grid sizing and launches.  Nothing here allocates, frees or synchronises device memory.
#include <hip/hip_runtime.h>
#include <stdlib.h>

#include <atomic>
#include <algorithm>
#include <cmath>
#include <mutex>

#include "pa.h"
#include "pa_internal.h"

namespace pa {
hipError_t launch_chunk(int dt, const DecodeArgs& a, int num_q_rows, hipStream_t st);
hipError_t launch_prefix(int dt, const DecodeArgs& a, int num_q_rows, hipStream_t st);
}

namespace {

constexpr int kMaxSeqs = 8192;  // the split kernels keep one int per sequence in LDS
constexpr int kMaxDevices = 64;

size_t elem_bytes(int dt) { return dt == PA_F32 ? 4 : dt == PA_FP8_E4M3 ? 1 : 2; }

bool dtype_ok(int dt) { return dt == PA_F32 || dt == PA_F16 || dt == PA_BF16; }

pa_status check_geom(const pa_geom* g) {
  if (!g) return PA_ERR_NULL;
  if (g->num_seqs < 0 || g->num_q_heads <= 0 || g->num_kv_heads <= 0 || g->head_dim <= 0 ||
      g->block_size <= 0 || g->num_blocks <= 0 || g->max_blocks_per_seq <= 0)
    return PA_ERR_SHAPE;
  if (g->num_q_heads % g->num_kv_heads) return PA_ERR_SHAPE;
  if (g->kv_dtype == PA_FP8_E4M3) {
    if (g->q_dtype != PA_F16 && g->q_dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
    if (!(std::isfinite(g->k_scale) && g->k_scale > 0.f && std::isfinite(g->v_scale) &&
          g->v_scale > 0.f))
      return PA_ERR_SHAPE;
  } else if (g->q_dtype != g->kv_dtype) {
    return dtype_ok(g->kv_dtype) ? PA_ERR_SHAPE : PA_ERR_UNSUPPORTED;
  }
  if (!dtype_ok(g->q_dtype) || !dtype_ok(g->out_dtype)) return PA_ERR_UNSUPPORTED;
  if (g->out_dtype != g->q_dtype && g->out_dtype != PA_F32) return PA_ERR_UNSUPPORTED;
  if (g->block_size != 8 && g->block_size != 16 && g->block_size != 32 && g->block_size != 64)
    return PA_ERR_UNSUPPORTED;
  // the kernels number pool tiles (16-token sub-blocks, or 8-token blocks) in int32
  if ((int64_t)g->num_blocks * (g->block_size > 16 ? g->block_size / pa::kBlock : 1) >
      0x7fffffffLL)
    return PA_ERR_SHAPE;
  if (g->head_dim != 64 && g->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (g->num_q_heads / g->num_kv_heads > 16) return PA_ERR_UNSUPPORTED;
  if (g->num_seqs > kMaxSeqs) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

// element type code of the kernels: the pool's, FP8 pools split by their query type
int kdt(const pa_geom* g) {
  if (g->kv_dtype != PA_FP8_E4M3) return g->kv_dtype;
  return g->q_dtype == PA_BF16 ? pa::DT_FP8B : pa::DT_FP8;
}

// log2 of the 16-token sub-blocks per block (blocks of 16 tokens and up)
int blk_shift(const pa_geom* g) { return g->block_size == 64 ? 2 : g->block_size == 32 ? 1 : 0; }

// 8-token blocks: the kernels pair two blocks into each 16-token tile
int b8(const pa_geom* g) { return g->block_size == 8 ? 1 : 0; }

int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  return dev;
}

int cu_count() {
  static std::atomic<int> cache[kMaxDevices];
  const int dev = current_device();
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Balancing units per segment of pa_decode's even split: the cost of starting a piece
// (query, table window, pipeline fill, partial) in the split's units of work.  That cost is
// roughly a fixed time, about as long as streaming 16-32 KiB of one head's K and V, so it
// is worth twice as many units over FP8 pools (half the bytes per unit).  Vector path
// (16-token tiles): 4 for 16-bit pools (LLaMA-7B batch 107.1 -> 106.6 us against 2), 8 for
// FP8 (63.2 -> 60.8 us), 2 for fp32.  Matrix-core path (32-token units): 1 for 16-bit (the
// GQA batch is best at 1), 4 for FP8 (GQA FP8 batch 153.3 -> 147.2 us at 2 against 1; with
// streaming tile loads the verify rows take 67.2 / 66.2 / 66.5 us at 2 / 4 / 6 and the GQA
// batch 133.1 / 133.2 / 134.2 us).  Optional override for tuning.
int seg_extra_default(const pa_geom* g, int path) {
  const bool f8 = g->kv_dtype == PA_FP8_E4M3;
  if (path) return f8 ? 4 : 1;
  return g->kv_dtype == PA_F32 ? 2 : f8 ? 8 : 4;
}
int seg_extra_override() {
  static int v = [] {
    const char* s = getenv("PA_DECODE_SEG_EXTRA");
    return s ? atoi(s) : -1;
  }();
  return v;
}

// optional choice of resident workgroups per CU for the split kernels (tuning; capped at the
// kernel's occupancy)
int wg_per_cu_override() {
  static int v = [] {
    const char* s = getenv("PA_DECODE_WG_PER_CU");
    return s ? atoi(s) : 0;
  }();
  return v;
}

// Per mille of the even split's work moved from the workgroups on odd XCDs to those on even
// XCDs (see make_part).  With cached loads the odd XCDs finished the decode's random 4 KiB
// tile reads about 7% later than the even ones; with the streaming loads the decode now uses,
// a sweep (0 / 20-30 / 55 / 80-100) puts the shortest call at 55 for the vector kernel on
// 16-bit pools (LLaMA-7B 97.3 / 95.7 / 95.3 / 96.0 us; shared prefix 190.4 / 189.0 /
// 187.3 us) and at 0 for FP8 pools on it (54.6 / 54.8 / 55.6 us) and for the matrix-core
// kernel (GQA 238.5 / 241.9 / 246.6 us, verify 107.6 / 108.7 / 110.6 us).  Optional
// override for tuning.
constexpr int kOddSkewVector16 = 55;
int odd_skew(const pa_geom* g, int path) {
  static const int v = [] {
    const char* s = getenv("PA_DECODE_ODD_SKEW");
    return s ? atoi(s) : -1;
  }();
  if (v >= 0) return v;
  return path == 0 && g->kv_dtype != PA_FP8_E4M3 ? kOddSkewVector16 : 0;
}

// The vector kernel's even split in (head group, sequence, tile) order over XCD-major
// owners (see Part in pa_device.h); optional override for tuning (0 / 1)
int xcd_major_override() {
  static const int v = [] {
    const char* s = getenv("PA_DECODE_XCD_MAJOR");
    return s ? atoi(s) : -1;
  }();
  return v;
}

bool use_mfma(const pa_geom* g) {
  return g->kv_dtype != PA_F32 && g->num_q_heads / g->num_kv_heads >= 2;
}

// Which decode kernel runs a pa_decode call, and which sequences it takes (max_len: an upper
// bound of the rows of any sequence; 1 without query_start_loc).
//  - GQA (16-bit or FP8, G >= 2): the matrix-core kernel; when sequences may have several rows it
//    also takes those of up to 16 / G rows (a speculative verify step), nr * G columns at once.
//  - MHA 16-bit or FP8 with sequences of several rows: the matrix-core kernel too (G = 1, up to 16
//    rows a sequence), so verify rows read their K and V once instead of through the chunk
//    kernel's 128-column items.
//  - otherwise the vector kernel, one row per sequence.
// Longer sequences go to the chunk kernel.  cols: query columns per partial slot.
struct Route {
  int path;      // 0: vector kernel, 1: matrix-core kernel
  int max_rows;  // rows per sequence the decode kernel takes
  int cols;
};

Route route(const pa_geom* g, int32_t max_len) {
  const int G = g->num_q_heads / g->num_kv_heads;
  const bool multi = max_len > 1;
  if (use_mfma(g)) return {1, multi ? 16 / G : 1, multi ? 16 / G * G : G};
  if (g->kv_dtype != PA_F32 && multi) return {1, 16, 16};
  return {0, 1, 1};
}

// LDS of the split kernels: the per-sequence plan (num_seqs + 1 ints).
// Occupancy is evaluated for num_seqs rounded up to a power of two, so a handful of cached
// values covers every batch size.
int seq_bucket(int num_seqs) {
  int b = 0;
  while ((1 << b) < num_seqs + 1) ++b;
  return b;  // (1 << b) >= num_seqs + 1; b <= 14 for kMaxSeqs = 8192
}

int bucket_lds_bytes(int bucket) { return (1 << bucket) * (int)sizeof(int32_t); }

// resident workgroups per CU for pa_decode's even split (vector path, matrix-core path)
constexpr int kEvenWgPerCu[2] = {1, 2};
// ... for the vector path of pa_decode_shared_prefix, whose sequences are left with their
// (short) private tails: more waves in flight hide the start of more, shorter segments
// (prefix-shared batch: 216 -> 210 us)
constexpr int kSharedWgPerCu = 2;

// Query heads per wave of the vector path's even split: a wave runs heads h0 + 4 j
// (j < HPW), so a workgroup reads 4 HPW adjacent heads of a block back to back, which the
// HBM serves faster than the same bytes in smaller pieces.  Larger groups also mean fewer,
// longer segments, and once there are fewer segments than workgroups every segment is cut
// into several pieces whose merge costs more than the locality gains.  So: the largest of
// 8, 4, 2 whose head groups tile num_q_heads exactly and leave at least one segment per
// workgroup (fp32: at most 2, its queries fill twice the registers; FP8: at most 4, its
// values are widened to fp32 in registers), else 1; optional cap for tuning.  wg: resident
// workgroups per CU of the call (0: kEvenWgPerCu).
int heads_per_wave(const pa_geom* g, int wg = 0) {
  static const int v = [] {
    const char* s = getenv("PA_DECODE_HPW");
    return s ? atoi(s) : 0;
  }();
  if (b8(g)) return 1;  // 8-token blocks: one head per wave
  const int cap = g->kv_dtype == PA_F32 ? 2 : g->kv_dtype == PA_FP8_E4M3 ? 4 : 8;
  const int o = wg_per_cu_override();
  const int64_t workgroups = (int64_t)cu_count() * (o > 0 ? o : wg > 0 ? wg : kEvenWgPerCu[0]);
  for (int h = 8; h >= 2; h /= 2) {
    if (h > cap || (v > 0 && h > v) || g->num_q_heads % (pa::kWavesPerWG * h)) continue;
    const int64_t segments = (int64_t)g->num_seqs * (g->num_q_heads / (pa::kWavesPerWG * h));
    if (segments >= workgroups) return h;
  }
  return 1;
}

int hpw_index(int hpw) { return hpw == 8 ? 3 : hpw == 4 ? 2 : hpw == 2 ? 1 : 0; }

// workgroups of the split kernel: every CU full at the kernel's occupancy (wg: the even
// split's resident workgroups per CU on the vector path, 0: kEvenWgPerCu)
int split_grid(const pa_geom* g, int mode, int path, int wg = 0) {
  static std::atomic<int> cache[kMaxDevices][2][5][2][2][4][15];
  const int dev = current_device();
  const int di = g->head_dim == 64 ? 0 : 1;
  const int bk = seq_bucket(g->num_seqs);
  const int hpw = path == 0 && mode == pa::MODE_EVEN ? heads_per_wave(g, wg) : 1;
  std::atomic<int>& c = cache[dev][path][kdt(g)][di][mode][hpw_index(hpw)][bk];
  int occ = c.load(std::memory_order_relaxed);
  if (occ <= 0) {
    const int lds = bucket_lds_bytes(bk);
    occ = path ? pa::mfma_decode_max_blocks_per_cu(kdt(g), g->head_dim, mode, lds)
               : pa::valu_decode_max_blocks_per_cu(kdt(g), g->head_dim, hpw, mode, lds);
    c.store(occ, std::memory_order_relaxed);
  }
  // The even split streams best with few resident workgroups per CU: each of them reads
  // four adjacent heads of a block at a time, and more of them only add split pieces.
  const int o = wg_per_cu_override();
  int want = o > 0 ? o
                   : mode != pa::MODE_EVEN ? occ
                   : path == 0 && wg > 0 ? wg
                                         : kEvenWgPerCu[path];
  if (want > occ) want = occ;
  if (want > pa::kMaxWgPerCu) want = pa::kMaxWgPerCu;  // the workspace's counters cover this
  return cu_count() * want;
}

// pa_decode's workspace: one arrival counter per wave of the largest split grid the device
// can have (so the counters sit at the same place for every geometry and stay zero between
// calls), then two partial slots per wave of this geometry's grid: o [W][2][C][D],
// m [W][2][C], l [W][2][C] (C: query columns per wave: heads per wave on the vector path,
// Route::cols on the matrix-core path).
size_t counter_bytes() {
  const size_t n = (size_t)cu_count() * pa::kMaxWgPerCu * pa::kWavesPerWG * sizeof(int32_t);
  return (n + 255) / 256 * 256;
}

size_t even_slots(const pa_geom* g, int grid, const Route& r, int wg = 0) {
  const int cols = r.path ? r.cols : heads_per_wave(g, wg);
  return (size_t)grid * pa::kWavesPerWG * 2 * cols;
}

size_t even_workspace_bytes(const pa_geom* g, const Route& r, int wg = 0) {
  const int grid = split_grid(g, pa::MODE_EVEN, r.path, wg);
  return counter_bytes() + even_slots(g, grid, r, wg) * ((size_t)g->head_dim + 2) * sizeof(float);
}

// enough for the call with and without query_start_loc
size_t decode_workspace_bytes(const pa_geom* g, int32_t num_q_rows, int wg = 0) {
  const size_t a = even_workspace_bytes(g, route(g, num_q_rows), wg);
  const size_t b = even_workspace_bytes(g, route(g, 1), wg);
  return a > b ? a : b;
}

pa_status hip_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// A second stream per device for the multi-row (chunk) kernel, so that it runs beside the
// decode kernel of the same call: the two write disjoint rows and the chunk kernel is bound
// by the matrix cores, the decode kernel by HBM.  Created once per device at default
// priority; its two events fork the caller's stream into it and join it back.  The mutex
// orders concurrent calls that share the events (their chunk kernels then run one after
// the other on the side stream).
struct SideStream {
  std::once_flag once;
  hipError_t err = hipSuccess;
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex mu;
};

SideStream* side_stream(int dev) {
  static SideStream sides[kMaxDevices];
  SideStream& s = sides[dev];
  std::call_once(s.once, [&] {
    s.err = hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking);
    if (s.err == hipSuccess) s.err = hipEventCreateWithFlags(&s.fork, hipEventDisableTiming);
    if (s.err == hipSuccess) s.err = hipEventCreateWithFlags(&s.join, hipEventDisableTiming);
  });
  return s.err == hipSuccess ? &s : nullptr;
}

float scale_to_log2(float scale) { return scale * 1.4426950408889634f; }

// ---- the workspace of pa_decode_scratch: a static device array (no allocation) ----
// Each device the library runs on holds its own copy until the process ends.  Host code
// never passes `scratch` itself to a kernel or a copy (in host code the name is a host-side
// stand-in, not a device address): it looks the device address up once per device with
// hipGetSymbolAddress and uses that pointer.
constexpr size_t kScratchBytes = PA_DECODE_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void scratch_clear_kernel(int32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

struct ScratchSlot {
  std::once_flag once;
  hipError_t err = hipSuccess;
  void* ptr = nullptr;  // this device's copy of `scratch`
};

// The device address of `scratch` on the current device (dev), looked up on the first call
// on that device, which also clears the arrival counters at its start with a small kernel on
// `st` (a kernel rather than a memset, so that a caller may capture the call in a graph).
// Every decode call returns the counters to zero, so later calls find them cleared.
void* scratch_ptr(int dev, hipStream_t st) {
  static ScratchSlot slots[kMaxDevices];
  ScratchSlot& s = slots[dev];
  std::call_once(s.once, [&] {
    void* p = nullptr;
    s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (s.err != hipSuccess || !p) {
      if (s.err == hipSuccess) s.err = hipErrorInvalidSymbol;
      return;
    }
    const int64_t n = (int64_t)(counter_bytes() / sizeof(int32_t));
    hipLaunchKernelGGL(scratch_clear_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       static_cast<int32_t*>(p), n);
    s.err = hipGetLastError();
    if (s.err == hipSuccess) s.ptr = p;
  });
  return s.err == hipSuccess ? s.ptr : nullptr;
}

// ---- shared prefixes (pa_decode_shared_prefix) ----
// The groups' shared keys are attended in partials of `tokens` keys, at most `parts` per
// (row, head): the longest prefix the call allows (max_prefix_blocks blocks, whole 32-token
// units) in at most 8 partials of at least 128 keys.
struct PrefixParts {
  int tokens = 0;
  int parts = 0;
};

// optional override of the least keys per partial, for tuning (a multiple of 32)
int prefix_min_tokens() {
  static const int v = [] {
    const char* s = getenv("PA_PREFIX_MIN_TOKENS");
    const int t = s ? atoi(s) : 0;
    return t >= pa::kMfmaUnit && t % pa::kMfmaUnit == 0 ? t : 128;
  }();
  return v;
}

PrefixParts prefix_parts(const pa_geom* g, int32_t max_prefix_blocks) {
  PrefixParts pp;
  const int64_t keys = (int64_t)max_prefix_blocks * g->block_size / pa::kMfmaUnit * pa::kMfmaUnit;
  if (keys <= 0) return pp;
  const int64_t t = ((keys + 7) / 8 + pa::kMfmaUnit - 1) / pa::kMfmaUnit * pa::kMfmaUnit;
  pp.tokens = (int)std::max<int64_t>(prefix_min_tokens(), t);
  pp.parts = (int)((keys + pp.tokens - 1) / pp.tokens);
  return pp;
}

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// behind pa_decode's workspace: skip [S] int32, then the prefix partials o [rows][Hq][P][D],
// m and l [rows][Hq][P] (fp32)
struct PrefixSpace {
  size_t skip, o, m, l, end;
};

PrefixSpace prefix_space(const pa_geom* g, int32_t num_q_rows, size_t even_bytes,
                         const PrefixParts& pp) {
  PrefixSpace w;
  const size_t n = (size_t)num_q_rows * g->num_q_heads * pp.parts;
  w.skip = align256(even_bytes);
  w.o = align256(w.skip + (size_t)g->num_seqs * sizeof(int32_t));
  w.m = align256(w.o + n * g->head_dim * sizeof(float));
  w.l = align256(w.m + n * sizeof(float));
  w.end = align256(w.l + n * sizeof(float));
  return w;
}

struct PrefixIn {
  const int32_t* groups;  // [num_groups + 1]
  const int32_t* blocks;  // [num_groups]
  int32_t num_groups;
  int32_t max_prefix_blocks;
};

// pa_decode, pa_decode_scratch and pa_decode_shared_prefix.  pa_decode runs the multi-row
// (chunk) kernel on a second stream beside the decode kernel; use_scratch: both run on `st`,
// one after the other, in the static workspace (no stream or event is created).  pre: the
// shared-prefix kernel runs first, on `st`.
pa_status decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens,
                      const int32_t* query_start_loc, int32_t num_q_rows,
                      int32_t max_query_len, float scale, void* workspace,
                      size_t workspace_bytes, const pa_geom* g, hipStream_t st,
                      bool use_scratch, const PrefixIn* pre = nullptr);

}  // namespace

extern "C" {

const char* pa_status_str(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "inconsistent sizes";
    case PA_ERR_UNSUPPORTED: return "unsupported head_dim / block_size / dtype / group combination";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP launch failed";
    case PA_ERR_NO_BLOCKS: return "not enough free blocks in the pool";
  }
  return "unknown status";
}

size_t pa_kv_cache_bytes(const pa_geom* g) {
  if (check_geom(g) != PA_OK) return 0;
  return (size_t)g->num_blocks * g->num_kv_heads * g->head_dim * g->block_size *
         elem_bytes(g->kv_dtype);
}

pa_status pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                               const int64_t* slot_mapping, int64_t num_tokens,
                               const pa_geom* g, void* stream) {
  const pa_status gs = check_geom(g);
  if (gs != PA_OK) return gs;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
  const int64_t X = 16 / (int64_t)elem_bytes(g->kv_dtype);
  const int64_t threads = num_tokens * g->num_kv_heads * (g->head_dim / X + g->head_dim);
  if ((threads + 255) / 256 > 0x7fffffffLL) return PA_ERR_SHAPE;
  pa::ReshapeArgs a{key, value, k_cache, v_cache, slot_mapping, num_tokens, g->num_kv_heads,
                    g->head_dim, g->k_scale, g->v_scale, b8(g) ? 3 : 4};
  return hip_status(pa::launch_reshape(kdt(g), a, (hipStream_t)stream));
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping,
                         int64_t num_pairs, const pa_geom* g, void* stream) {
  const pa_status gs = check_geom(g);
  if (gs != PA_OK) return gs;
  if (num_pairs < 0) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_mapping) return PA_ERR_NULL;
  pa::CopyBlocksArgs a{};
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_mapping = block_mapping;
  a.num_pairs = num_pairs;
  a.block_bytes = (int64_t)g->num_kv_heads * g->block_size * g->head_dim * elem_bytes(g->kv_dtype);
  a.num_blocks = g->num_blocks;
  const int64_t pieces = (a.block_bytes + 16383) / 16384;
  if (num_pairs * 2 * pieces > 0x7fffffffLL) return PA_ERR_SHAPE;
  return hip_status(pa::launch_copy_blocks(a, (hipStream_t)stream));
}

pa_status pa_swap_blocks(void* k_cache, void* v_cache, void* host_k, void* host_v,
                         int64_t host_num_blocks, const int64_t* block_mapping,
                         int64_t num_pairs, int32_t direction, const pa_geom* g,
                         void* stream) {
  const pa_status gs = check_geom(g);
  if (gs != PA_OK) return gs;
  if (num_pairs < 0 || host_num_blocks < 0) return PA_ERR_SHAPE;
  if (direction != PA_SWAP_OUT && direction != PA_SWAP_IN) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !host_k || !host_v || !block_mapping) return PA_ERR_NULL;
  const bool out = direction == PA_SWAP_OUT;
  const int64_t src_n = out ? g->num_blocks : host_num_blocks;
  const int64_t dst_n = out ? host_num_blocks : g->num_blocks;
  for (int64_t p = 0; p < num_pairs; ++p) {
    const int64_t s = block_mapping[2 * p], d = block_mapping[2 * p + 1];
    if (s < 0 || s >= src_n || d < 0 || d >= dst_n) return PA_ERR_SHAPE;
  }
  const size_t bb = (size_t)g->num_kv_heads * g->block_size * g->head_dim * elem_bytes(g->kv_dtype);
  hipStream_t st = (hipStream_t)stream;

  // pinned host pools are mapped into the device's address space: one kernel per
  // kSwapPairs pairs moves every block over PCIe
  void* hk_dev = nullptr;
  void* hv_dev = nullptr;
  if (hipHostGetDevicePointer(&hk_dev, host_k, 0) == hipSuccess &&
      hipHostGetDevicePointer(&hv_dev, host_v, 0) == hipSuccess && hk_dev && hv_dev) {
    pa::SwapArgs a{};
    a.src_k = static_cast<const char*>(out ? k_cache : hk_dev);
    a.src_v = static_cast<const char*>(out ? v_cache : hv_dev);
    a.dst_k = static_cast<char*>(out ? hk_dev : k_cache);
    a.dst_v = static_cast<char*>(out ? hv_dev : v_cache);
    a.block_bytes = (int64_t)bb;
    for (int64_t p0 = 0; p0 < num_pairs; p0 += pa::kSwapPairs) {
      const int64_t n = std::min<int64_t>(pa::kSwapPairs, num_pairs - p0);
      a.num_pairs = (int32_t)n;
      for (int64_t i = 0; i < n; ++i) {
        a.pairs[i][0] = block_mapping[2 * (p0 + i)];
        a.pairs[i][1] = block_mapping[2 * (p0 + i) + 1];
      }
      if (pa::launch_swap_blocks(a, st) != hipSuccess) return PA_ERR_HIP;
    }
    return PA_OK;
  }
  (void)hipGetLastError();  // the failed lookup (pageable host memory) is not an error here

  // pageable host pools: one copy-engine transfer per run of consecutive ids
  const hipMemcpyKind kind = out ? hipMemcpyDeviceToHost : hipMemcpyHostToDevice;
  char* dk = static_cast<char*>(out ? host_k : k_cache);
  char* dv = static_cast<char*>(out ? host_v : v_cache);
  const char* sk = static_cast<const char*>(out ? k_cache : host_k);
  const char* sv = static_cast<const char*>(out ? v_cache : host_v);
  for (int64_t p = 0; p < num_pairs;) {
    const int64_t s = block_mapping[2 * p], d = block_mapping[2 * p + 1];
    int64_t n = 1;  // pairs continuing both runs
    while (p + n < num_pairs && block_mapping[2 * (p + n)] == s + n &&
           block_mapping[2 * (p + n) + 1] == d + n)
      ++n;
    hipError_t e = hipMemcpyAsync(dk + d * bb, sk + s * bb, n * bb, kind, st);
    if (e == hipSuccess) e = hipMemcpyAsync(dv + d * bb, sv + s * bb, n * bb, kind, st);
    if (e != hipSuccess) return PA_ERR_HIP;
    p += n;
  }
  return PA_OK;
}

size_t pa_workspace_size(const pa_geom* g, int32_t num_q_rows) {
  if (check_geom(g) != PA_OK || num_q_rows < 0) return 0;
  return decode_workspace_bytes(g, num_q_rows);
}

pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens,
                    const int32_t* query_start_loc, int32_t num_q_rows, int32_t max_query_len,
                    float scale, void* workspace, size_t workspace_bytes, const pa_geom* g,
                    void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                     num_q_rows, max_query_len, scale, workspace, workspace_bytes, g,
                     (hipStream_t)stream, false);
}

pa_status pa_decode_scratch(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            const int32_t* query_start_loc, int32_t num_q_rows,
                            int32_t max_query_len, float scale, const pa_geom* g,
                            void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                     num_q_rows, max_query_len, scale, nullptr, 0, g, (hipStream_t)stream, true);
}

size_t pa_shared_prefix_workspace_size(const pa_geom* g, int32_t num_q_rows,
                                       int32_t max_prefix_blocks) {
  if (check_geom(g) != PA_OK || num_q_rows < 0 || max_prefix_blocks < 0 ||
      max_prefix_blocks > g->max_blocks_per_seq)
    return 0;
  const size_t even = decode_workspace_bytes(g, num_q_rows, kSharedWgPerCu);
  return prefix_space(g, num_q_rows, even, prefix_parts(g, max_prefix_blocks)).end;
}

pa_status pa_decode_shared_prefix(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, const int32_t* query_start_loc,
                                  int32_t num_q_rows, int32_t max_query_len,
                                  const int32_t* prefix_groups, const int32_t* prefix_blocks,
                                  int32_t num_groups, int32_t max_prefix_blocks, float scale,
                                  void* workspace, size_t workspace_bytes, const pa_geom* g,
                                  void* stream) {
  const pa_status gs = check_geom(g);
  if (gs != PA_OK) return gs;
  if (num_groups < 0 || max_prefix_blocks < 0 || max_prefix_blocks > g->max_blocks_per_seq)
    return PA_ERR_SHAPE;
  if (num_groups > kMaxSeqs) return PA_ERR_UNSUPPORTED;
  if (num_groups > 0 && (!prefix_groups || !prefix_blocks)) return PA_ERR_NULL;
  // the prefix kernel is the chunk kernel's: 16-bit or FP8 pools, 16 % G == 0
  if (g->kv_dtype == PA_F32 || 16 % (g->num_q_heads / g->num_kv_heads) != 0)
    return PA_ERR_UNSUPPORTED;
  const PrefixIn pre{prefix_groups, prefix_blocks, num_groups, max_prefix_blocks};
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                     num_q_rows, max_query_len, scale, workspace, workspace_bytes, g,
                     (hipStream_t)stream, false, &pre);
}

}  // extern "C"

namespace {

pa_status decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens,
                      const int32_t* query_start_loc, int32_t num_q_rows,
                      int32_t max_query_len, float scale, void* workspace,
                      size_t workspace_bytes, const pa_geom* g, hipStream_t st,
                      bool use_scratch, const PrefixIn* pre) {
  const pa_status gs = check_geom(g);
  if (gs != PA_OK) return gs;
  if (num_q_rows < 0 || max_query_len < 0) return PA_ERR_SHAPE;
  if (!query_start_loc && num_q_rows != g->num_seqs) return PA_ERR_SHAPE;
  if (g->num_seqs == 0 || num_q_rows == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
  if (!std::isfinite(scale)) return PA_ERR_SHAPE;
  const int G = g->num_q_heads / g->num_kv_heads;
  if (query_start_loc && (g->kv_dtype == PA_F32 || 16 % G != 0)) return PA_ERR_UNSUPPORTED;

  // rows of the longest sequence: at most max_query_len (0: unknown) and num_q_rows
  int32_t max_len = 1;
  if (query_start_loc)
    max_len = max_query_len > 0 && max_query_len < num_q_rows ? max_query_len : num_q_rows;
  const Route rt = route(g, max_len);
  const int wg = pre ? kSharedWgPerCu : 0;
  const int grid = split_grid(g, pa::MODE_EVEN, rt.path, wg);
  const size_t even = even_workspace_bytes(g, rt, wg);
  const PrefixParts pp = pre ? prefix_parts(g, pre->max_prefix_blocks) : PrefixParts{};
  const bool prefix = pre && pre->num_groups > 0 && pp.parts > 0;
  const PrefixSpace ps = prefix_space(g, num_q_rows, even, pp);
  const size_t need = prefix ? ps.end : even;
  if (use_scratch) {
    if (need > kScratchBytes) return PA_ERR_WORKSPACE;
    workspace = scratch_ptr(current_device(), st);
    if (!workspace) return PA_ERR_HIP;
    workspace_bytes = kScratchBytes;
  }
  if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
  const size_t slots = even_slots(g, grid, rt, wg);
  int32_t* counters = static_cast<int32_t*>(workspace);
  float* part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + counter_bytes());
  float* part_m = part_o + slots * g->head_dim;
  float* part_l = part_m + slots;

  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.qsl = query_start_loc;
  a.part_o = part_o;
  a.part_m = part_m;
  a.part_l = part_l;
  a.counters = counters;
  a.num_seqs = g->num_seqs;
  a.num_q_heads = g->num_q_heads;
  a.num_kv_heads = g->num_kv_heads;
  a.head_dim = g->head_dim;
  a.max_blocks_per_seq = g->max_blocks_per_seq;
  a.out_f32 = g->out_dtype == PA_F32 && g->kv_dtype != PA_F32;
  a.scale_log2 = scale_to_log2(scale);
  if (g->kv_dtype == PA_FP8_E4M3) {
    // a stored element stands for its E4M3 value times the pool's scale
    a.scale_log2 *= g->k_scale;
    a.v_factor = g->v_scale;
  }
  a.seg_extra = seg_extra_override() >= 0 ? seg_extra_override() : seg_extra_default(g, rt.path);
  a.heads_per_wave = rt.path == 0 ? heads_per_wave(g, wg) : 1;
  a.xcd_major = xcd_major_override() > 0 ? 1 : 0;
  a.odd_skew = odd_skew(g, rt.path);
  a.max_rows = rt.max_rows;
  a.cols = rt.cols;
  a.blk_shift = blk_shift(g);
  a.b8 = b8(g);
  // no multi-row kernel runs: the rows of a sequence with more rows than max_query_len
  // promised are written NaN
  a.nan_rows = query_start_loc && max_len <= rt.max_rows ? 1 : 0;

  if (prefix) {
    // the groups' shared keys first: partials for every row of a group, and each sequence's
    // skip (the keys the decode kernel then leaves out and folds back from the partials)
    char* ws = static_cast<char*>(workspace);
    int32_t* skip = reinterpret_cast<int32_t*>(ws + ps.skip);
    float* pre_o = reinterpret_cast<float*>(ws + ps.o);
    float* pre_m = reinterpret_cast<float*>(ws + ps.m);
    float* pre_l = reinterpret_cast<float*>(ws + ps.l);
    pa::DecodeArgs pa_ = a;
    pa_.part_tokens = pp.tokens;
    pa_.max_partitions = pp.parts;
    pa_.part_o = pre_o;
    pa_.part_m = pre_m;
    pa_.part_l = pre_l;
    pa_.grp_start = pre->groups;
    pa_.grp_blocks = pre->blocks;
    pa_.num_groups = pre->num_groups;
    pa_.max_prefix_blocks = pre->max_prefix_blocks;
    pa_.block_size = g->block_size;
    pa_.skip_out = skip;
    if (pa::launch_prefix(kdt(g), pa_, num_q_rows, st) != hipSuccess) return PA_ERR_HIP;
    a.skip = skip;
    a.pre_o = pre_o;
    a.pre_m = pre_m;
    a.pre_l = pre_l;
    a.pre_parts = pp.parts;
    a.pre_tokens = pp.tokens;
  }

  auto decode = [&] {
    return rt.path ? pa::launch_mfma_decode(kdt(g), pa::MODE_EVEN, a, grid, st)
                   : pa::launch_valu_decode(kdt(g), pa::MODE_EVEN, a, grid, st);
  };
  // without query_start_loc, or when no sequence has more rows than the decode kernel takes,
  // there is no chunk work
  if (!query_start_loc || max_len <= rt.max_rows) return hip_status(decode());
  if (use_scratch) {
    // one stream: the chunk kernel, then the decode kernel
    const hipError_t ec = pa::launch_chunk(kdt(g), a, num_q_rows, st);
    if (ec != hipSuccess) return PA_ERR_HIP;
    return hip_status(decode());
  }
  // the chunk kernel runs beside the decode kernel: the lean matrix-core decode shares the CUs
  a.lean = 1;

  // multi-row sequences: the chunk kernel on the side stream, forked from and joined back
  // into the caller's stream around the decode kernel
  SideStream* side = side_stream(current_device());
  if (!side) return PA_ERR_HIP;
  std::lock_guard<std::mutex> lock(side->mu);
  hipError_t e = hipEventRecord(side->fork, st);
  if (e == hipSuccess) e = hipStreamWaitEvent(side->stream, side->fork, 0);
  if (e == hipSuccess) e = pa::launch_chunk(kdt(g), a, num_q_rows, side->stream);
  const hipError_t ed = decode();
  if (e == hipSuccess) e = hipEventRecord(side->join, side->stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(st, side->join, 0);
  return e == hipSuccess && ed == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

extern "C" {

pa_status pa_decode_partitioned(float* tmp_out, float* max_logits, float* exp_sums,
                                const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* context_lens,
                                const int32_t* query_start_loc, int32_t num_q_rows,
                                float scale, int32_t partition_size, int32_t max_partitions,
                                const pa_geom* g, void* stream) {
  const pa_status gs = check_geom(g);
  if (gs != PA_OK) return gs;
  if (num_q_rows < 0) return PA_ERR_SHAPE;
  if (!query_start_loc && num_q_rows != g->num_seqs) return PA_ERR_SHAPE;
  if (partition_size <= 0 || partition_size % pa::kMfmaUnit || max_partitions <= 0)
    return PA_ERR_SHAPE;
  if ((int64_t)max_partitions * partition_size < (int64_t)g->max_blocks_per_seq * g->block_size)
    return PA_ERR_SHAPE;
  if (g->num_seqs == 0 || num_q_rows == 0) return PA_OK;
  if (!tmp_out || !max_logits || !exp_sums || !q || !k_cache || !v_cache || !block_tables ||
      !context_lens)
    return PA_ERR_NULL;
  if (!std::isfinite(scale)) return PA_ERR_SHAPE;
  const int G = g->num_q_heads / g->num_kv_heads;
  if (query_start_loc && (g->kv_dtype == PA_F32 || 16 % G != 0)) return PA_ERR_UNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  pa::DecodeArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.qsl = query_start_loc;
  a.part_o = tmp_out;
  a.part_m = max_logits;
  a.part_l = exp_sums;
  a.num_seqs = g->num_seqs;
  a.num_q_heads = g->num_q_heads;
  a.num_kv_heads = g->num_kv_heads;
  a.head_dim = g->head_dim;
  a.max_blocks_per_seq = g->max_blocks_per_seq;
  a.scale_log2 = scale_to_log2(scale);
  if (g->kv_dtype == PA_FP8_E4M3) {
    a.scale_log2 *= g->k_scale;  // a stored key stands for its E4M3 value times k_scale
    a.v_factor = g->v_scale;
  }
  a.max_partitions = max_partitions;
  const bool mf = use_mfma(g);
  a.partition_units = partition_size / (mf ? pa::kMfmaUnit : pa::kValuUnit);
  a.max_rows = 1;
  a.cols = g->num_q_heads / g->num_kv_heads;
  a.blk_shift = blk_shift(g);
  a.b8 = b8(g);
  const int grid = split_grid(g, pa::MODE_PARTITION, mf ? 1 : 0);
  // sequences with one row: the decode kernel, which also marks every row's partitions past
  // its context
  hipError_t e = mf ? pa::launch_mfma_decode(kdt(g), pa::MODE_PARTITION, a, grid, st)
                    : pa::launch_valu_decode(kdt(g), pa::MODE_PARTITION, a, grid, st);
  if (e != hipSuccess || !query_start_loc) return hip_status(e);
  // sequences with several rows: the chunk kernel, one item per (column block, partition)
  a.part_tokens = partition_size;
  a.max_rows = 1;
  return hip_status(pa::launch_chunk(kdt(g), a, num_q_rows, st));
}

pa_status pa_decode_reduce(void* out, const float* tmp_out, const float* max_logits,
                           const float* exp_sums, int32_t num_q_rows, int32_t max_partitions,
                           const pa_geom* g, void* stream) {
  const pa_status gs = check_geom(g);
  if (gs != PA_OK) return gs;
  if (num_q_rows < 0 || max_partitions <= 0) return PA_ERR_SHAPE;
  if (num_q_rows == 0) return PA_OK;
  if (!out || !tmp_out || !max_logits || !exp_sums) return PA_ERR_NULL;
  pa::PartReduceArgs a{};
  a.out = out;
  a.tmp_out = tmp_out;
  a.max_logits = max_logits;
  a.exp_sums = exp_sums;
  a.num_items = (int64_t)num_q_rows * g->num_q_heads;
  a.head_dim = g->head_dim;
  a.max_partitions = max_partitions;
  a.out_f32 = g->out_dtype == PA_F32 && g->kv_dtype != PA_F32;
  // the merged rows take the queries' type (fp16 or bf16 behind FP8 pools) unless fp32
  return hip_status(pa::launch_part_reduce(g->q_dtype, a, (hipStream_t)stream));
}

}  // extern "C"
