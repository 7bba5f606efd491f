// chunk.hip — multi-row (chunked-prefill) attention over the paged cache.
//
// "vLLM 架构源码解析 第1篇" §1.1 runs a long prompt as 512-token chunks in the same step as
// other requests' decode rows, and §3.3.2 marks each request's rows with query_start_loc.
// A sequence s with n > 1 rows has its context_lens entry counting those rows (they were
// written by reshape_and_cache first, §3.3.3); row j sits at position ctx - n + j and attends
// keys [0, ctx - n + j] (causal).  Sequences with few rows (a decode row, or on the
// matrix-core path up to 16 / G rows, as in a speculative verify step) are left to the decode
// kernels.
//
// Work item = (sequence, KV head g, block of 128 query columns), a column being one (row,
// head) pair: 128 / G consecutive rows x the G query heads of g.  The workgroup stages each
// 32-token K/V unit in LDS once and its four waves each run 32 columns over it through the
// matrix-core step of pa_mfma.h, so one unit read from memory serves 128 columns.
//
// FP8 pools ("vLLM 深度拆解" §10.1) take the same path: each 8-byte half of an E4M3 chunk is
// widened to the query's 16-bit type (exact for every E4M3 value) on its way into LDS, where
// the unit then has the 16-bit layout; k_scale is in the score factor and v_scale multiplies
// the output.
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma.h"

namespace pa {

constexpr int kChunkBlocks = 2;                       // 16-column MFMA blocks per wave
constexpr int kWaveCols = 16 * kChunkBlocks;          // query columns per wave
constexpr int kItemCols = kWaveCols * kWavesPerWG;    // query columns per workgroup

template <int D>
struct ChunkTile {
  static constexpr int TILE = 16 * D * 2;                  // one block of one KV head, bytes
  static constexpr int UNIT = 4 * TILE;                    // K and V of a 32-token unit
  static constexpr int LOADS = UNIT / (kWG * 16);          // 16-byte loads per thread per unit
  static constexpr int CPT = TILE / 16;                    // 16-byte chunks per tile
};

struct ChunkPlanIn {
  const int32_t* qsl;
  int32_t num_seqs;
  int32_t rows_per_item;
  int32_t min_rows;  // sequences with fewer rows are the decode kernel's
};

// work items per sequence: ceil(n / rows_per_item) for sequences of at least min_rows rows,
// else 0
__device__ inline void build_chunk_plan(int32_t* base, const ChunkPlanIn& p) {
  wave_plan(base, p.num_seqs, [&](int s) {
    const int32_t n = p.qsl[s + 1] - p.qsl[s];
    return n >= p.min_rows ? (n + p.rows_per_item - 1) / p.rows_per_item : 0;
  });
}

// One work item: rows [j0, j0 + kItemCols / G) of multi-row sequence s for KV head g.  The
// workgroup streams the item's keys in 32-token units: every unit (K and V of two blocks) is
// loaded once by the whole workgroup, two units ahead, into one of two LDS buffers, and each
// wave then runs its 32 query columns (two 16-column MFMA blocks, per-column causal limits)
// over it.  DT is the 16-bit type of the queries and of the staged unit; F8: the pools hold
// E4M3 bytes.
template <int DT, int D, bool F8>
__device__ void chunk_item(const DecodeArgs& a, int s, int g, int cb, char* lds_units) {
  using C = MfmaCfg<DT, D>;
  using CT = ChunkTile<D>;
  using T = op8_t<DT>;
  constexpr int NCB = kChunkBlocks;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int r = lane >> 4, n = lane & 15;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int q0 = __builtin_amdgcn_readfirstlane(a.qsl[s]);
  const int nrows = __builtin_amdgcn_readfirstlane(a.qsl[s + 1]) - q0;
  const int ctx = __builtin_amdgcn_readfirstlane(a.context_lens[s]);
  const int RW = kWaveCols / G;                    // rows per wave
  const int j0g = cb * (kItemCols / G);            // first row of the workgroup
  const int jendg = min(nrows, j0g + kItemCols / G);
  const int j0 = j0g + wave * RW;                  // first row of this wave
  const int jend = min(jendg, j0 + RW);
  const int nkeys_g = ctx - nrows + jendg;         // keys any column of the item may see
  const int nkeys_w = jend > j0 ? ctx - nrows + jend : 0;  // ... of this wave's columns

  T qb[NCB][C::NKK];
  int pos[NCB];     // this lane's column's last visible key (-1: column past the rows)
  int first[NCB];   // smallest last-visible key over the block's columns (uniform)
  bool full[NCB];   // every column of the block is a real row (uniform)
  bool live[NCB];   // the block has a real row (uniform)
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    const int col = 16 * c + n;
    const int jc = j0 + col / G, hc = col % G;
    const bool ok = jc < jend;
    pos[c] = ok ? ctx - nrows + jc : -1;
    first[c] = ctx - nrows + j0 + (16 * c) / G;
    full[c] = j0 + (16 * c + 15) / G < jend;
    live[c] = j0 + (16 * c) / G < jend;
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     ((int64_t)(q0 + jc) * a.num_q_heads + (int64_t)g * G + hc) * D * C::E;
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
      const uint4 v = ok ? ld16(qp + (4 * kk + r) * 16) : make_uint4(0, 0, 0, 0);
      qb[c][kk] = __builtin_bit_cast(T, v);
    }
  }
  MfmaState<DT, D> st[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    st[c].m = -INFINITY;
    st[c].l = 0.f;
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) st[c].acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const MfmaLaneOffsets<DT, D> o = mfma_offsets<DT, D>();
  constexpr int64_t PTILE = F8 ? C::TILE / 2 : C::TILE;  // a block of one KV head in the pool
  const int64_t blk_stride = (int64_t)a.num_kv_heads * PTILE;
  const char* kc = reinterpret_cast<const char*>(a.k_cache) + (int64_t)g * PTILE;
  const char* vc = reinterpret_cast<const char*>(a.v_cache) + (int64_t)g * PTILE;
  const int32_t* bt_row = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int nblk = (nkeys_g + kBlock - 1) / kBlock;
  const int nu = (nkeys_g + kMfmaUnit - 1) / kMfmaUnit;

  // this thread's share of a unit: chunk k * kWG + threadIdx.x of the four tiles
  // [K block a, K block b, V block a, V block b]
  // (16-bit chunk c of a tile; FP8: its 8 source bytes, half of E4M3 K chunk
  // (c / 32) * 16 + c % 16, or bytes 8c.. of the V tile)
  int ld_tile[CT::LOADS], ld_off[CT::LOADS], src_off[CT::LOADS];
#pragma unroll
  for (int k = 0; k < CT::LOADS; ++k) {
    const int c = k * kWG + threadIdx.x;
    ld_tile[k] = c / CT::CPT;
    const int cc = c % CT::CPT;
    ld_off[k] = cc * 16;
    if constexpr (F8)
      src_off[k] = ld_tile[k] & 2 ? cc * 8 : (((cc >> 5) << 4) + (cc & 15)) * 16 + 8 * ((cc >> 4) & 1);
    else
      src_off[k] = cc * 16;
  }
  using Raw = typename std::conditional<F8, uint2, uint4>::type;
  constexpr int WDT = DT == DT_BF16 ? DT_FP8B : DT_FP8;  // widening of FP8 staged bytes
  int win0 = 0, win1 = 0, wbase = -1;  // block-table windows of 64 entries: [wbase, wbase + 128)
  auto load_unit = [&](Raw* regs, int u) {
    const int e = 2 * u;
    if (wbase < 0 || e >= wbase + 128) {  // uniform; happens every 64 units
      wbase = e;
      win0 = (e + lane < nblk) ? tile_block(bt_row, e + lane, a.blk_shift) : 0;
      win1 = (e + 64 + lane < nblk) ? tile_block(bt_row, e + 64 + lane, a.blk_shift) : 0;
    }
    const int ia = e - wbase;
    const int64_t ba = ia < 64 ? readlane(win0, ia) : readlane(win1, ia - 64);
    // a second block past the keys is replaced by the first (its tokens are masked)
    const int64_t bb = e + 1 < nblk ? (ia + 1 < 64 ? readlane(win0, ia + 1) : readlane(win1, ia + 1 - 64)) : ba;
#pragma unroll
    for (int k = 0; k < CT::LOADS; ++k) {
      const int t = ld_tile[k];
      const char* base = (t & 2 ? vc : kc) + (t & 1 ? bb : ba) * blk_stride;
      regs[k] = *reinterpret_cast<const Raw*>(base + src_off[k]);
    }
  };
  auto store_unit = [&](const Raw* regs, int buf) {
#pragma unroll
    for (int k = 0; k < CT::LOADS; ++k) {
      uint4 v;
      if constexpr (F8)
        v = __builtin_bit_cast(uint4, operand<WDT>(regs[k]));
      else
        v = regs[k];
      *reinterpret_cast<uint4*>(lds_units + buf * CT::UNIT + ld_tile[k] * CT::TILE + ld_off[k]) = v;
    }
  };

  // Unit pipeline: the loads of unit u + 2 go out at the start of step u, unit u is computed
  // from LDS buffer u % 2, and unit u + 1 (loaded since the start of step u - 1, so two
  // compute phases ago) is stored into the other buffer at the end of the step.  Even units
  // are staged in ra, odd ones in rb.  Loads and stores run on every step (past the last unit
  // they repeat it and the result is never read), and the barrier between steps does not wait
  // for outstanding loads, so the compiler's wait before each store covers only that unit.
  auto barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  const int ulast = nu - 1;
  auto compute = [&](int u) {
    const int t0 = u * kMfmaUnit;
    if (u < nu && t0 < nkeys_w) {  // uniform: this wave's columns see keys of this unit
      const char* ub = lds_units + (u & 1) * CT::UNIT;
      // scores of both column blocks from K, then P . V from V: K and V are never live together
      MfmaK<DT, D> kb;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk)
          kb[b][kk] = *reinterpret_cast<const uint4*>(ub + o.kt[b] * CT::TILE + o.koff(b, kk));
      bool masked[NCB];
      MfmaP<DT> pp[NCB];
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        masked[c] = !(t0 + kMfmaUnit - 1 <= first[c] && full[c]);
        if (!live[c]) continue;
        if (!masked[c])
          pp[c] = mfma_scores<DT, D, false, true>(st[c], kb, qb[c], a.scale_log2, kMfmaUnit - 1);
        else
          pp[c] = mfma_scores<DT, D, true, true>(st[c], kb, qb[c], a.scale_log2, pos[c] - t0);
      }
      MfmaV<DT, D> vb;
#pragma unroll
      for (int j = 0; j < C::NJ; ++j)
        vb[j] = *reinterpret_cast<const uint4*>(ub + (2 + o.vt) * CT::TILE + o.voff(j));
      // V is masked in place for the first block that needs it; the masked tokens are the
      // same for every column, so later blocks may use it either way
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        if (!live[c]) continue;
        if (!masked[c])
          mfma_pv<DT, D, false>(st[c], vb, pp[c], kMfmaUnit);
        else
          mfma_pv<DT, D, true>(st[c], vb, pp[c], nkeys_g - t0);
      }
    }
  };
  Raw ra[CT::LOADS], rb[CT::LOADS];
  load_unit(ra, 0);
  load_unit(rb, min(1, ulast));
  store_unit(ra, 0);
  barrier();
  for (int u = 0; u < nu; u += 2) {
    load_unit(ra, min(u + 2, ulast));
    compute(u);
    store_unit(rb, 1);
    barrier();
    load_unit(rb, min(u + 3, ulast));
    compute(u + 1);
    store_unit(ra, 0);
    barrier();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the repeated loads past the last unit

  // emit: lane (r, n) holds dimensions 16 j + 4 r + i of column 16 c + n, which is
  // (row j0 + col / G, head col % G)
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    const float ltot = cross_rows_sum(st[c].l);
    // FP8: a stored V value stands for its E4M3 value times v_scale
    const float inv = ltot > 0.f ? (F8 ? a.v_factor : 1.f) / ltot : 0.f;
    const int col = 16 * c + n;
    const int jr = j0 + col / G, hr = col % G;
    if (jr < jend) {
      const int64_t ob = ((int64_t)(q0 + jr) * a.num_q_heads + (int64_t)g * G + hr) * D;
#pragma unroll
      for (int j = 0; j < C::NJ; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          store_out<DT>(a.out, ob + 16 * j + 4 * r + i, st[c].acc[j][i] * inv, a.out_f32);
    }
  }
}

// Most multi-row sequences whose items are ordered longest first (see chunk_kernel).
constexpr int kMaxOrdered = 256;

// Work items, one per workgroup.  Items differ in length by up to the longest context over
// the shortest, and workgroups start in index order as earlier ones finish, so the items are
// numbered longest first: multi-row sequences by decreasing number of prior keys, within a
// sequence column blocks last to first (the longest causal ranges first), and the KV heads
// of one (sequence, column block) consecutively.  With more than kMaxOrdered multi-row
// sequences the items keep the sequence order instead, KV head slowest, numbered XCD-locally
// so that each XCD works through mostly one KV head.
template <int DT, int D, bool F8>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(2))) void chunk_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) char lds_raw[];
  char* lds_units = lds_raw;  // two unit buffers
  int32_t* base = reinterpret_cast<int32_t*>(lds_raw + 2 * ChunkTile<D>::UNIT);
  int32_t* order = base + a.num_seqs + 1;  // [kMaxOrdered] multi-row sequences, longest first
  int32_t* rbase = order + kMaxOrdered;    // [kMaxOrdered + 1] item prefix in that order
  int32_t* pkeys = rbase + kMaxOrdered + 1;  // [kMaxOrdered] prior keys of order[] entries
  int32_t* count = pkeys + kMaxOrdered;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int S = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  ChunkPlanIn pin{a.qsl, S, kItemCols / G, a.max_rows + 1};
  build_chunk_plan(base, pin);
  const int64_t per_head = base[S];
  const int64_t total = per_head * Hkv;

  // collect the multi-row sequences (any order), then rank them by prior keys (ties: index)
  if (threadIdx.x == 0) *count = 0;
  __syncthreads();
  for (int t = threadIdx.x; t < S; t += kWG) {
    if (base[t + 1] > base[t]) {
      const int slot = atomicAdd(count, 1);
      if (slot < kMaxOrdered) {
        order[slot] = t;
        pkeys[slot] = a.context_lens[t] - (a.qsl[t + 1] - a.qsl[t]);
      }
    }
  }
  __syncthreads();
  const int M = *count;
  const bool ordered = M <= kMaxOrdered;
  if (ordered) {
    int mine = -1, rank = 0;
    if (threadIdx.x < M) {
      mine = order[threadIdx.x];
      const int pm = pkeys[threadIdx.x];
      for (int k = 0; k < M; ++k) {
        const int o = order[k], po = pkeys[k];
        rank += (po > pm || (po == pm && o < mine)) ? 1 : 0;
      }
    }
    __syncthreads();
    if (mine >= 0) order[rank] = mine;
    __syncthreads();
    wave_plan(rbase, M, [&](int r) { return (base[order[r] + 1] - base[order[r]]) * Hkv; });
  }

  for (int64_t i = ordered ? (int64_t)blockIdx.x : xcd_local_block(blockIdx.x, gridDim.x);
       i < total; i += gridDim.x) {
    int s, g, cb;
    if (ordered) {
      const int rk = find_seq(rbase, M, i, 1);
      s = order[rk];
      const int k = (int)(i - rbase[rk]);
      const int nb = base[s + 1] - base[s];
      cb = nb - 1 - k / Hkv;
      g = k % Hkv;
    } else {
      g = (int)(i / per_head);
      const int64_t k = i - (int64_t)g * per_head;
      s = find_seq(base, S, k, 1);
      const int nb = base[s + 1] - base[s];
      cb = nb - 1 - (int)(k - base[s]);
    }
    chunk_item<DT, D, F8>(a, s, g, cb, lds_units);
    __syncthreads();  // the unit buffers are reused by the next item
  }
}

template <int DT, bool F8>
static hipError_t launch_c(const DecodeArgs& a, int grid, size_t lds, hipStream_t st) {
  if (a.head_dim == 64)
    hipLaunchKernelGGL((chunk_kernel<DT, 64, F8>), dim3(grid), dim3(kWG), lds, st, a);
  else
    hipLaunchKernelGGL((chunk_kernel<DT, 128, F8>), dim3(grid), dim3(kWG), lds, st, a);
  return hipGetLastError();
}

// dt: DT_F16 / DT_BF16 pools, or DT_FP8 / DT_FP8B (FP8 pools behind fp16 / bf16 queries)
hipError_t launch_chunk(int dt, const DecodeArgs& a, int num_q_rows, hipStream_t st) {
  // one workgroup per work item: at most ceil(rows / rows_per_item) + num_seqs items per KV
  // head; a multiple of the XCD count keeps the XCD-local numbering on
  const int rpi = kItemCols / (a.num_q_heads / a.num_kv_heads);
  const int64_t items = ((int64_t)(num_q_rows + rpi - 1) / rpi + a.num_seqs) * a.num_kv_heads;
  const int64_t wgs = (items + kXcds - 1) / kXcds * kXcds;
  const int grid = (int)(wgs < (1 << 20) ? wgs : (1 << 20) / kXcds * kXcds);
  const size_t lds = (size_t)2 * (a.head_dim == 64 ? ChunkTile<64>::UNIT : ChunkTile<128>::UNIT) +
                     (size_t)(a.num_seqs + 1 + 3 * kMaxOrdered + 2) * sizeof(int32_t);
  if (grid <= 0) return hipSuccess;
  if (dt == DT_F16) return launch_c<DT_F16, false>(a, grid, lds, st);
  if (dt == DT_BF16) return launch_c<DT_BF16, false>(a, grid, lds, st);
  if (dt == DT_FP8) return launch_c<DT_F16, true>(a, grid, lds, st);
  return launch_c<DT_BF16, true>(a, grid, lds, st);
}

}  // namespace pa
