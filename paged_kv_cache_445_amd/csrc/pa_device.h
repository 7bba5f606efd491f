// pa_device.h — device-side helpers shared by the gfx950 kernels of libpa.so.
//
// Pool layout (the ABI of include/pa.h): elem E bytes, X = 16 / E elements per 16-byte chunk,
//   K tile of (16-token sub-block, kv_head): [D / X chunks][16 tokens][X]   = 16 * D * E bytes
//   V tile of (16-token sub-block, kv_head): [D dims][16 tokens]            = 16 * D * E bytes
// Tiles of consecutive kv heads of one sub-block are adjacent; a block of 16 R tokens is R
// consecutive sub-blocks.  The kernels address sub-blocks ("blocks" below: 16 tokens).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "pa_internal.h"

namespace pa {

template <int DT>
struct DtInfo {
  static constexpr int bytes = DT == DT_F32 ? 4 : is_fp8(DT) ? 1 : 2;  // pool element
  static constexpr int x = 16 / bytes;  // elements per 16-byte chunk
  static constexpr int qbytes = DT == DT_F32 ? 4 : 2;  // query / key / value / out element
};

typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf162_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---------------------------------------------------------------- block table

// Pool sub-block of a sequence's 16-token tile j.  A block of 16 R tokens (R = 1 << shift) is
// R consecutive 16-token sub-blocks of the pool, so table entry j >> shift names sub-blocks
// R * entry .. R * entry + R - 1 and tile j is the (j mod R)-th of them.  shift = 0: the
// table entry itself.
__device__ __forceinline__ int32_t tile_block(const int32_t* bt_row, int j, int shift) {
  return (bt_row[j >> shift] << shift) | (j & ((1 << shift) - 1));
}

// Block-table window of a sequence's 16-token tiles [c0, c1), c1 - c0 <= (B8 ? 64 : 128),
// held one entry per lane in two registers.  16-token tiles: w0 = entry for tile c0 + lane,
// w1 = tile c0 + 64 + lane (sub-block ids, tile_block).  8-token blocks (B8): tile j is blocks
// 2 j and 2 j + 1, so w0 / w1 hold the block ids of entries 2 c0 + lane / 2 c0 + 64 + lane;
// entries at or past the context's last block (ceil(ctx / 8)) are never read and hold 0
// (their tokens are masked).  Outside the window's range the registers hold 0.
template <bool B8>
__device__ __forceinline__ void load_window(const int32_t* bt_row, int c0, int c1, int ctx,
                                            int shift, int& w0, int& w1) {
  const int lane = __lane_id();
  if constexpr (B8) {
    const int e0 = 2 * c0, eend = min(2 * c1, (ctx + 7) >> 3);
    w0 = e0 + lane < eend ? bt_row[e0 + lane] : 0;
    w1 = e0 + 64 + lane < eend ? bt_row[e0 + 64 + lane] : 0;
  } else {
    w0 = (c0 + lane < c1) ? tile_block(bt_row, c0 + lane, shift) : 0;
    w1 = (c0 + 64 + lane < c1) ? tile_block(bt_row, c0 + 64 + lane, shift) : 0;
  }
}

// ---------------------------------------------------------------- 16-byte global loads

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// A streaming (non-temporal) 16-byte load, for the K and V tiles of the decode kernels: every
// tile is read once per call, and loads that allocate normally in L2 and the last-level
// cache cost the LLaMA-7B decode 11 % (106.8 -> 95.4 us with this policy).
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_nt;
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

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

// ---------------------------------------------------------------- FP8 E4M3
//
// E4M3 ("E4M3FN": bias 7, 3 fraction bits, no infinity, S.1111.111 NaN, largest finite 448).
// gfx950's v_cvt_pk_f32_fp8 widens two E4M3 bytes of a word (bytes 0-1, or 2-3 with the
// word select) to two exact fp32 values in this format; checked on all 256 codes, NaN
// included.
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

// the four E4M3 bytes of w as fp32, byte k in f[k]
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float (&f)[4]) {
  const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = lo[0];
  f[1] = lo[1];
  f[2] = hi[0];
  f[3] = hi[1];
}

// gfx950's v_cvt_scalef32_pk_{f16,bf16}_fp8 widens two E4M3 bytes of a word (bytes 0-1, or
// 2-3 with HI) straight to two 16-bit values, times the scale's power of two (1 here): one
// instruction per pair.  fp16 and bf16 both hold every E4M3 value (subnormals included)
// exactly.
template <bool BF16, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_16(uint32_t w) {
  if constexpr (BF16)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, HI));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, HI));
}

// The E4M3 code of an fp32 value: round to nearest, ties to even; magnitudes from 448 up
// saturate to 448, NaN stays NaN.  Bit arithmetic on the fp32 encoding.
__device__ __forceinline__ uint32_t f32_to_fp8(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7Fu;  // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // >= 448 (and infinity): saturate
  if (a < 0x3C800000u) {                      // below 2^-6: multiples of 2^-9
    // a * 2^9 is exact (a power-of-two factor); rintf rounds half to even; 8 is the
    // smallest normal number, code 0x08
    return sign | (uint32_t)rintf(__uint_as_float(a) * 512.0f);
  }
  const uint32_t e = (a >> 23) - 127 + 7;    // biased E4M3 exponent, 1..15
  uint32_t q = (a >> 20) & 7u;                // top three fraction bits
  const uint32_t rest = a & 0xFFFFFu;         // the 20 bits below them
  if (rest > 0x80000u || (rest == 0x80000u && (q & 1u))) ++q;  // to nearest, ties to even
  return sign | ((e << 3) + q);               // q = 8 carries into the exponent
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

// store one output element in the output dtype (round to nearest even for 16-bit; FP8
// pools have the outputs of their queries: fp16 or bf16)
template <int DT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v, bool out_f32) {
  if (out_f32 || DT == DT_F32) {
    reinterpret_cast<float*>(out)[idx] = v;
  } else if constexpr (DT == DT_F16 || DT == DT_FP8) {
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

// v[l] + v[l ^ 16] and v[l] + v[l ^ 32] through the gfx950 lane-swap instructions:
// v_permlane16_swap exchanges the odd rows of its first operand with the even rows of its
// second, v_permlane32_swap the upper half of the first with the lower half of the second.
// With both operands equal to v, the two results hold v and its partner lane's value.
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// sum / max over lanes {l, l^16, l^32, l^48}: the four DPP rows
__device__ __forceinline__ float cross_rows_sum(float v) { return xor32_sum(xor16_sum(v)); }
__device__ __forceinline__ float cross_rows_max(float v) { return xor32_max(xor16_max(v)); }

__device__ __forceinline__ int readlane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float readlane(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// ---------------------------------------------------------------- XCD-aware numbering
//
// The dispatcher hands consecutive workgroups to the 8 XCDs in turn (workgroup b runs on
// XCD b % 8), and each XCD has its own L2.  Renumbering b -> (b % 8) * ceil(n / 8) + b / 8
// makes consecutive logical workgroups share an XCD, so work that re-reads the same K/V
// (neighbouring logical workgroups) finds it in one L2.  The map is a bijection of
// [0, n) whenever n % 8 == 0 and is the identity otherwise; it only affects locality.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_local_block(int b, int n) {
  if (n % kXcds) return b;
  return (b % kXcds) * (n / kXcds) + b / kXcds;
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
  int32_t extra;       // balancing units appended to every non-empty segment (no work)
  int32_t max_rows;    // sequences with more query rows are left to the chunk kernel
  const int32_t* skip = nullptr;  // leading keys of each sequence attended elsewhere (a
                                  // multiple of unit_tokens, below the context), or NULL
};

// units of sequence s in the flattened list: its real units ceil(ctx / unit_tokens), plus
// `extra` trailing units that stand for the cost of starting a piece (a share that takes a
// segment boundary gets that many fewer real units; a share that starts inside them has
// nothing to do for that segment)
__device__ __forceinline__ int32_t seq_units(const PlanIn& p, int s) {
  const int32_t rows = p.qsl ? p.qsl[s + 1] - p.qsl[s] : 1;
  if (rows < 1 || rows > p.max_rows) return 0;  // no rows, or rows for the chunk kernel
  const int32_t ctx = p.context_lens[s] - (p.skip ? p.skip[s] : 0);
  return ctx > 0 ? (ctx + p.unit_tokens - 1) / p.unit_tokens + p.extra : 0;
}

// Decode rows (sequences with one query row) whose context is empty get a zero output.
// nan_rows: no kernel of the call takes sequences with more than p.max_rows rows, whose rows
// are written NaN instead of being left as they were.  Wave w of W handles sequences w,
// w + W, ...
template <int DT>
__device__ void zero_empty_rows(const PlanIn& p, void* out, int Hq, int D, int64_t w, int64_t W,
                                bool out_f32, bool nan_rows) {
  for (int64_t s = w; s < p.num_seqs; s += W) {
    const int32_t rows = p.qsl ? p.qsl[s + 1] - p.qsl[s] : 1;
    const bool empty = rows == 1 && p.context_lens[s] <= 0;
    const bool lost = nan_rows && rows > p.max_rows;
    if (!empty && !lost) continue;
    const int64_t row = p.qsl ? p.qsl[s] : s;
    const float v = empty ? 0.f : __builtin_nanf("");
    for (int64_t e = __lane_id(); e < (int64_t)rows * Hq * D; e += kWave)
      store_out<DT>(out, row * Hq * D + e, v, out_f32);
  }
}

// pa_decode_partitioned: the partitions of a row that lie past its sequence's context get
// max_logits = -inf and exp_sums = 0 (the row's partitions [0, ceil(ctx / part_tokens)) are
// written by whichever kernel computes the row).  Rows are (row, head, partition) blocks of
// Hq * P entries; wave w of W handles rows w, w + W, ... of the num_rows rows, each row's
// sequence found by a binary search over qsl (NULL: row r is sequence r).
__device__ inline void fill_past_partitions(const int32_t* context_lens, const int32_t* qsl,
                                            int S, int64_t num_rows, int Hq, int P,
                                            int part_tokens, float* pm, float* pl, int64_t w,
                                            int64_t W) {
  for (int64_t row = w; row < num_rows; row += W) {
    int s = (int)row;
    if (qsl) {  // the largest s with qsl[s] <= row
      int lo = 0, hi = S - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (qsl[mid] <= row)
          lo = mid;
        else
          hi = mid - 1;
      }
      s = lo;
    }
    const int np = (context_lens[s] + part_tokens - 1) / part_tokens;
    if (np >= P) continue;
    float* m = pm + row * Hq * P;
    float* l = pl + row * Hq * P;
    for (int e = __lane_id(); e < Hq * P; e += kWave) {
      if (e % P >= np) {
        m[e] = -INFINITY;
        l[e] = 0.f;
      }
    }
  }
}

// Exclusive prefix sums of units(s) over s < S into base[0..S] (LDS): the first wave of the
// workgroup reads 256 sequences at a time (four independent loads per lane) and scans them
// with lane shuffles; one barrier publishes the result.  Must be called by every thread.
template <class Units>
__device__ inline void wave_plan(int32_t* base, int S, Units&& units) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int32_t run = 0;
    for (int c = 0; c < S; c += 4 * kWave) {
      int32_t u[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int s = c + k * kWave + lane;
        u[k] = s < S ? units(s) : 0;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        int32_t incl = u[k];
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
          const int32_t v = __shfl_up(incl, d, kWave);
          if (lane >= d) incl += v;
        }
        const int s = c + k * kWave + lane;
        if (s < S) base[s] = run + incl - u[k];
        run += __shfl(incl, kWave - 1, kWave);
      }
    }
    if (lane == 0) base[S] = run;
  }
  __syncthreads();
}

// base[0..S] in LDS: exclusive prefix sums of seq_units.  Must be called by all threads.
__device__ inline void build_plan(int32_t* base, const PlanIn& p) {
  wave_plan(base, p.num_seqs, [&](int s) { return seq_units(p, s); });
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

// The flattened work list [0, total) is split over the NK workgroups that get work
// (NK = min(workgroups, total)): workgroup ("owner") o owns [part_lo(o), part_lo(o + 1)),
// and wave i of it takes head i of every group of that range.  Shares are proportional to
// a weight per owner.  Workgroups are dispatched to the XCDs round robin (workgroup b runs
// on XCD b mod 8), and on gfx950 the odd XCDs stream this access pattern measurably slower
// than the even ones, so owners on odd XCDs get slightly less work; the weights stay equal
// unless every share keeps at least four units, which keeps every share non-empty.
//  - identity mapping: owner o is workgroup o, on XCD o mod 8; weights alternate per owner.
//  - XCD-major mapping (xcd): owner o is the workgroup b with xcd_local_block(b) = o, so
//    owners [x B, (x + 1) B) (B = NK / 8) all run on XCD x and consecutive stretches of the
//    list stay on one XCD (and in its L2); weights alternate per block of B owners.  Used
//    only when every workgroup is an owner and their count is a multiple of 8.
struct Part {
  int64_t total;   // units
  int64_t NK;      // owners
  int64_t we, wo;  // weights of owners on even and odd XCDs
  int64_t B;       // owners per weight block (1, or NK / 8 with xcd)
  bool xcd;        // XCD-major owner mapping
};

// odd_skew: per mille taken from odd owners' weights and given to even owners'
__device__ __forceinline__ Part make_part(int64_t total, int64_t workgroups, int odd_skew,
                                          bool xcd_major = false) {
  Part p;
  p.total = total;
  p.NK = min(workgroups, total);
  const bool skew = odd_skew > 0 && odd_skew < 500 && total >= 4 * p.NK;
  p.we = skew ? 1000 + odd_skew : 1000;
  p.wo = skew ? 1000 - odd_skew : 1000;
  p.xcd = xcd_major && p.NK == workgroups && workgroups % kXcds == 0;
  p.B = p.xcd ? p.NK / kXcds : 1;
  return p;
}

// summed weight of owners [0, o): f whole blocks of B owners (alternately even and odd
// XCDs), then rem owners of block f
__device__ __forceinline__ int64_t part_weight(const Part& p, int64_t o) {
  const int64_t f = o / p.B, rem = o - f * p.B;
  const int64_t even = ((f + 1) >> 1) * p.B + ((f & 1) ? 0 : rem);
  const int64_t odd = (f >> 1) * p.B + ((f & 1) ? rem : 0);
  return even * p.we + odd * p.wo;
}

// first unit of owner o (o in [0, NK]; part_lo(NK) == total)
__device__ __forceinline__ int64_t part_lo(const Part& p, int64_t o) {
  return p.NK ? p.total * part_weight(p, o) / part_weight(p, p.NK) : 0;
}
// owner of unit u (u < total): the largest o with part_lo(o) <= u, i.e. with
// part_weight(o) <= X below
__device__ __forceinline__ int64_t part_owner(const Part& p, int64_t u) {
  const int64_t X = ((u + 1) * part_weight(p, p.NK) - 1) / p.total;
  const int64_t pair = p.B * (p.we + p.wo);  // an even block and the odd one after it
  const int64_t m = X / pair, r = X - m * pair;
  const int64_t j = r < p.B * p.we ? r / p.we : p.B + (r - p.B * p.we) / p.wo;
  return min(2 * m * p.B + j, p.NK - 1);
}

// Split-segment bookkeeping.  A segment (one sequence and head group) whose real units
// [seg0, seg1] cross an owner boundary has one piece in each owner o0..o1 (o0 = owner of
// seg0, o1 = owner of seg1); wave i's piece of owner o sits in partial slot
// 2 (4o + i) + 0 when it is the first piece of o's range and + 1 otherwise (only o0's piece
// can be a later piece).  Every owner has at most one segment that starts in its range and
// continues past it, so counter 4 o0 + i of the workspace belongs to that segment alone.
struct SplitSeg {
  int64_t k0, k1;  // first and last owner
  bool k0_later;   // k0's piece is not the first piece of k0's range
  int wave;        // wave index inside the workgroups (the head within the group)
};

__device__ __forceinline__ SplitSeg split_seg(const Part& p, int64_t seg0, int64_t seg1,
                                              int wave) {
  SplitSeg r;
  r.k0 = part_owner(p, seg0);
  r.k1 = part_owner(p, seg1);
  r.k0_later = part_lo(p, r.k0) < seg0;
  r.wave = wave;
  return r;
}

__device__ __forceinline__ int64_t piece_slot(const SplitSeg& sg, int64_t k) {
  return 2 * (kWavesPerWG * k + sg.wave) + ((k == sg.k0 && sg.k0_later) ? 1 : 0);
}

// Runs the workgroup's share: range(o, lo, hi) processes owner o's units, every wave its
// own head.
template <class F>
__device__ __forceinline__ void even_split_drive(const Part& p, F&& range) {
  const int64_t k = p.xcd ? xcd_local_block(blockIdx.x, gridDim.x) : blockIdx.x;
  if (k < p.NK) range(k, part_lo(p, k), part_lo(p, k + 1));
}

// ---- in-kernel merge of split segments ----
// The pieces of a split segment are computed by different workgroups, often on different
// XCDs, whose L2 caches are not kept coherent with each other.  A piece therefore publishes
// its partial (softmax-normalised o, max m in the natural-log domain, sum l) with
// device-scope stores (cache policy sc1: written through to the device's point of
// coherence, and counted as done only once they are there), waits for them to complete, and
// then arrives at the segment's counter with a device-scope atomic add.  The piece that
// arrives last (or that finds every other piece already arrived) reads the others back with
// device-scope loads, which never hit a stale L2 line, merges them with its own registers
// and writes the output.  This is a release/acquire handshake restricted to the data it
// orders, so no L2 of the device is written back or invalidated as a whole.  The merging
// wave returns the counter to zero, which keeps a workspace ready for the next call.
constexpr int kCohPolicy = 16;  // buffer-op cache policy: sc1 (device scope), as the
                                // compiler gives device-scope atomic loads and stores

// single floats through 64-bit addresses
__device__ __forceinline__ float coh_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coh_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// four consecutive floats at element offset e (< 2^29) of a wave-uniform base, as one
// buffer access
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coh_rsrc(const float* base) {
  // raw buffer: stride 0, the largest record count, 32-bit data format
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ f32x4_t coh_load4(const float* base, int e) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(coh_rsrc(base), 4 * e, 0, kCohPolicy));
}
__device__ __forceinline__ void coh_store4(float* base, int e, f32x4_t v) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), coh_rsrc(base), 4 * e, 0, kCohPolicy);
}

// Device-scope read of a segment counter (every lane gets the value; not yet made uniform,
// so the read can be issued well before it is used: a split piece reads it before its first
// unit, and again when it ends if the first value did not show every other piece arrived).
__device__ __forceinline__ int counter_peek(int32_t* c) {
  return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave-uniform: true in exactly one of the segment's pieces, the one that merges.  `others`
// is the number of other pieces, `seen` an earlier counter_peek of c, and `publish` writes
// this piece's partial with device-scope stores; it is skipped when every other piece has
// already arrived (that piece merges from its registers and nobody reads its slot).
// `between` runs exactly once, before any wait for this protocol's own memory operations
// but after the stores of the partial are issued, so that loads it issues (the wave's next
// piece) travel together with them.
template <class Pub, class Between>
__device__ __forceinline__ bool split_arrive(int32_t* c, int others, int seen, Pub&& publish,
                                             Between&& between) {
  if (__builtin_amdgcn_readfirstlane(seen) == others) {
    between();
    return true;
  }
  const int fresh = counter_peek(c);  // a fresh look
  between();
  if (__builtin_amdgcn_readfirstlane(fresh) == others) return true;
  publish();
  // every store of this wave, the partial included, has reached the point of coherence
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  int old = 0;
  if (__lane_id() == 0) old = __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_amdgcn_readfirstlane(old) == others;
}

__device__ __forceinline__ void counter_reset(int32_t* c) {
  if (__lane_id() == 0) __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Log-sum-exp merge, per lane, of R rows of NE output elements over the pieces k0..k1 in
// that order: fetch(k, m, l, o) gives piece k's per-row max (natural-log domain), sum and
// normalised output, by device-scope loads or, for the merging piece itself, from the
// registers it would have published.  The arithmetic depends only on the pieces' values and
// the fixed order, so every call gives the same bits whichever piece merges.  Pieces are
// fetched B at a time into two alternating batches, so the loads of the next batch are in
// flight while the current one is combined.  Returns each row's merged output in U, its sum
// in L and its max (natural-log domain) in M (the output is U / L).
template <int R, int NE, int B>
struct MergeBatch {
  float m[B][R], l[B][R], o[B][R][NE];
};

template <int R, int NE, int B, class Fetch>
__device__ __forceinline__ void merge_ordered(float (&M)[R], float (&L)[R], float (&U)[R][NE],
                                              int64_t k0, int64_t k1, Fetch&& fetch) {
  const int n = (int)(k1 - k0 + 1);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    M[r] = -INFINITY;
    L[r] = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) U[r][e] = 0.f;
  }
  auto load = [&](MergeBatch<R, NE, B>& bt, int q0) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (q0 + b < n) {
        fetch(k0 + q0 + b, bt.m[b], bt.l[b], bt.o[b]);
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          bt.m[b][r] = -INFINITY;
          bt.l[b][r] = 0.f;
#pragma unroll
          for (int e = 0; e < NE; ++e) bt.o[b][r][e] = 0.f;
        }
      }
    }
  };
  auto combine = [&](const MergeBatch<R, NE, B>& bt) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float mn = M[r];
#pragma unroll
      for (int b = 0; b < B; ++b) mn = fmaxf(mn, bt.m[b][r]);
      const float s = M[r] == -INFINITY ? 0.f : __expf(M[r] - mn);
      L[r] *= s;
#pragma unroll
      for (int e = 0; e < NE; ++e) U[r][e] *= s;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float w = bt.m[b][r] == -INFINITY ? 0.f : bt.l[b][r] * __expf(bt.m[b][r] - mn);
        L[r] += w;
#pragma unroll
        for (int e = 0; e < NE; ++e) U[r][e] = fmaf(w, bt.o[b][r][e], U[r][e]);
      }
      M[r] = mn;
    }
  };
  MergeBatch<R, NE, B> ba, bb;
  load(ba, 0);
  for (int q0 = 0; q0 < n; q0 += 2 * B) {
    if (q0 + B < n) load(bb, q0 + B);
    combine(ba);
    if (q0 + B >= n) break;
    if (q0 + 2 * B < n) load(ba, q0 + 2 * B);
    combine(bb);
  }
}

// Folds the shared-prefix partials of one (row, query head) into that row's merged result:
// pm, pl, po point at its first partial (max in the natural-log domain, sum, D-float
// normalised output), np <= kMaxPrefixParts partials follow one another, and (M, L, U) is
// the running merge (max, sum, unnormalised output of this lane's NE dimensions dim(k)) that
// the fold updates.  A partial without keys (l = 0) changes nothing.  Every max and sum is
// loaded at once; with the merged max known, the outputs are weighted sums of independent
// terms, loaded B partials at a time with all their loads in flight (partials past np are
// read from partial 0 and weighted 0).
constexpr int kMaxPrefixParts = 8;

template <int NE, int B, class Dim>
__device__ __forceinline__ void fold_prefix(float& M, float& L, float (&U)[NE], const float* pm,
                                            const float* pl, const float* po, int D, int np,
                                            Dim&& dim) {
  static_assert(kMaxPrefixParts % B == 0, "whole batches");
  float mp[kMaxPrefixParts], lp[kMaxPrefixParts];
#pragma unroll
  for (int p = 0; p < kMaxPrefixParts; ++p) {
    const int q = p < np ? p : 0;
    mp[p] = pm[q];
    lp[p] = pl[q];
  }
  float mn = M;
#pragma unroll
  for (int p = 0; p < kMaxPrefixParts; ++p)
    if (p < np && lp[p] > 0.f) mn = fmaxf(mn, mp[p]);
  const float sa = M == -INFINITY ? 0.f : __expf(M - mn);
  L *= sa;
#pragma unroll
  for (int k = 0; k < NE; ++k) U[k] *= sa;
  float w[kMaxPrefixParts];
#pragma unroll
  for (int p = 0; p < kMaxPrefixParts; ++p) {
    w[p] = p < np && lp[p] > 0.f ? lp[p] * __expf(mp[p] - mn) : 0.f;
    L += w[p];
  }
#pragma unroll
  for (int p0 = 0; p0 < kMaxPrefixParts; p0 += B) {
    if (p0 >= np) break;  // uniform
    float o[B][NE];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int q = p0 + b < np ? p0 + b : 0;
#pragma unroll
      for (int k = 0; k < NE; ++k) o[b][k] = po[(int64_t)q * D + dim(k)];
    }
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int k = 0; k < NE; ++k) U[k] = fmaf(w[p0 + b], o[b][k], U[k]);
  }
  M = mn;
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled: i is a constant in f.
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

}  // namespace pa
