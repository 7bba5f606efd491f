// pa_internal.h — kernel argument blocks and launchers inside libpa.so (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kWave = 64;
constexpr int kWavesPerWG = 4;
constexpr int kWG = kWave * kWavesPerWG;
constexpr int kBlock = 16;  // tokens per physical block

// element types; DT_FP8 / DT_FP8B: FP8 E4M3 pools with fp16 / bf16 queries, keys and values
enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_FP8 = 3, DT_FP8B = 4 };

constexpr bool is_fp8(int dt) { return dt == DT_FP8 || dt == DT_FP8B; }

// How a split kernel distributes and emits its work.
enum SplitMode : int {
  // pa_decode: every workgroup owns an equal share of the flattened unit list; a segment
  // that lies inside one share is written to `out`; the pieces of a segment that crosses
  // share boundaries are merged inside the kernel by the piece that finishes last.
  MODE_EVEN = 0,
  // pa_decode_partitioned: fixed partitions of `partition_units` units; every (seq,
  // segment, partition) is one item, written to tmp_out / max_logits / exp_sums.
  MODE_PARTITION = 1,
};

struct DecodeArgs {
  void* out;                // [rows][Hq][D], out dtype
  const void* q;            // [rows][Hq][D]
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* qsl;       // NULL: one row per sequence
  float* part_o;            // MODE_EVEN: [W][2][G][D]; MODE_PARTITION: tmp_out [rows][Hq][P][D]
  float* part_m;            // MODE_EVEN: [W][2][G];    MODE_PARTITION: max_logits [rows][Hq][P]
  float* part_l;            // MODE_EVEN: [W][2][G];    MODE_PARTITION: exp_sums   [rows][Hq][P]
  int32_t* counters;        // MODE_EVEN: [4 o + i] arrival counters, zero before and after a call
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_blocks_per_seq;
  int32_t out_f32;          // 1: out is fp32; 0: out has the KV dtype
  float scale_log2;         // scale * log2(e): scores are kept in the base-2 domain
  int32_t partition_units;  // MODE_PARTITION: units per partition
  int32_t max_partitions;   // MODE_PARTITION
  int32_t seg_extra;        // MODE_EVEN: balancing units per segment (see PlanIn)
  int32_t heads_per_wave;   // MODE_EVEN, vector kernel: query heads per wave (1, 2, 4, 8)
  int32_t odd_skew;         // MODE_EVEN: per mille of work moved from odd to even workgroups
  int32_t max_rows;         // MODE_EVEN: query rows per sequence the decode kernel takes (1, or
                            // 16 / G on the matrix-core path); longer sequences: chunk kernel
  int32_t cols;             // MODE_EVEN, matrix-core path: query columns per partial slot
  float v_factor;           // DT_FP8: the outputs' factor (v_scale)
  int32_t blk_shift;        // log2(block_size / 16): table entries name 2^blk_shift sub-blocks
  int32_t lean;             // MODE_EVEN, matrix-core path with several rows: the lean stream
  int32_t part_tokens;      // chunk kernel: > 0 for pa_decode_partitioned's key partitions
  int32_t nan_rows;         // MODE_EVEN with qsl and no chunk kernel: rows of sequences with
                            // more than max_rows rows are written NaN
  int32_t b8;               // 8-token blocks: a 16-token tile is two blocks (table entries
                            // 2 j and 2 j + 1), each a pool tile of 8 tokens
  int32_t xcd_major;        // MODE_EVEN, vector kernel: list in (head group, sequence, tile)
                            // order with XCD-major owners (see Part)
  // shared prefixes (pa_decode_shared_prefix).  Decode kernels: keys [0, skip[s]) of sequence
  // s were attended by the prefix kernel, whose partials (normalised output, max in the
  // natural-log domain, sum) for row r and query head h sit at pre_* [(r Hq + h) pre_parts +
  // p], one per pre_tokens keys; the decode kernel folds them into the row's result.  NULL
  // skip: no shared prefix.
  const int32_t* skip;
  const float* pre_o;
  const float* pre_m;
  const float* pre_l;
  int32_t pre_parts;
  int32_t pre_tokens;
  // prefix kernel (chunk kernel, prefix mode): group i is sequences [grp_start[i],
  // grp_start[i + 1]) sharing their first grp_blocks[i] table entries (at most
  // max_prefix_blocks are used); it writes skip_out[s] for every sequence
  const int32_t* grp_start;
  const int32_t* grp_blocks;
  int32_t num_groups;
  int32_t max_prefix_blocks;
  int32_t block_size;
  int32_t* skip_out;
};

struct ReshapeArgs {
  const void* key;
  const void* value;
  void* k_cache;
  void* v_cache;
  const int64_t* slot_mapping;
  int64_t num_tokens;
  int32_t num_kv_heads;
  int32_t head_dim;
  float k_scale;  // DT_FP8: stored K = e4m3(key / k_scale)
  float v_scale;  // DT_FP8: stored V = e4m3(value / v_scale)
  int32_t tile_shift;  // log2 of the tokens of one pool tile: 3 (8-token blocks) or 4
};

struct CopyBlocksArgs {
  void* k_cache;
  void* v_cache;
  const int64_t* block_mapping;  // [num_pairs][2]: source block, destination block
  int64_t num_pairs;
  int64_t block_bytes;           // one block of one pool: Hkv * 16 * D * elem
  int64_t num_blocks;
};

// Block swap between device pools and device-mapped pinned host pools: one launch takes up
// to kSwapPairs pairs, carried in the kernel arguments (the host mapping need not be
// device-visible).
constexpr int kSwapPairs = 224;
struct SwapArgs {
  const char* src_k;
  const char* src_v;
  char* dst_k;
  char* dst_v;
  int64_t block_bytes;  // one block of one pool
  int32_t num_pairs;    // <= kSwapPairs
  int64_t pairs[kSwapPairs][2];  // source, destination (checked by the host)
};

struct PartReduceArgs {
  void* out;
  const float* tmp_out;
  const float* max_logits;
  const float* exp_sums;
  int64_t num_items;  // rows * Hq
  int32_t head_dim;
  int32_t max_partitions;
  int32_t out_f32;
};

// launchers (return hipSuccess or the launch error)
hipError_t launch_reshape(int dt, const ReshapeArgs& a, hipStream_t st);
// VALU kernel: one query head per segment (segs = Hq), any head_dim in {64, 128}
hipError_t launch_valu_decode(int dt, int mode, const DecodeArgs& a, int grid, hipStream_t st);
int valu_decode_max_blocks_per_cu(int dt, int head_dim, int hpw, int mode, int lds_bytes);
// MFMA kernel: one kv head (all G query heads) per segment, 16-bit dtypes
hipError_t launch_mfma_decode(int dt, int mode, const DecodeArgs& a, int grid, hipStream_t st);
int mfma_decode_max_blocks_per_cu(int dt, int head_dim, int mode, int lds_bytes);
hipError_t launch_part_reduce(int dt, const PartReduceArgs& a, hipStream_t st);
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t st);
hipError_t launch_swap_blocks(const SwapArgs& a, hipStream_t st);

// resident workgroups per CU at most (32 waves of 64 lanes): bounds the even split's grid
constexpr int kMaxWgPerCu = 8;

// unit sizes (tokens) of the split kernels
constexpr int kValuUnit = 16;
constexpr int kMfmaUnit = 32;

}  // namespace pa
