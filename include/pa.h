/*
 * pa.h — paged-attention decode for MI355X (gfx950): the C ABI of libpa.so.
 *
 * The operation ("vLLM 深度拆解：当 KV Cache 学会「分页」" §2.2, §3.3, §6.2; "vLLM 架构源码解析
 * 第1篇" §3.3.3): each step first scatters the new tokens' K and V into a pool of
 * fixed-size physical blocks (reshape_and_cache), then computes, for every query row r and
 * query head h,
 *
 *     out[r][h] = softmax(scale * q[r][h] . K^T) . V
 *
 * over the row's visible keys, gathered block by block through a per-sequence block table.
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers into caller-owned memory, except `geom`
 *     (host).  The library allocates, frees and synchronises nothing; every launch is
 *     enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *   - Arrays are dense, row-major, and 16-byte aligned.
 *   - Errors: arguments are checked on the host before any launch and reported as a
 *     pa_status; nothing is launched on error.  A failed launch returns PA_ERR_HIP.
 *     Device-resident values (block ids < num_blocks, context_lens <= max_blocks_per_seq
 *     * block_size, unique slots) are the caller's contract and are not checked.
 *   - block_size is 16 ("vLLM 架构源码解析 第1篇" §4.2: 16-token blocks), 8, 32 or 64 (§5.1
 *     weighs block sizes 8, 16 and 32 against each other).  head_dim is 64 or 128.
 *     kv_dtype is PA_F32, PA_F16 or PA_BF16 (q, key, value and both pools share it), or
 *     PA_FP8_E4M3 (see "FP8 pools").
 *
 * Pool layout (part of this ABI).  elem = 4 (fp32), 2 (fp16, bf16) or 1 (FP8) bytes,
 * X = 16 / elem, T = min(block_size, 16) tokens per tile, R = block_size / T:
 *   k_cache: [num_blocks][R][num_kv_heads][head_dim / X][T][X]
 *   v_cache: [num_blocks][R][num_kv_heads][head_dim][T]
 * For 16-token blocks (R = 1) v_cache is the pages' [num_blocks, num_heads, head_size,
 * block_size] ("vLLM 深度拆解" §6.2); k_cache splits head_size into 16-byte chunks so one
 * token's chunk is one 16-byte load and the 16 tokens of a chunk are 256 contiguous bytes.
 * A larger block is R consecutive 16-token sub-blocks in that layout, token t of the block
 * in sub-block t / 16 at position t % 16 (so slot / 16 names a sub-block for every block
 * size from 16 up).  An 8-token block is one tile of T = 8 (its V is the pages' layout with
 * block_size 8).
 *
 * FP8 pools ("vLLM 深度拆解" §10.1 names FP8 KV with calibrated scales).  kv_dtype
 * PA_FP8_E4M3: one byte per element in the layout above with elem = 1, X = 16; q, key and
 * value are fp16 or bf16 (q_dtype PA_F16 or PA_BF16), out is q_dtype or fp32.  Each pool
 * has one scale: reshape_and_cache stores e4m3(fp32(x) / scale), the fp32 quotient rounded to the nearest
 * E4M3 ("E4M3FN": bias 7, no infinity, largest 448) with ties to even, magnitudes from 448
 * up saturating to 448; attention reads an element as its E4M3 value times the scale.
 * Every entry point takes FP8 pools.
 *
 * Rows and positions.  query_start_loc ("vLLM 架构源码解析 第1篇" §3.3.2) is NULL when every sequence has one
 * query row (row r belongs to sequence r, num_q_rows == num_seqs), else an int32 [S + 1]
 * prefix array: sequence s owns rows [qsl[s], qsl[s+1]).  context_lens[s] counts every
 * token of s including this step's rows; row j of an n-row sequence sits at position
 * ctx - n + j and sees keys [0, ctx - n + j] (causal).  A row with no visible key
 * produces 0.  Query head h reads KV head h / (num_q_heads / num_kv_heads).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3 } pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = -2,       /* inconsistent sizes (negative counts, Hq % Hkv != 0, ...) */
  PA_ERR_UNSUPPORTED = -3, /* a valid but unimplemented combination (head_dim, dtype, ...) */
  PA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than pa_workspace_size() */
  PA_ERR_HIP = -5,         /* a HIP launch failed (hipGetLastError after the launch) */
  PA_ERR_NO_BLOCKS = -6    /* the block pool has too few free blocks (block manager) */
} pa_status;

/* Geometry shared by all calls (host struct, read during the call only). */
typedef struct {
  int32_t num_seqs;           /* S */
  int32_t num_q_heads;        /* Hq */
  int32_t num_kv_heads;       /* Hkv; Hq % Hkv == 0, Hq / Hkv <= 16 */
  int32_t head_dim;           /* D: 64 or 128 */
  int32_t block_size;         /* tokens per physical block: 16, 32 or 64 */
  int32_t num_blocks;         /* NB: blocks in each pool */
  int32_t max_blocks_per_seq; /* MB: row stride of block_tables */
  int32_t kv_dtype;           /* pa_dtype of k_cache, v_cache (and of q, key, value unless FP8) */
  int32_t out_dtype;          /* pa_dtype of out: q_dtype or PA_F32 */
  int32_t q_dtype;            /* pa_dtype of q, key, value: kv_dtype, or PA_F16 / PA_BF16 for FP8 pools */
  float k_scale;              /* FP8 pools: stored K = e4m3(fp32(key) / k_scale); else ignored */
  float v_scale;              /* FP8 pools: stored V = e4m3(fp32(value) / v_scale); else ignored */
} pa_geom;

/* Bytes of one pool (K or V): num_blocks * num_kv_heads * head_dim * block_size * elem.
 * Returns 0 for an invalid geometry. */
size_t pa_kv_cache_bytes(const pa_geom* geom);

/*
 * Cache write ("vLLM 架构源码解析 第1篇" §3.3.3 reshape_and_cache(k, v, kv_cache,
 * slot_mapping); slot arithmetic from §4.2's `//` and `%`).  For every token t with
 * slot_mapping[t] >= 0: block = slot / block_size, offset = slot % block_size, and for every
 * KV head g the bits of key[t][g][:] / value[t][g][:] are copied to k_cache / v_cache at
 * (block, g, offset).  Negative slots are skipped (padding).
 *   key, value     [num_tokens][num_kv_heads][head_dim], kv_dtype
 *   k_cache, v_cache  the pools (layout above), written in place
 *   slot_mapping   int64 [num_tokens]; slots must be unique and < num_blocks * block_size
 * num_tokens == 0 is a no-op.  Writes into a block shared by several sequences are the
 * caller's responsibility (copy-on-write happens before this call).
 */
pa_status pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                               const int64_t* slot_mapping, int64_t num_tokens,
                               const pa_geom* geom, void* stream);

/*
 * Block copy for copy-on-write ("vLLM 架构源码解析 第1篇" §4.3.2: samples forked from one
 * prompt share its blocks; a sample that is about to write into a block other sequences
 * still reference first gets a new block holding a copy of it).  For every pair p,
 * physical block block_mapping[2p] (source) is copied bit for bit onto physical block
 * block_mapping[2p + 1] (destination) in both pools, for every KV head.
 *   k_cache, v_cache  the pools (layout above), written in place
 *   block_mapping     int64 [num_pairs][2]: source, destination
 * A pair with an id outside [0, num_blocks) is skipped.  Destinations must be distinct and
 * no destination may be the source of another pair of the same call (the copies run in
 * parallel); this is the caller's contract and is not checked.  num_pairs == 0 is a no-op.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping,
                         int64_t num_pairs, const pa_geom* geom, void* stream);

/*
 * Block swap between the device pools and a host copy of them (preemption by swapping,
 * "vLLM 架构源码解析 第1篇" §1.1: a preempted request's KV blocks go to CPU memory and come
 * back to the GPU when it resumes).  direction PA_SWAP_OUT: for every pair p, device block
 * block_mapping[2p] of k_cache / v_cache is copied bit for bit onto host block
 * block_mapping[2p + 1] of host_k / host_v; PA_SWAP_IN: host block block_mapping[2p] onto
 * device block block_mapping[2p + 1].  A block is all KV heads of one block id.
 *   k_cache, v_cache  the device pools (geom->num_blocks blocks, layout above)
 *   host_k, host_v    host memory holding host_num_blocks blocks in the same layout.  Pinned
 *                     memory (hipHostMalloc) is read or written by one kernel over PCIe for
 *                     all pairs; other host memory goes through one copy per run
 *   block_mapping     host memory, int64 [num_pairs][2]: source, destination
 * Every id is checked against its pool before anything is queued (PA_ERR_SHAPE).  Without a
 * device mapping, pairs whose source and destination ids both continue the previous pair's
 * are copied as one run.
 * The copies are queued on stream and the caller keeps both sides alive until they finish.
 * Destinations must be distinct (not checked).  num_pairs == 0 is a no-op.
 */
typedef enum { PA_SWAP_OUT = 0, PA_SWAP_IN = 1 } pa_swap_direction;
pa_status pa_swap_blocks(void* k_cache, void* v_cache, void* host_k, void* host_v,
                         int64_t host_num_blocks, const int64_t* block_mapping,
                         int64_t num_pairs, int32_t direction, const pa_geom* geom,
                         void* stream);

/* Workspace bytes pa_decode needs for this geometry and row count (0 is never returned
 * for a valid geometry; returns 0 for an invalid one).  The workspace holds the partials of
 * the context splits pa_decode makes inside one kernel (see pa_decode): two partial slots
 * per wave of that kernel's grid plus one arrival counter per wave of the largest grid the
 * device can have.  Its size therefore depends on the device, the head size, the query
 * group and whether sequences may have several rows, not on context lengths or a partition
 * size.  The pages name a split-context kernel ("vLLM 架构源码解析 第1篇" §4.2,
 * paged_attention_v2) without describing it; the split, its partials and their merge are
 * this library's. */
size_t pa_workspace_size(const pa_geom* geom, int32_t num_q_rows);

/*
 * Full decode step ("vLLM 深度拆解" §2.2 formula, §3.3 block walk, §6.2 arguments:
 * output, query, k_cache, v_cache, block_tables, context_lens, scale).
 *   out           [num_q_rows][num_q_heads][head_dim], out_dtype
 *   q             [num_q_rows][num_q_heads][head_dim], kv_dtype
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]: logical block j of sequence s lives
 *                 in physical block block_tables[s * max_blocks_per_seq + j]
 *   context_lens  int32 [num_seqs]
 *   query_start_loc  int32 [num_seqs + 1] or NULL (see "Rows and positions")
 *   num_q_rows    rows of q and out (num_seqs without query_start_loc)
 *   max_query_len with query_start_loc: an upper bound of any sequence's row count,
 *                 qsl[s + 1] - qsl[s], or 0 when unknown (then num_q_rows is taken).  It
 *                 picks the kernels from the host, which never reads device data: when the
 *                 bound lets every sequence fit the decode kernel (one row; on the
 *                 matrix-core path up to 16 / G rows), the multi-row kernel is not launched.
 *                 A bound below some sequence's row count is a caller error: that
 *                 sequence's rows are then written NaN (unless the multi-row kernel runs
 *                 for another sequence, in which case they are computed), and the call
 *                 returns PA_OK.  Ignored without query_start_loc; must be >= 0.
 *   scale         multiplies q . k (normally 1 / sqrt(head_dim))
 *   workspace     device scratch of at least pa_workspace_size(geom, num_q_rows) bytes for
 *                 split-context partials and their arrival counters.  Zero-fill it once
 *                 before its first use (e.g. hipMemset after allocating it): every call
 *                 leaves the counters at zero again, so the workspace can then be reused
 *                 across calls and geometries on the same device without clearing it.
 *                 Calls that may run concurrently must not share a workspace.
 * The (sequence, head) work is split evenly over the workgroups of one kernel; a long
 * context crossing a split boundary is computed in pieces, and the piece that finishes last
 * merges them by log-sum-exp inside the same kernel.  A second kernel runs the multi-row
 * sequences when query_start_loc is given.
 * Sequences with several rows (query_start_loc) need a 16-bit or FP8 kv_dtype and a query
 * group G = Hq / Hkv that divides 16; otherwise PA_ERR_UNSUPPORTED.
 */
pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens,
                    const int32_t* query_start_loc, int32_t num_q_rows, int32_t max_query_len,
                    float scale, void* workspace, size_t workspace_bytes, const pa_geom* geom,
                    void* stream);

/*
 * pa_decode without a workspace, for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops that must not call hipMalloc, harnesses that forbid it.
 * Arguments, results and errors are pa_decode's, less workspace and workspace_bytes.  The
 * split-context partials and arrival counters live in a static device array of
 * PA_DECODE_SCRATCH_BYTES bytes that the library holds on every device it runs on until the
 * process ends; the call allocates, frees and creates nothing.  The first call on a device
 * looks up the array's device address and clears its arrival counters with one small kernel
 * on `stream`; every call leaves them at zero again, as pa_decode does with a workspace.
 * All calls on one device share that array: calls that may run at the same time on one
 * device (different streams, or threads without ordering) race on it and must not be
 * issued; calls queued on one stream are ordered and safe.  Sequences with several rows
 * run their chunk kernel on `stream` before the decode kernel (pa_decode runs the two side
 * by side on a second stream).  PA_ERR_WORKSPACE: this geometry and row count need more
 * than PA_DECODE_SCRATCH_BYTES (pa_workspace_size gives the need).
 */
#define PA_DECODE_SCRATCH_BYTES ((size_t)36 << 20)
pa_status pa_decode_scratch(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            const int32_t* query_start_loc, int32_t num_q_rows,
                            int32_t max_query_len, float scale, const pa_geom* geom,
                            void* stream);

/*
 * Split-context partials (flash-decoding).  The pages name the split-context decode kernel
 * only by its file ("vLLM 架构源码解析 第1篇" §4.2, paged_attention_v2); what it computes is
 * this library's reading: the attention of "vLLM 深度拆解" §2.2 restricted to fixed key
 * partitions, whose partials pa_decode_reduce merges by log-sum-exp into exactly the
 * softmax over all keys.  Partition p of a row is the row's visible keys (see "Rows and
 * positions") among positions [p * partition_size, (p + 1) * partition_size).
 *   tmp_out     float [num_q_rows][num_q_heads][max_partitions][head_dim]: the partition's
 *               softmax-normalised output
 *   max_logits  float [num_q_rows][num_q_heads][max_partitions]: max of scale * q . k over
 *               the partition's keys
 *   exp_sums    float [num_q_rows][num_q_heads][max_partitions]: sum of
 *               exp(scale * q . k - max_logits) over those keys
 *   query_start_loc  int32 [num_seqs + 1] or NULL (one row per sequence, num_q_rows ==
 *               num_seqs); with it, sequences of several rows (chunked-prefill or verify
 *               rows) get their partials from the multi-row kernel, which then runs after
 *               the decode kernel on `stream`.  Needs a 16-bit or FP8 kv_dtype and a query
 *               group G = Hq / Hkv that divides 16 (else PA_ERR_UNSUPPORTED), as pa_decode.
 * Every max_logits / exp_sums entry is written; a partition with no key of the row gets
 * max_logits = -inf and exp_sums = 0 and its tmp_out entries are not written.
 * partition_size is a positive multiple of 32; max_partitions must cover the longest
 * possible context: max_partitions * partition_size >= max_blocks_per_seq * block_size.
 * Other arguments as pa_decode.
 */
pa_status pa_decode_partitioned(float* tmp_out, float* max_logits, float* exp_sums,
                                const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* context_lens,
                                const int32_t* query_start_loc, int32_t num_q_rows,
                                float scale, int32_t partition_size, int32_t max_partitions,
                                const pa_geom* geom, void* stream);

/*
 * Log-sum-exp merge of pa_decode_partitioned's output (the merge of its split-context
 * partials; see there for what the pages say of it): over the partitions with
 * exp_sums > 0, M = max_p max_logits[p], w_p = exp_sums[p] * exp(max_logits[p] - M) and
 * out = sum_p w_p * tmp_out[p] / sum_p w_p.  Rows with no key get 0.  Arguments as in
 * pa_decode_partitioned; out [num_q_rows][num_q_heads][head_dim] in out_dtype.
 */
pa_status pa_decode_reduce(void* out, const float* tmp_out, const float* max_logits,
                           const float* exp_sums, int32_t num_q_rows, int32_t max_partitions,
                           const pa_geom* geom, void* stream);

/*
 * Decode with shared prefixes.  "vLLM 深度拆解" §5.2 has many requests start with the same
 * 512-token system prompt, and "vLLM 架构源码解析 第1篇" §4.3.1 keeps such prefix blocks
 * once, in the block tables of every request that uses them (ref_cnt > 1).  The result is
 * pa_decode's (every row's attention over its visible keys); what changes is the work: the
 * keys of a group's shared leading blocks are read once per KV head for the rows of all the
 * group's sequences (the matrix-core multi-row kernel, those rows as its columns, in
 * partials of at least 128 keys), and the decode kernel then reads each sequence's keys
 * past the prefix only and folds the prefix partials into its result by log-sum-exp.  The
 * grouping is this library's addition; the pages describe the sharing, not how a kernel
 * uses it.
 *   prefix_groups  int32 [num_groups + 1] (device), non-decreasing: group i is sequences
 *                  [prefix_groups[i], prefix_groups[i + 1]) (clamped to the batch);
 *                  sequences outside every group are decoded as pa_decode does, and so is
 *                  every sequence when the array decreases anywhere (overlapping groups)
 *   prefix_blocks  int32 [num_groups] (device): leading block-table entries the group's
 *                  sequences are said to share; at most max_prefix_blocks of them are used
 *   max_prefix_blocks  bound of the shared blocks used (<= max_blocks_per_seq); sizes the
 *                  workspace
 * The claim is checked on the device: the prefix of group i is its first
 * min(prefix_blocks[i], max_prefix_blocks) blocks cut down to whole 32-token units, and a
 * sequence takes it only when it is a decode or verify sequence (the rows pa_decode's decode
 * kernel takes), every one of its rows sees every prefix key (prefix <= context_len - rows)
 * and its table entries over the prefix equal those of the group's first sequence, which
 * must satisfy the same; any other sequence attends all its keys itself.  A wrong claim
 * costs work, never correctness.  Needs a 16-bit or FP8 kv_dtype and G | 16 (else
 * PA_ERR_UNSUPPORTED); the workspace (pa_shared_prefix_workspace_size bytes, device memory,
 * the caller's) holds pa_decode's workspace, one int per sequence and the prefix partials
 * (num_q_rows * num_q_heads * up to 8 partials of head_dim + 2 floats).  Other arguments,
 * ordering and errors as pa_decode; PA_ERR_SHAPE: num_groups or max_prefix_blocks negative
 * or max_prefix_blocks > max_blocks_per_seq; PA_ERR_NULL: num_groups > 0 without the group
 * arrays.  Calls that share a workspace must be ordered.
 */
size_t pa_shared_prefix_workspace_size(const pa_geom* geom, int32_t num_q_rows,
                                       int32_t max_prefix_blocks);
pa_status pa_decode_shared_prefix(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, const int32_t* query_start_loc,
                                  int32_t num_q_rows, int32_t max_query_len,
                                  const int32_t* prefix_groups, const int32_t* prefix_blocks,
                                  int32_t num_groups, int32_t max_prefix_blocks, float scale,
                                  void* workspace, size_t workspace_bytes,
                                  const pa_geom* geom, void* stream);

/* Static description of a status code. */
const char* pa_status_str(pa_status status);

#ifdef __cplusplus
}
#endif
#endif /* PA_H */
