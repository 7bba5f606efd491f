/*
 * pa_block_manager.h — host-side block manager of the paged KV cache (C ABI of libpa.so).
 *
 * It owns the bookkeeping the decode kernels read: which physical blocks of the pool each
 * sequence holds, in logical order, and which slot every new token is written to.  Pure host
 * code: no call here touches the GPU.  Its outputs are the inputs of include/pa.h:
 * block tables and context lengths for pa_decode, slot mappings for pa_reshape_and_cache,
 * and (source, destination) pairs for pa_copy_blocks.
 *
 * What it follows:
 *   - Block pool ("vLLM 深度拆解：当 KV Cache 学会「分页」" §3.2): all blocks exist from the start;
 *     a block is taken from the tail of a free list and returned to its tail, both O(1), and
 *     an empty list is an out-of-memory error.
 *   - Block table ("2. 核心思想"; "vLLM 深度拆解" §3.3): logical block j of a sequence maps to a
 *     physical block; token t sits in logical block t / block_size at offset t % block_size,
 *     slot = physical block * block_size + offset ("vLLM 架构源码解析 第1篇" §4.2).
 *   - Growth ("vLLM 架构源码解析 第1篇" §4.3.3): blocks are taken on demand, a new one whenever
 *     a token falls past the last block.  A sequence of n tokens holds ceil(n / block_size)
 *     blocks (the page's prompt formula floors; the ceiling is the count that holds every
 *     token).
 *   - Prefix caching ("vLLM 架构源码解析 第1篇" §4.3.1): every full block of a prompt is looked
 *     up by its contents; a hit shares the cached block and raises its reference count.
 *     Reading taken: a block's key is its 16 token ids together with the physical block
 *     that precedes it in the table (so a hit also requires the same earlier tokens, which
 *     the block's keys and values depend on); keys are compared exactly, not by hash alone.
 *     The last token of a prompt is never served from the cache (its query row must run),
 *     so at most the full blocks before it are shared.
 *   - Reference counts and freeing ("vLLM 架构源码解析 第1篇" §4.3.1): freeing a sequence
 *     drops one reference of each of its blocks; a block whose count reaches zero returns to
 *     the free list and leaves the prefix cache.
 *   - Copy-on-write ("vLLM 架构源码解析 第1篇" §4.3.2): a fork shares every block of its parent.
 *     Appending into a partly filled last block that another sequence still references first
 *     moves the appending sequence onto a fresh block and records the pair (shared block,
 *     fresh block) for pa_copy_blocks, which must run before the new tokens are written.
 *   - Preemption by swapping ("vLLM 架构源码解析 第1篇" §1.1): a sequence's blocks can move to
 *     a pool of host blocks (their own LIFO free list) and back; each move returns the
 *     (source, destination) pairs for pa_swap_blocks.  While swapped out, a sequence keeps
 *     its length and tokens but holds no device block, and only pa_bm_swap_in,
 *     pa_bm_free_sequence and pa_bm_seq_len accept it.
 *
 * Errors: every call checks its arguments and returns a pa_status; a call that fails
 * changes nothing.  The manager is not thread-safe: one caller at a time.
 */
#ifndef PA_BLOCK_MANAGER_H
#define PA_BLOCK_MANAGER_H

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager; /* opaque */

/* New manager over physical blocks [0, num_blocks) of block_size tokens (16 for the decode
 * kernels), at most max_blocks_per_seq blocks per sequence.  Initially every block is free;
 * the first allocations take the highest ids first (the tail of the free list).  Returns
 * NULL on invalid sizes or when host memory runs out.  The caller frees it with
 * pa_bm_destroy. */
pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq);
void pa_bm_destroy(pa_block_manager* bm);

int32_t pa_bm_num_free_blocks(const pa_block_manager* bm);
/* Reference count of a physical block (0: free), or -1 for an id outside the pool. */
int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t block);
/* Tokens of a live sequence, or -1 for an unknown id. */
int32_t pa_bm_seq_len(const pa_block_manager* bm, int32_t seq);

/*
 * New sequence holding a prompt of num_tokens tokens (num_tokens >= 0).  token_ids
 * [num_tokens] enables prefix caching (NULL: no lookup and nothing registered).  On success
 * *seq_id is the new sequence's id and *num_cached_tokens the length of the prompt prefix
 * whose keys and values already sit in shared blocks (a multiple of block_size; the caller
 * writes only tokens [num_cached_tokens, num_tokens)).
 * PA_ERR_NO_BLOCKS if the pool lacks free blocks, PA_ERR_SHAPE if the prompt needs more than
 * max_blocks_per_seq blocks.
 */
pa_status pa_bm_add_sequence(pa_block_manager* bm, const int32_t* token_ids, int32_t num_tokens,
                             int32_t* seq_id, int32_t* num_cached_tokens);

/* New sequence sharing every block of `parent` (each block's reference count rises by one);
 * it has the parent's length and tokens. */
pa_status pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t* child_id);

/*
 * Grow a sequence by num_tokens tokens and return their slots (slots_out [num_tokens],
 * int64, the slot_mapping entries of pa_reshape_and_cache).  token_ids [num_tokens] or NULL
 * as in pa_bm_add_sequence: with ids, every block the new tokens complete is registered in
 * the prefix cache.  If the last block is partly filled and shared, the sequence first
 * moves onto a fresh block and a copy pair is queued (pa_bm_take_copies).
 * PA_ERR_NO_BLOCKS / PA_ERR_SHAPE as in pa_bm_add_sequence.
 */
pa_status pa_bm_append(pa_block_manager* bm, int32_t seq, const int32_t* token_ids,
                       int32_t num_tokens, int64_t* slots_out);

/* Slots of positions [first, first + count) of a sequence (int64 [count]); PA_ERR_SHAPE if
 * the range is not inside the sequence. */
pa_status pa_bm_slots(const pa_block_manager* bm, int32_t seq, int32_t first, int32_t count,
                      int64_t* slots_out);

/* Release a sequence: one reference of each of its blocks is dropped (last block first);
 * blocks that reach zero return to the free list and leave the prefix cache.  A swapped-out
 * sequence returns its host blocks to the host free list. */
pa_status pa_bm_free_sequence(pa_block_manager* bm, int32_t seq);

/* Size the host block pool [0, num_host_blocks) for swapped-out sequences (0 at creation);
 * PA_ERR_SHAPE while any sequence is swapped out. */
pa_status pa_bm_set_host_blocks(pa_block_manager* bm, int32_t num_host_blocks);
/* Free host blocks, or -1 on NULL. */
int32_t pa_bm_num_free_host_blocks(const pa_block_manager* bm);
/* Swap a sequence out: each of its device blocks, in logical order, gets a host block (taken
 * from the host free list) and the pair (device block, host block) is written to pairs_out
 * (int64 [max_pairs][2], pa_swap_blocks's PA_SWAP_OUT mapping); then one reference of each
 * device block is dropped as by pa_bm_free_sequence (blocks still shared stay for the other
 * sequences).  *num_pairs = the sequence's block count.  The copies must run before anything
 * else is written into the released blocks, and queued copy-on-write pairs that involve the
 * sequence before the swap.  PA_ERR_NO_BLOCKS if the host pool has too few free blocks,
 * PA_ERR_SHAPE if the sequence is unknown or swapped out or max_pairs is too small. */
pa_status pa_bm_swap_out(pa_block_manager* bm, int32_t seq, int64_t* pairs_out,
                         int64_t max_pairs, int64_t* num_pairs);
/* Swap a sequence back in: each host block, in logical order, gets a fresh device block and
 * the pair (host block, device block) is written to pairs_out (pa_swap_blocks's PA_SWAP_IN
 * mapping); the host blocks return to the host free list.  The sequence's table holds the
 * new blocks (none shared, none in the prefix cache).  PA_ERR_NO_BLOCKS if the device pool
 * has too few free blocks, PA_ERR_SHAPE if the sequence is not swapped out or max_pairs is
 * too small. */
pa_status pa_bm_swap_in(pa_block_manager* bm, int32_t seq, int64_t* pairs_out,
                        int64_t max_pairs, int64_t* num_pairs);

/* Number of queued copy pairs. */
int64_t pa_bm_num_pending_copies(const pa_block_manager* bm);
/* Move up to max_pairs queued pairs, oldest first, into pairs_out (int64 [max_pairs][2]:
 * source, destination: pa_copy_blocks's block_mapping); returns how many were moved, or -1
 * on a NULL argument. */
int64_t pa_bm_take_copies(pa_block_manager* bm, int64_t* pairs_out, int64_t max_pairs);

/*
 * Block tables and context lengths of num_seqs sequences, in the order of seq_ids, for
 * pa_decode: tables_out int32 [num_seqs][max_blocks_per_seq] (entries past a sequence's
 * blocks hold pad_block), context_lens_out int32 [num_seqs].  PA_ERR_SHAPE on an unknown id.
 */
pa_status pa_bm_block_tables(const pa_block_manager* bm, const int32_t* seq_ids, int32_t num_seqs,
                             int32_t pad_block, int32_t* tables_out, int32_t* context_lens_out);

/*
 * Groups of sequences for pa_decode_shared_prefix, over num_seqs sequences in the order of
 * seq_ids (the order of the tables pa_bm_block_tables writes): runs of consecutive sequences
 * each of which holds at least min_blocks leading blocks (the same physical blocks, shared
 * through the prefix cache or a fork: "vLLM 架构源码解析 第1篇" §4.3.1) in common with the
 * sequence before it, counting only blocks that end before the sequence's last token.  A
 * group's count is the smallest of those overlaps (the blocks every member shares with the
 * first); a sequence that overlaps its predecessor by fewer than min_blocks starts a new
 * group, and a group of one sequence gets 0.  groups_out int32 [num_seqs + 1] (group i is
 * sequences [groups_out[i], groups_out[i + 1]) of the order), blocks_out int32 [num_seqs],
 * *num_groups_out = the number of groups.  PA_ERR_SHAPE on an unknown or swapped-out id or
 * min_blocks < 1.
 */
pa_status pa_bm_prefix_groups(const pa_block_manager* bm, const int32_t* seq_ids,
                              int32_t num_seqs, int32_t min_blocks, int32_t* groups_out,
                              int32_t* blocks_out, int32_t* num_groups_out);

#ifdef __cplusplus
}
#endif
#endif /* PA_BLOCK_MANAGER_H */
