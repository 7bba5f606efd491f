// block_manager.cpp — host-side block manager of the paged KV cache (include/pa_block_manager.h).
//
// Free list: a vector used as a stack, so taking and returning a block are O(1) at its tail
// ("vLLM 深度拆解：当 KV Cache 学会「分页」" §3.2).  Reference counts per block, sequences as
// vectors of physical block ids (their block tables), and a prefix cache keyed exactly by
// (preceding physical block, the block's token ids) ("vLLM 架构源码解析 第1篇" §4.3.1).  Every
// entry point checks first and mutates only once it cannot fail, so a failed call leaves the
// state unchanged.
#include "pa_block_manager.h"

#include <stdint.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <vector>

namespace {

struct KeyHash {
  size_t operator()(const std::vector<int32_t>& k) const {
    uint64_t h = 1469598103934665603ull;  // FNV-1a over the key's 32-bit words
    for (int32_t v : k) {
      h ^= (uint32_t)v;
      h *= 1099511628211ull;
    }
    return (size_t)h;
  }
};

struct Seq {
  bool live = false;
  bool swapped = false;           // its blocks are in host memory (host), not on the device
  bool track = true;              // every token so far came with an id: full blocks may be cached
  int32_t len = 0;
  std::vector<int32_t> blocks;    // logical block j -> physical block
  std::vector<int32_t> tail;      // token ids of the partly filled last block (when tracked)
  std::vector<int32_t> host;      // while swapped: logical block j -> host block
};

}  // namespace

struct pa_block_manager {
  int32_t num_blocks, block_size, max_blocks;
  std::vector<int32_t> free_list;  // taken from and returned to the back
  std::vector<int32_t> ref;        // per block
  std::vector<Seq> seqs;
  std::vector<int32_t> free_ids;   // released sequence ids, reused last-in first-out
  std::unordered_map<std::vector<int32_t>, int32_t, KeyHash> cache;  // key -> block
  std::vector<std::vector<int32_t>> key_of;  // block -> its key in the cache (empty: none)
  std::vector<int64_t> copies;     // queued (source, destination) pairs, flattened
  int32_t num_host = 0;            // host blocks for swapped-out sequences
  std::vector<int32_t> host_free;  // free host blocks, taken from and returned to the back
  size_t copies_head = 0;          // pairs before this index have been taken

  int32_t take_block() {
    const int32_t b = free_list.back();
    free_list.pop_back();
    ref[b] = 1;
    return b;
  }

  void drop_ref(int32_t b) {
    if (--ref[b] == 0) {
      if (!key_of[b].empty()) {
        cache.erase(key_of[b]);
        key_of[b].clear();
      }
      free_list.push_back(b);
    }
  }

  std::vector<int32_t> key(int32_t parent, const int32_t* tokens) const {
    std::vector<int32_t> k((size_t)block_size + 1);
    k[0] = parent;
    for (int32_t i = 0; i < block_size; ++i) k[i + 1] = tokens[i];
    return k;
  }

  // register a full block under (parent, tokens) unless that key already names a block; the
  // cache only saves recomputation, so a block that cannot be registered (no host memory) is
  // simply not shared
  void remember(int32_t block, int32_t parent, const int32_t* tokens) noexcept {
    try {
      std::vector<int32_t> k = key(parent, tokens);
      if (cache.count(k) || !key_of[block].empty()) return;
      std::vector<int32_t> mine = k;
      cache.emplace(std::move(k), block);
      key_of[block] = std::move(mine);
    } catch (const std::bad_alloc&) {
    }
  }

  // a sequence whose blocks are on the device (what every call but the swap, free and length
  // queries works on)
  Seq* seq(int32_t id) {
    Seq* s = any_seq(id);
    return s && !s->swapped ? s : nullptr;
  }
  const Seq* seq(int32_t id) const {
    const Seq* s = any_seq(id);
    return s && !s->swapped ? s : nullptr;
  }
  // a live sequence, on the device or swapped out
  Seq* any_seq(int32_t id) {
    return id >= 0 && id < (int32_t)seqs.size() && seqs[id].live ? &seqs[id] : nullptr;
  }
  const Seq* any_seq(int32_t id) const {
    return id >= 0 && id < (int32_t)seqs.size() && seqs[id].live ? &seqs[id] : nullptr;
  }

  int32_t new_seq_id() {
    if (!free_ids.empty()) {
      const int32_t id = free_ids.back();
      free_ids.pop_back();
      return id;
    }
    seqs.emplace_back();
    return (int32_t)seqs.size() - 1;
  }

  int64_t blocks_for(int64_t tokens) const { return (tokens + block_size - 1) / block_size; }
};

extern "C" {

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq) {
  if (num_blocks <= 0 || block_size <= 0 || max_blocks_per_seq <= 0) return nullptr;
  try {
    pa_block_manager* bm = new pa_block_manager();
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->max_blocks = max_blocks_per_seq;
    bm->free_list.resize(num_blocks);
    for (int32_t i = 0; i < num_blocks; ++i) bm->free_list[i] = i;
    bm->ref.assign(num_blocks, 0);
    bm->key_of.resize(num_blocks);
    return bm;
  } catch (const std::bad_alloc&) {
    return nullptr;
  }
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int32_t pa_bm_num_free_blocks(const pa_block_manager* bm) {
  return bm ? (int32_t)bm->free_list.size() : -1;
}

int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[block];
}

int32_t pa_bm_seq_len(const pa_block_manager* bm, int32_t seq) {
  const Seq* s = bm ? bm->any_seq(seq) : nullptr;
  return s ? s->len : -1;
}

pa_status pa_bm_add_sequence(pa_block_manager* bm, const int32_t* token_ids, int32_t num_tokens,
                             int32_t* seq_id, int32_t* num_cached_tokens) {
  if (!bm || !seq_id || !num_cached_tokens) return PA_ERR_NULL;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  const int32_t BS = bm->block_size;
  const int64_t nblk = bm->blocks_for(num_tokens);
  if (nblk > bm->max_blocks) return PA_ERR_SHAPE;
  try {
    // cached leading blocks: full blocks that end before the prompt's last token
    std::vector<int32_t> hits;
    if (token_ids) {
      const int32_t reusable = num_tokens > 0 ? (num_tokens - 1) / BS : 0;
      int32_t parent = -1;
      for (int32_t j = 0; j < reusable; ++j) {
        auto it = bm->cache.find(bm->key(parent, token_ids + (int64_t)j * BS));
        if (it == bm->cache.end()) break;
        hits.push_back(it->second);
        parent = it->second;
      }
    }
    const int64_t fresh = nblk - (int64_t)hits.size();
    if (fresh > (int64_t)bm->free_list.size()) return PA_ERR_NO_BLOCKS;
    // build the sequence aside, then commit: nothing below the reservations can throw
    Seq s;
    s.live = true;
    s.track = token_ids != nullptr;
    s.len = num_tokens;
    s.blocks.reserve(nblk);
    if (token_ids) {
      s.tail.reserve(BS);
      s.tail.assign(token_ids + (int64_t)(num_tokens / BS) * BS, token_ids + num_tokens);
    }
    bm->seqs.reserve(bm->seqs.size() + 1);
    const int32_t id = bm->new_seq_id();
    for (int32_t b : hits) {
      ++bm->ref[b];
      s.blocks.push_back(b);
    }
    for (int64_t j = (int64_t)hits.size(); j < nblk; ++j) {
      const int32_t b = bm->take_block();
      s.blocks.push_back(b);
      if (token_ids && (j + 1) * BS <= num_tokens)
        bm->remember(b, j ? s.blocks[j - 1] : -1, token_ids + j * BS);
    }
    bm->seqs[id] = std::move(s);
    *seq_id = id;
    *num_cached_tokens = (int32_t)hits.size() * BS;
    return PA_OK;
  } catch (const std::bad_alloc&) {
    return PA_ERR_NO_BLOCKS;
  }
}

pa_status pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t* child_id) {
  if (!bm || !child_id) return PA_ERR_NULL;
  if (!bm->seq(parent)) return PA_ERR_SHAPE;
  try {
    Seq c = bm->seqs[parent];  // same blocks, length and pending tail tokens
    bm->seqs.reserve(bm->seqs.size() + 1);
    const int32_t id = bm->new_seq_id();
    for (int32_t b : c.blocks) ++bm->ref[b];
    bm->seqs[id] = std::move(c);
    *child_id = id;
    return PA_OK;
  } catch (const std::bad_alloc&) {
    return PA_ERR_NO_BLOCKS;
  }
}

pa_status pa_bm_append(pa_block_manager* bm, int32_t seq, const int32_t* token_ids,
                       int32_t num_tokens, int64_t* slots_out) {
  if (!bm) return PA_ERR_NULL;
  Seq* s = bm->seq(seq);
  if (!s || num_tokens < 0) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!slots_out) return PA_ERR_NULL;
  const int32_t BS = bm->block_size;
  const int64_t L = s->len, total = L + num_tokens;
  const int64_t need = bm->blocks_for(total);
  if (need > bm->max_blocks) return PA_ERR_SHAPE;
  const bool cow = L % BS != 0 && bm->ref[s->blocks.back()] > 1;
  const int64_t fresh = need - (int64_t)s->blocks.size() + (cow ? 1 : 0);
  if (fresh > (int64_t)bm->free_list.size()) return PA_ERR_NO_BLOCKS;
  try {
    s->blocks.reserve(need);
    s->tail.reserve(BS);
    if (cow) bm->copies.reserve(bm->copies.size() + 2);
    if (cow) {  // move onto a private copy of the shared, partly filled last block
      const int32_t old = s->blocks.back();
      const int32_t b = bm->take_block();
      bm->copies.push_back(old);
      bm->copies.push_back(b);
      --bm->ref[old];  // still referenced by another sequence: never reaches zero here
      s->blocks.back() = b;
    }
    if (!token_ids) {
      s->track = false;
      s->tail.clear();
    }
    for (int32_t i = 0; i < num_tokens; ++i) {
      const int64_t pos = L + i;
      const int64_t j = pos / BS;
      if (j == (int64_t)s->blocks.size()) s->blocks.push_back(bm->take_block());
      slots_out[i] = (int64_t)s->blocks[j] * BS + pos % BS;
      if (s->track) {
        s->tail.push_back(token_ids[i]);
        if ((int32_t)s->tail.size() == BS) {
          bm->remember(s->blocks[j], j ? s->blocks[j - 1] : -1, s->tail.data());
          s->tail.clear();
        }
      }
    }
    s->len = (int32_t)total;
    return PA_OK;
  } catch (const std::bad_alloc&) {
    return PA_ERR_NO_BLOCKS;
  }
}

pa_status pa_bm_slots(const pa_block_manager* bm, int32_t seq, int32_t first, int32_t count,
                      int64_t* slots_out) {
  if (!bm) return PA_ERR_NULL;
  const Seq* s = bm->seq(seq);
  if (!s || first < 0 || count < 0 || (int64_t)first + count > s->len) return PA_ERR_SHAPE;
  if (count == 0) return PA_OK;
  if (!slots_out) return PA_ERR_NULL;
  const int32_t BS = bm->block_size;
  for (int32_t i = 0; i < count; ++i) {
    const int64_t pos = (int64_t)first + i;
    slots_out[i] = (int64_t)s->blocks[pos / BS] * BS + pos % BS;
  }
  return PA_OK;
}

pa_status pa_bm_free_sequence(pa_block_manager* bm, int32_t seq) {
  if (!bm) return PA_ERR_NULL;
  Seq* s = bm->any_seq(seq);
  if (!s) return PA_ERR_SHAPE;
  try {
    bm->free_ids.reserve(bm->free_ids.size() + 1);
  } catch (const std::bad_alloc&) {
    return PA_ERR_NO_BLOCKS;
  }
  // host blocks go back in reverse (capacity for all of them was reserved at creation)
  for (size_t j = s->host.size(); j-- > 0;) bm->host_free.push_back(s->host[j]);
  // last block first: a block is never freed before the blocks that follow it in a table
  for (size_t j = s->blocks.size(); j-- > 0;) bm->drop_ref(s->blocks[j]);
  *s = Seq();
  bm->free_ids.push_back(seq);
  return PA_OK;
}

pa_status pa_bm_set_host_blocks(pa_block_manager* bm, int32_t num_host_blocks) {
  if (!bm) return PA_ERR_NULL;
  if (num_host_blocks < 0) return PA_ERR_SHAPE;
  for (const Seq& s : bm->seqs)
    if (s.live && s.swapped) return PA_ERR_SHAPE;  // host blocks in use
  try {
    std::vector<int32_t> f((size_t)num_host_blocks);
    for (int32_t i = 0; i < num_host_blocks; ++i) f[i] = i;
    bm->host_free = std::move(f);
  } catch (const std::bad_alloc&) {
    return PA_ERR_NO_BLOCKS;
  }
  bm->num_host = num_host_blocks;
  return PA_OK;
}

int32_t pa_bm_num_free_host_blocks(const pa_block_manager* bm) {
  return bm ? (int32_t)bm->host_free.size() : -1;
}

pa_status pa_bm_swap_out(pa_block_manager* bm, int32_t seq, int64_t* pairs_out,
                         int64_t max_pairs, int64_t* num_pairs) {
  if (!bm || !num_pairs) return PA_ERR_NULL;
  Seq* s = bm->seq(seq);
  if (!s) return PA_ERR_SHAPE;
  const size_t nb = s->blocks.size();
  if (nb > bm->host_free.size()) return PA_ERR_NO_BLOCKS;
  if ((int64_t)nb > max_pairs) return PA_ERR_SHAPE;
  if (nb > 0 && !pairs_out) return PA_ERR_NULL;
  try {
    s->host.reserve(nb);
  } catch (const std::bad_alloc&) {
    return PA_ERR_NO_BLOCKS;
  }
  for (size_t j = 0; j < nb; ++j) {
    const int32_t h = bm->host_free.back();
    bm->host_free.pop_back();
    s->host.push_back(h);
    pairs_out[2 * j] = s->blocks[j];
    pairs_out[2 * j + 1] = h;
  }
  // the device blocks are released like a free (last first); shared ones stay with the others
  for (size_t j = nb; j-- > 0;) bm->drop_ref(s->blocks[j]);
  s->blocks.clear();
  s->swapped = true;
  *num_pairs = (int64_t)nb;
  return PA_OK;
}

pa_status pa_bm_swap_in(pa_block_manager* bm, int32_t seq, int64_t* pairs_out,
                        int64_t max_pairs, int64_t* num_pairs) {
  if (!bm || !num_pairs) return PA_ERR_NULL;
  Seq* s = bm->any_seq(seq);
  if (!s || !s->swapped) return PA_ERR_SHAPE;
  const size_t nb = s->host.size();
  if (nb > bm->free_list.size()) return PA_ERR_NO_BLOCKS;
  if ((int64_t)nb > max_pairs) return PA_ERR_SHAPE;
  if (nb > 0 && !pairs_out) return PA_ERR_NULL;
  try {
    s->blocks.reserve(nb);
  } catch (const std::bad_alloc&) {
    return PA_ERR_NO_BLOCKS;
  }
  for (size_t j = 0; j < nb; ++j) {
    const int32_t b = bm->take_block();
    s->blocks.push_back(b);
    pairs_out[2 * j] = s->host[j];
    pairs_out[2 * j + 1] = b;
  }
  for (size_t j = nb; j-- > 0;) bm->host_free.push_back(s->host[j]);
  s->host.clear();
  s->swapped = false;
  *num_pairs = (int64_t)nb;
  return PA_OK;
}

int64_t pa_bm_num_pending_copies(const pa_block_manager* bm) {
  return bm ? (int64_t)(bm->copies.size() / 2 - bm->copies_head) : -1;
}

int64_t pa_bm_take_copies(pa_block_manager* bm, int64_t* pairs_out, int64_t max_pairs) {
  if (!bm || (!pairs_out && max_pairs > 0)) return -1;
  const int64_t avail = (int64_t)(bm->copies.size() / 2 - bm->copies_head);
  const int64_t n = max_pairs < avail ? (max_pairs > 0 ? max_pairs : 0) : avail;
  for (int64_t i = 0; i < 2 * n; ++i) pairs_out[i] = bm->copies[2 * bm->copies_head + i];
  bm->copies_head += (size_t)n;
  if (bm->copies_head * 2 == bm->copies.size()) {
    bm->copies.clear();
    bm->copies_head = 0;
  }
  return n;
}

pa_status pa_bm_block_tables(const pa_block_manager* bm, const int32_t* seq_ids, int32_t num_seqs,
                             int32_t pad_block, int32_t* tables_out, int32_t* context_lens_out) {
  if (!bm) return PA_ERR_NULL;
  if (num_seqs < 0) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!seq_ids || !tables_out || !context_lens_out) return PA_ERR_NULL;
  for (int32_t i = 0; i < num_seqs; ++i)
    if (!bm->seq(seq_ids[i])) return PA_ERR_SHAPE;
  const int32_t MB = bm->max_blocks;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Seq& s = *bm->seq(seq_ids[i]);
    int32_t* row = tables_out + (int64_t)i * MB;
    const int32_t n = (int32_t)s.blocks.size();
    for (int32_t j = 0; j < MB; ++j) row[j] = j < n ? s.blocks[j] : pad_block;
    context_lens_out[i] = s.len;
  }
  return PA_OK;
}

pa_status pa_bm_prefix_groups(const pa_block_manager* bm, const int32_t* seq_ids,
                              int32_t num_seqs, int32_t min_blocks, int32_t* groups_out,
                              int32_t* blocks_out, int32_t* num_groups_out) {
  if (!bm || !num_groups_out) return PA_ERR_NULL;
  if (num_seqs < 0 || min_blocks < 1) return PA_ERR_SHAPE;
  if (num_seqs == 0) {
    *num_groups_out = 0;
    if (groups_out) groups_out[0] = 0;
    return PA_OK;
  }
  if (!seq_ids || !groups_out || !blocks_out) return PA_ERR_NULL;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Seq* s = bm->seq(seq_ids[i]);
    if (!s || s->swapped) return PA_ERR_SHAPE;
  }
  // blocks that end before the sequence's last token
  auto full = [&](const Seq& s) { return s.len > 0 ? (s.len - 1) / bm->block_size : 0; };
  int32_t ng = 0, start = 0;
  groups_out[0] = 0;
  int32_t common = full(*bm->seq(seq_ids[0]));
  auto close = [&](int32_t end) {
    blocks_out[ng] = end - start > 1 ? common : 0;
    groups_out[++ng] = end;
    start = end;
  };
  for (int32_t i = 1; i < num_seqs; ++i) {
    const Seq& a = *bm->seq(seq_ids[i - 1]);
    const Seq& b = *bm->seq(seq_ids[i]);
    const int32_t lim = std::min(std::min(full(a), full(b)), common);
    int32_t l = 0;
    while (l < lim && a.blocks[l] == b.blocks[l]) ++l;
    if (l >= min_blocks) {
      common = l;  // l <= common: the blocks every member shares with the first
    } else {
      close(i);
      common = full(b);
    }
  }
  close(num_seqs);
  *num_groups_out = ng;
  return PA_OK;
}

}  // extern "C"
