// Host-side KV block manager (C ABI in include/pa_block_manager.h).
//
// Blocks of one pool are handed to sequences, freed at the end of a request
// and handed out again ("Nano-vLLM：轻量高效的大模型推理框架…", 三.1, 块管理器).
// Prefix caching ("Nano-vLLM…", 三.2 (1) 前缀缓存): a full block's key is a
// 64-bit hash chained over the token ids of every block up to it; a sequence
// whose leading full blocks match cached ones (hash and token ids) reuses them.
// Freed blocks keep their key until they are handed out again, least recently
// freed first, so a later request with the same prefix can still hit them.
#include <stdint.h>

#include <list>
#include <unordered_map>
#include <vector>

#include "pa_block_manager.h"

namespace {

constexpr uint64_t kNoHash = 0;

// 64-bit chained hash over int32 token ids (FNV-1a over bytes, then a final mix).
uint64_t chain_hash(uint64_t prev, const int32_t* tok, int32_t n) {
  uint64_t h = 1469598103934665603ull ^ prev;
  for (int32_t i = 0; i < n; ++i) {
    uint32_t v = static_cast<uint32_t>(tok[i]);
    for (int b = 0; b < 4; ++b) {
      h ^= (v >> (8 * b)) & 0xffu;
      h *= 1099511628211ull;
    }
  }
  h ^= h >> 33;
  h *= 0xff51afd7ed558ccdull;
  h ^= h >> 33;
  return h == kNoHash ? 1 : h;
}

struct Block {
  int32_t ref = 0;
  uint64_t hash = kNoHash;           // set while the block is registered for reuse
  std::vector<int32_t> tokens;       // token ids of a registered (full) block
  std::list<int32_t>::iterator free_pos;
  bool in_free = false;
};

struct Seq {
  std::vector<int32_t> table;
  std::vector<int32_t> tokens;
  std::vector<uint64_t> block_hash;  // chain hash of each full block (kNoHash if not full)
};

}  // namespace

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  bool prefix_caching = false;
  std::vector<Block> blocks;
  std::list<int32_t> free_list;      // front = next to hand out
  std::unordered_map<uint64_t, int32_t> cached;
  std::unordered_map<int64_t, Seq> seqs;
  int64_t next_id = 1;

  void push_free(int32_t b) {
    blocks[b].free_pos = free_list.insert(free_list.end(), b);
    blocks[b].in_free = true;
  }
  void take_free(int32_t b) {
    free_list.erase(blocks[b].free_pos);
    blocks[b].in_free = false;
  }
  void unregister(int32_t b) {
    Block& blk = blocks[b];
    if (blk.hash != kNoHash) {
      auto it = cached.find(blk.hash);
      if (it != cached.end() && it->second == b) cached.erase(it);
      blk.hash = kNoHash;
      blk.tokens.clear();
    }
  }
  // hands out the least recently freed block; its cached key (if any) is dropped
  int32_t allocate() {
    const int32_t b = free_list.front();
    take_free(b);
    unregister(b);
    blocks[b].ref = 1;
    return b;
  }
  void reg(int32_t b, uint64_t h, const int32_t* tok) {
    if (!prefix_caching) return;
    if (cached.count(h)) return;  // an equal block is already cached
    blocks[b].hash = h;
    blocks[b].tokens.assign(tok, tok + block_size);
    cached[h] = b;
  }
  int32_t lookup(uint64_t h, const int32_t* tok) const {
    auto it = cached.find(h);
    if (it == cached.end()) return -1;
    const Block& blk = blocks[it->second];
    for (int32_t i = 0; i < block_size; ++i)
      if (blk.tokens[i] != tok[i]) return -1;
    return it->second;
  }
  void release(int32_t b) {
    if (--blocks[b].ref == 0) push_free(b);
  }
};

extern "C" {

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t enable_prefix_caching,
                       pa_block_manager** out) {
  if (!out) return PA_ERR_NULL;
  if (num_blocks <= 0 || block_size <= 0) return PA_ERR_SHAPE;
  if (enable_prefix_caching != 0 && enable_prefix_caching != 1) return PA_ERR_SHAPE;
  pa_block_manager* bm = new pa_block_manager;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->prefix_caching = enable_prefix_caching == 1;
  bm->blocks.resize(num_blocks);
  for (int32_t b = 0; b < num_blocks; ++b) bm->push_free(b);
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int32_t pa_bm_num_free_blocks(const pa_block_manager* bm) {
  return bm ? static_cast<int32_t>(bm->free_list.size()) : 0;
}

pa_status pa_bm_add_sequence(pa_block_manager* bm, const int32_t* tokens, int32_t num_tokens,
                             int64_t* seq_id, int32_t* num_cached_tokens) {
  if (!bm || !seq_id || !num_cached_tokens || (num_tokens > 0 && !tokens)) return PA_ERR_NULL;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  const int32_t bs = bm->block_size;
  const int32_t nblk = (num_tokens + bs - 1) / bs;
  // plan: which leading full blocks hit the cache
  std::vector<int32_t> hits;
  std::vector<uint64_t> hashes(nblk, kNoHash);
  uint64_t h = 0;
  bool hitting = bm->prefix_caching;
  for (int32_t j = 0; j < nblk; ++j) {
    const bool full = (j + 1) * bs <= num_tokens;
    if (!full) break;
    h = chain_hash(h, tokens + j * bs, bs);
    hashes[j] = h;
    if (hitting) {
      const int32_t b = bm->lookup(h, tokens + j * bs);
      if (b >= 0) hits.push_back(b); else hitting = false;
    }
  }
  // free blocks needed: the misses, plus hit blocks that currently sit in the free list
  int32_t reclaimed = 0;
  for (int32_t b : hits) reclaimed += bm->blocks[b].in_free ? 1 : 0;
  const int32_t misses = nblk - static_cast<int32_t>(hits.size());
  if (misses + reclaimed > static_cast<int32_t>(bm->free_list.size())) return PA_ERR_NO_BLOCKS;
  Seq seq;
  seq.tokens.assign(tokens, tokens + num_tokens);
  seq.block_hash = hashes;
  for (int32_t b : hits) {
    if (bm->blocks[b].in_free) bm->take_free(b);
    ++bm->blocks[b].ref;
    seq.table.push_back(b);
  }
  for (int32_t j = static_cast<int32_t>(hits.size()); j < nblk; ++j) {
    const int32_t b = bm->allocate();
    if (hashes[j] != kNoHash) bm->reg(b, hashes[j], tokens + j * bs);
    seq.table.push_back(b);
  }
  const int64_t id = bm->next_id++;
  bm->seqs.emplace(id, std::move(seq));
  *seq_id = id;
  *num_cached_tokens = static_cast<int32_t>(hits.size()) * bs;
  return PA_OK;
}

pa_status pa_bm_append_token(pa_block_manager* bm, int64_t seq_id, int32_t token, int32_t* slot,
                             int32_t* cow_src, int32_t* cow_dst) {
  if (!bm || !slot || !cow_src || !cow_dst) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  Seq& s = it->second;
  const int32_t bs = bm->block_size;
  const int32_t pos = static_cast<int32_t>(s.tokens.size());
  *cow_src = *cow_dst = -1;
  if (pos % bs == 0) {
    if (bm->free_list.empty()) return PA_ERR_NO_BLOCKS;
    s.table.push_back(bm->allocate());
    s.block_hash.push_back(kNoHash);
  } else {
    const int32_t last = s.table.back();
    if (bm->blocks[last].ref > 1) {  // shared partial block: write into a private copy
      if (bm->free_list.empty()) return PA_ERR_NO_BLOCKS;
      const int32_t copy = bm->allocate();
      --bm->blocks[last].ref;
      s.table.back() = copy;
      *cow_src = last;
      *cow_dst = copy;
    }
  }
  s.tokens.push_back(token);
  *slot = s.table.back() * bs + pos % bs;
  // a block that just became full gets its chained key
  if ((pos + 1) % bs == 0) {
    const int32_t j = pos / bs;
    const uint64_t prev = j > 0 ? s.block_hash[j - 1] : 0;
    const uint64_t h = (j == 0 || prev != kNoHash) ? chain_hash(prev, s.tokens.data() + j * bs, bs) : kNoHash;
    s.block_hash[j] = h;
    if (h != kNoHash) bm->reg(s.table.back(), h, s.tokens.data() + j * bs);
  }
  return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager* bm, int64_t seq_id, int64_t* new_seq_id) {
  if (!bm || !new_seq_id) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  Seq copy = it->second;
  for (int32_t b : copy.table) ++bm->blocks[b].ref;
  const int64_t id = bm->next_id++;
  bm->seqs.emplace(id, std::move(copy));
  *new_seq_id = id;
  return PA_OK;
}

pa_status pa_bm_free_sequence(pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  // last blocks first, so a sequence's prefix blocks are the last to be handed out again
  const std::vector<int32_t>& t = it->second.table;
  for (auto b = t.rbegin(); b != t.rend(); ++b) bm->release(*b);
  bm->seqs.erase(it);
  return PA_OK;
}

pa_status pa_bm_sequence_info(const pa_block_manager* bm, int64_t seq_id, int32_t* num_tokens,
                              int32_t* num_blocks) {
  if (!bm || !num_tokens || !num_blocks) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  *num_tokens = static_cast<int32_t>(it->second.tokens.size());
  *num_blocks = static_cast<int32_t>(it->second.table.size());
  return PA_OK;
}

pa_status pa_bm_block_table(const pa_block_manager* bm, int64_t seq_id, int32_t* row,
                            int32_t max_blocks, int32_t pad_block) {
  if (!bm || (max_blocks > 0 && !row)) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  const std::vector<int32_t>& t = it->second.table;
  if (static_cast<int32_t>(t.size()) > max_blocks) return PA_ERR_SHAPE;
  for (int32_t j = 0; j < max_blocks; ++j) row[j] = j < static_cast<int32_t>(t.size()) ? t[j] : pad_block;
  return PA_OK;
}

pa_status pa_bm_slots(const pa_block_manager* bm, int64_t seq_id, int32_t first_pos, int32_t count,
                      int32_t* slots) {
  if (!bm || (count > 0 && !slots)) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  const Seq& s = it->second;
  const int32_t bs = bm->block_size;
  if (first_pos < 0 || count < 0 || first_pos + count > static_cast<int32_t>(s.table.size()) * bs)
    return PA_ERR_SHAPE;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t p = first_pos + i;
    slots[i] = s.table[p / bs] * bs + p % bs;
  }
  return PA_OK;
}

int32_t pa_bm_block_refcount(const pa_block_manager* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->blocks[block].ref;
}

}  // extern "C"
