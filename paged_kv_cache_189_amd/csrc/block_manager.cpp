// Host block manager: the per-sequence block tables of a paged KV cache.
//
// "Optimizing Llama 3.1 405B Inference with vLLM PagedAttention", section
// "PagedAttention Mechanics": every sequence has a page table; appending a
// token takes a fresh physical page only when the sequence needs one; several
// sequences can point at the same physical pages (shared prefixes).
// "vLLM PagedAttention: Memory Optimization & High-Throughput LLM Inference
// Tuning", §2 (logical blocks map to physical blocks through a block table)
// and §4 (a finished request's blocks are freed at once).
//
// Policy choices the pages leave open: free blocks are a FIFO ring seeded with
// a caller-given order; freed blocks rejoin at the tail in table order; an
// append batch is all-or-nothing; appending into a partially filled block that
// is shared is refused by pkv_bm_append_slots, and resolved by copy-on-write
// in pkv_bm_append_slots_cow (the sequence takes a fresh block, the caller
// copies the shared block's contents into it on the device).
//
// Plain C++17 with no HIP dependency.
#include <cstdint>
#include <cstring>
#include <list>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/pkv.h"
#include "pkv_internal.h"

// Prefix cache.  A full block of a sequence whose token ids are known is
// registered under its content: its block_size token ids and its parent, the
// registered block of the previous logical block (none for block 0), so a
// lookup that walks a prompt block by block matches exactly the blocks whose
// whole token prefix equals the prompt's.  A 64-bit chain hash (FNV-1a over
// the parent's hash and the ids, then a splitmix64 finish) only narrows the
// search.  Registered blocks whose reference count drops to 0 stay cached in
// an LRU list; allocation takes the free queue first, then evicts the least
// recently released cached block.  Evicting a block also drops its cached
// descendants (they are only reachable through it): the block, then its
// descendants depth first, join the free queue.
struct CacheEntry {
  bool cached = false;
  uint64_t hash = 0;
  int32_t parent = -1;
  std::vector<int32_t> tokens;
  std::vector<int32_t> children;  // in registration order
  bool in_lru = false;
  std::list<int32_t>::iterator lru_pos;
};

struct pkv_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  int32_t max_blocks = 0;
  std::vector<int32_t> ring;  // free FIFO: ring[(head + i) % num_blocks], i < free_count
  int32_t head = 0;
  int32_t free_count = 0;
  std::vector<int32_t> ref;
  struct Seq {
    int32_t len = 0;
    std::vector<int32_t> table;   // ceil(len / block_size) live entries
    bool tracked = false;         // token ids known: full blocks are registered
    std::vector<int32_t> tokens;  // the ids, when tracked
  };
  std::unordered_map<int64_t, Seq> seqs;
  std::vector<CacheEntry> cache;                  // per physical block
  std::unordered_multimap<uint64_t, int32_t> by_hash;
  std::list<int32_t> lru;                         // cached blocks with no reference, oldest first
  int32_t num_cached = 0;

  int32_t available() const { return free_count + (int32_t)lru.size(); }

  void push_free(int32_t b) {
    ring[(head + free_count) % num_blocks] = b;
    ++free_count;
  }
  // Drops b and its cached descendants from the cache; unreferenced ones join
  // the free queue (b first, then descendants depth first).
  void uncache(int32_t b) {
    CacheEntry& e = cache[b];
    auto range = by_hash.equal_range(e.hash);
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == b) {
        by_hash.erase(it);
        break;
      }
    e.cached = false;
    --num_cached;
    if (e.in_lru) {
      lru.erase(e.lru_pos);
      e.in_lru = false;
      push_free(b);
    }
    std::vector<int32_t> kids;
    kids.swap(e.children);
    for (int32_t c : kids) uncache(c);
  }
  // A block for a new table entry: the free queue's head, else the least
  // recently released cached block (evicted with its descendants).
  int32_t pop_block() {
    if (free_count == 0) {
      const int32_t victim = lru.front();
      const int32_t parent = cache[victim].parent;
      if (parent >= 0 && cache[parent].cached) {
        auto& ch = cache[parent].children;
        for (size_t i = 0; i < ch.size(); ++i)
          if (ch[i] == victim) {
            ch.erase(ch.begin() + (long)i);
            break;
          }
      }
      uncache(victim);
    }
    int32_t b = ring[head];
    head = (head + 1) % num_blocks;
    --free_count;
    return b;
  }
  // One reference fewer; at 0 a cached block waits in the LRU list, others
  // rejoin the free queue.
  void release(int32_t b) {
    if (--ref[b] != 0) return;
    CacheEntry& e = cache[b];
    if (e.cached) {
      lru.push_back(b);
      e.lru_pos = std::prev(lru.end());
      e.in_lru = true;
    } else {
      push_free(b);
    }
  }
  // One reference more (a cached block leaves the LRU list).
  void acquire(int32_t b) {
    CacheEntry& e = cache[b];
    if (ref[b]++ == 0 && e.in_lru) {
      lru.erase(e.lru_pos);
      e.in_lru = false;
    }
  }

  static uint64_t chain_hash(uint64_t parent_hash, const int32_t* ids, int32_t n) {
    uint64_t h = 1469598103934665603ull;  // FNV-1a offset basis
    auto mix = [&](uint64_t v) {
      for (int k = 0; k < 8; ++k) {
        h ^= (v >> (8 * k)) & 0xFFu;
        h *= 1099511628211ull;  // FNV-1a prime
      }
    };
    mix(parent_hash);
    for (int32_t i = 0; i < n; ++i) mix((uint64_t)(uint32_t)ids[i]);
    h ^= h >> 30;  // splitmix64 finish
    h *= 0xbf58476d1ce4e5b9ull;
    h ^= h >> 27;
    h *= 0x94d049bb133111ebull;
    h ^= h >> 31;
    return h;
  }
  uint64_t hash_of(int32_t parent, const int32_t* ids) const {
    return chain_hash(parent >= 0 ? cache[parent].hash : 0, ids, block_size);
  }
  // The cached block holding `ids` after `parent` (-1: none).
  int32_t lookup(int32_t parent, const int32_t* ids) const {
    const uint64_t h = hash_of(parent, ids);
    auto range = by_hash.equal_range(h);
    for (auto it = range.first; it != range.second; ++it) {
      const CacheEntry& e = cache[it->second];
      if (e.parent == parent && std::memcmp(e.tokens.data(), ids, sizeof(int32_t) * block_size) == 0)
        return it->second;
    }
    return -1;
  }
  // Registers full block `b` (logical block i of a tracked sequence) unless
  // its parent is not the cached block of that prefix or an equal block is
  // already cached.
  void register_block(const Seq& q, int32_t i) {
    const int32_t b = q.table[i];
    const int32_t parent = i > 0 ? q.table[i - 1] : -1;
    if (cache[b].cached || (parent >= 0 && !cache[parent].cached)) return;
    const int32_t* ids = q.tokens.data() + (int64_t)i * block_size;
    if (lookup(parent, ids) >= 0) return;
    CacheEntry& e = cache[b];
    e.cached = true;
    e.hash = hash_of(parent, ids);
    e.parent = parent;
    e.tokens.assign(ids, ids + block_size);
    e.children.clear();
    by_hash.emplace(e.hash, b);
    if (parent >= 0) cache[parent].children.push_back(b);
    ++num_cached;
  }
};

extern "C" {

pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                         const int32_t* free_order, pkv_block_manager** out) {
  if (!out) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_bm_create: out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0 || max_blocks_per_seq <= 0)
    return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_bm_create: sizes must be positive");
  auto* bm = new (std::nothrow) pkv_block_manager();
  if (!bm) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_bm_create: out of host memory");
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->max_blocks = max_blocks_per_seq;
  bm->ring.resize(num_blocks);
  bm->ref.assign(num_blocks, 0);
  bm->cache.resize(num_blocks);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return pkv_fail(PKV_ERR_INVALID_ARG,
                        "pkv_bm_create: free_order is not a permutation of the blocks");
      }
      seen[b] = 1;
      bm->ring[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) bm->ring[i] = i;
  }
  bm->free_count = num_blocks;
  *out = bm;
  return PKV_OK;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

pkv_status pkv_bm_add_seq(pkv_block_manager* bm, int64_t seq_id) {
  if (!bm) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_bm_add_seq: NULL manager");
  if (bm->seqs.count(seq_id)) return pkv_fail(PKV_ERR_SEQ_EXISTS, "pkv_bm_add_seq: id is live");
  bm->seqs.emplace(seq_id, pkv_block_manager::Seq{});
  return PKV_OK;
}

pkv_status pkv_bm_fork_seq(pkv_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_bm_fork_seq: NULL manager");
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return pkv_fail(PKV_ERR_UNKNOWN_SEQ, "pkv_bm_fork_seq: no parent");
  if (bm->seqs.count(child)) return pkv_fail(PKV_ERR_SEQ_EXISTS, "pkv_bm_fork_seq: child is live");
  pkv_block_manager::Seq c = it->second;  // copy of table and length
  for (int32_t b : c.table) bm->ref[b] += 1;
  bm->seqs.emplace(child, std::move(c));
  return PKV_OK;
}

}  // extern "C"

namespace {

// One append batch.  cow == false: SHARED_TAIL refuses a batch that would
// write into a partially filled shared block.  cow == true: the first token
// such a sequence receives takes a fresh block first; the shared block loses
// one reference and (old, new) is reported as a copy.
pkv_status append_batch(pkv_block_manager* bm, const int64_t* seq_ids, int32_t n,
                        int64_t* slot_mapping_out, bool cow, int32_t* copy_src,
                        int32_t* copy_dst, int32_t* num_copies, const char* fn,
                        const int32_t* token_ids = nullptr) {
  if (!bm) return pkv_fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": NULL manager");
  if (n < 0 || (n > 0 && (!seq_ids || !slot_mapping_out)) ||
      (cow && (!num_copies || (n > 0 && (!copy_src || !copy_dst)))))
    return pkv_fail(PKV_ERR_INVALID_ARG, std::string(fn) + ": bad list");
  const int32_t BS = bm->block_size;
  // Dry run: resolve every id, count the blocks the batch takes, and check
  // that nothing would fail, before touching any state.
  std::vector<pkv_block_manager::Seq*> target(n);
  std::unordered_map<pkv_block_manager::Seq*, int32_t> pending;
  std::unordered_map<int32_t, int32_t> released;  // references dropped by earlier copies
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end())
      return pkv_fail(PKV_ERR_UNKNOWN_SEQ, std::string(fn) + ": unknown sequence id");
    pkv_block_manager::Seq* q = &it->second;
    target[i] = q;
    int32_t& extra = pending[q];
    int64_t p = (int64_t)q->len + extra;
    if (p / BS >= bm->max_blocks)
      return pkv_fail(PKV_ERR_INVALID_ARG,
                      std::string(fn) + ": sequence would outgrow max_blocks_per_seq");
    if (p % BS == 0) {
      ++need;
    } else if (extra == 0) {
      const int32_t tail = q->table[p / BS];
      auto rel = released.find(tail);
      if (bm->ref[tail] - (rel == released.end() ? 0 : rel->second) > 1) {
        if (!cow)
          return pkv_fail(PKV_ERR_SHARED_TAIL,
                          std::string(fn) + ": last block is partially filled and shared");
        ++need;  // its private copy
        ++released[tail];
      }
    }
    ++extra;
  }
  if (need > bm->available())
    return pkv_fail(PKV_ERR_OUT_OF_BLOCKS, std::string(fn) + ": KV cache full");
  int32_t copies = 0;
  for (int32_t i = 0; i < n; ++i) {
    pkv_block_manager::Seq* q = target[i];
    int32_t p = q->len;
    if (p % BS == 0) {
      int32_t b = bm->pop_block();
      bm->ref[b] = 1;
      q->table.push_back(b);
    } else if (cow && bm->ref[q->table[p / BS]] > 1) {
      const int32_t old = q->table[p / BS];
      const int32_t b = bm->pop_block();
      bm->ref[b] = 1;
      bm->ref[old] -= 1;  // stays >= 1: another sequence holds it
      q->table[p / BS] = b;
      copy_src[copies] = old;
      copy_dst[copies] = b;
      ++copies;
    }
    slot_mapping_out[i] = (int64_t)q->table[p / BS] * BS + p % BS;
    q->len = p + 1;
    if (token_ids && q->tracked) {
      q->tokens.push_back(token_ids[i]);
      if ((p + 1) % BS == 0) bm->register_block(*q, p / BS);
    } else {
      q->tracked = false;  // ids unknown from here on
      q->tokens.clear();
    }
  }
  if (cow) *num_copies = copies;
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_bm_append_slots(pkv_block_manager* bm, const int64_t* seq_ids, int32_t n,
                               int64_t* slot_mapping_out) {
  return append_batch(bm, seq_ids, n, slot_mapping_out, false, nullptr, nullptr, nullptr,
                      "pkv_bm_append_slots");
}

pkv_status pkv_bm_append_slots_cow(pkv_block_manager* bm, const int64_t* seq_ids, int32_t n,
                                   int64_t* slot_mapping_out, int32_t* copy_src_out,
                                   int32_t* copy_dst_out, int32_t* num_copies_out) {
  return append_batch(bm, seq_ids, n, slot_mapping_out, true, copy_src_out, copy_dst_out,
                      num_copies_out, "pkv_bm_append_slots_cow");
}

pkv_status pkv_bm_append_tokens(pkv_block_manager* bm, const int64_t* seq_ids,
                                const int32_t* token_ids, int32_t n, int64_t* slot_mapping_out) {
  if (n > 0 && !token_ids) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_bm_append_tokens: NULL token ids");
  return append_batch(bm, seq_ids, n, slot_mapping_out, false, nullptr, nullptr, nullptr,
                      "pkv_bm_append_tokens", token_ids);
}

pkv_status pkv_bm_add_seq_prompt(pkv_block_manager* bm, int64_t seq_id, const int32_t* token_ids,
                                 int32_t n, int64_t* slot_mapping_out, int32_t* num_cached_out) {
  if (!bm) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_bm_add_seq_prompt: NULL manager");
  if (n < 0 || (n > 0 && (!token_ids || !slot_mapping_out)) || !num_cached_out)
    return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_bm_add_seq_prompt: bad arguments");
  if (bm->seqs.count(seq_id)) return pkv_fail(PKV_ERR_SEQ_EXISTS, "pkv_bm_add_seq_prompt: id is live");
  const int32_t BS = bm->block_size;
  const int64_t nblk = ((int64_t)n + BS - 1) / BS;
  if (nblk > bm->max_blocks)
    return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_bm_add_seq_prompt: prompt outgrows max_blocks_per_seq");
  // longest chain of cached full blocks; the last prompt token is always
  // computed, so at most (n - 1) / BS blocks are reused
  std::vector<int32_t> hit;
  const int32_t limit = n > 0 ? (n - 1) / BS : 0;
  int32_t parent = -1;
  for (int32_t i = 0; i < limit; ++i) {
    const int32_t b = bm->lookup(parent, token_ids + (int64_t)i * BS);
    if (b < 0) break;
    hit.push_back(b);
    parent = b;
  }
  int32_t from_lru = 0;
  for (int32_t b : hit) from_lru += bm->ref[b] == 0;
  if (nblk - (int64_t)hit.size() > bm->available() - from_lru)
    return pkv_fail(PKV_ERR_OUT_OF_BLOCKS, "pkv_bm_add_seq_prompt: KV cache full");
  pkv_block_manager::Seq q;
  q.tracked = true;
  for (int32_t b : hit) {
    bm->acquire(b);
    q.table.push_back(b);
  }
  const int32_t cached_tokens = (int32_t)hit.size() * BS;
  q.tokens.assign(token_ids, token_ids + cached_tokens);
  q.len = cached_tokens;
  for (int32_t t = 0; t < cached_tokens; ++t)
    slot_mapping_out[t] = (int64_t)q.table[t / BS] * BS + t % BS;
  auto& slot = bm->seqs.emplace(seq_id, std::move(q)).first->second;
  for (int32_t t = cached_tokens; t < n; ++t) {
    if (t % BS == 0) {
      const int32_t b = bm->pop_block();
      bm->ref[b] = 1;
      slot.table.push_back(b);
    }
    slot_mapping_out[t] = (int64_t)slot.table[t / BS] * BS + t % BS;
    slot.tokens.push_back(token_ids[t]);
    slot.len = t + 1;
    if ((t + 1) % BS == 0) bm->register_block(slot, t / BS);
  }
  *num_cached_out = cached_tokens;
  return PKV_OK;
}

pkv_status pkv_bm_free_seq(pkv_block_manager* bm, int64_t seq_id) {
  if (!bm) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_bm_free_seq: NULL manager");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return pkv_fail(PKV_ERR_UNKNOWN_SEQ, "pkv_bm_free_seq: unknown id");
  for (int32_t b : it->second.table) bm->release(b);
  bm->seqs.erase(it);
  return PKV_OK;
}

pkv_status pkv_bm_export(const pkv_block_manager* bm, const int64_t* seq_ids, int32_t n,
                         int32_t* block_tables_out, int32_t* context_lens_out) {
  if (!bm) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_bm_export: NULL manager");
  if (n < 0 || (n > 0 && !seq_ids)) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_bm_export: bad list");
  for (int32_t i = 0; i < n; ++i)
    if (!bm->seqs.count(seq_ids[i]))
      return pkv_fail(PKV_ERR_UNKNOWN_SEQ, "pkv_bm_export: unknown sequence id");
  for (int32_t i = 0; i < n; ++i) {
    const auto& q = bm->seqs.at(seq_ids[i]);
    if (block_tables_out) {
      int32_t* row = block_tables_out + (int64_t)i * bm->max_blocks;
      int32_t nb = (int32_t)q.table.size();
      for (int32_t j = 0; j < bm->max_blocks; ++j) row[j] = j < nb ? q.table[j] : -1;
    }
    if (context_lens_out) context_lens_out[i] = q.len;
  }
  return PKV_OK;
}

int32_t pkv_bm_num_free_blocks(const pkv_block_manager* bm) { return bm ? bm->available() : -1; }

int32_t pkv_bm_num_cached_blocks(const pkv_block_manager* bm) { return bm ? bm->num_cached : -1; }

int32_t pkv_bm_refcount(const pkv_block_manager* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[block];
}

}  // extern "C"
