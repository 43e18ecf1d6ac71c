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
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/pkv.h"
#include "pkv_internal.h"

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
    std::vector<int32_t> table;  // ceil(len / block_size) live entries
  };
  std::unordered_map<int64_t, Seq> seqs;

  int32_t pop_free() {
    int32_t b = ring[head];
    head = (head + 1) % num_blocks;
    --free_count;
    return b;
  }
  void push_free(int32_t b) {
    ring[(head + free_count) % num_blocks] = b;
    ++free_count;
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
                        int32_t* copy_dst, int32_t* num_copies, const char* fn) {
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
  if (need > bm->free_count)
    return pkv_fail(PKV_ERR_OUT_OF_BLOCKS, std::string(fn) + ": KV cache full");
  int32_t copies = 0;
  for (int32_t i = 0; i < n; ++i) {
    pkv_block_manager::Seq* q = target[i];
    int32_t p = q->len;
    if (p % BS == 0) {
      int32_t b = bm->pop_free();
      bm->ref[b] = 1;
      q->table.push_back(b);
    } else if (cow && bm->ref[q->table[p / BS]] > 1) {
      const int32_t old = q->table[p / BS];
      const int32_t b = bm->pop_free();
      bm->ref[b] = 1;
      bm->ref[old] -= 1;  // stays >= 1: another sequence holds it
      q->table[p / BS] = b;
      copy_src[copies] = old;
      copy_dst[copies] = b;
      ++copies;
    }
    slot_mapping_out[i] = (int64_t)q->table[p / BS] * BS + p % BS;
    q->len = p + 1;
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

pkv_status pkv_bm_free_seq(pkv_block_manager* bm, int64_t seq_id) {
  if (!bm) return pkv_fail(PKV_ERR_INVALID_ARG, "pkv_bm_free_seq: NULL manager");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return pkv_fail(PKV_ERR_UNKNOWN_SEQ, "pkv_bm_free_seq: unknown id");
  for (int32_t b : it->second.table) {
    if (--bm->ref[b] == 0) bm->push_free(b);
  }
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

int32_t pkv_bm_num_free_blocks(const pkv_block_manager* bm) { return bm ? bm->free_count : -1; }

int32_t pkv_bm_refcount(const pkv_block_manager* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[block];
}

}  // extern "C"
