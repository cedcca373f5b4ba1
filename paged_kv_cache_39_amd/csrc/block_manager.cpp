// Host-side block manager: allocation of cache blocks to sequences,
// reference-counted sharing and copy-on-write, and the block_table /
// slot_mapping producers. Declared in include/pkv_block_manager.h, which
// states the rules and the passages they follow.
//
// Data layout: per block a reference count and a "locked" flag (named by a
// copy not yet taken); a bitmap of allocatable blocks (count 0, not locked)
// scanned from the lowest word that can hold a set bit, so taking the
// lowest-numbered free block costs one word scan in the common case.

#include <limits.h>
#include <stdint.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pagedkv.h"
#include "pkv_block_manager.h"

struct pkv_block_manager {
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t len = 0;
  };

  int64_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> ref;
  std::vector<uint8_t> locked;        // named by a pending copy
  std::vector<uint8_t> pending_dst;   // destination of a pending copy
  std::vector<uint64_t> free_bits;    // allocatable: ref == 0 and not locked
  int64_t n_free = 0;                 // ref == 0
  int64_t n_alloc = 0;                // allocatable
  int64_t hint = 0;                   // no set bit below word `hint`
  std::unordered_map<int64_t, Seq> seqs;
  std::vector<std::pair<int32_t, int32_t>> pending;

  void set_bit(int64_t b) {
    free_bits[b >> 6] |= 1ull << (b & 63);
    hint = std::min(hint, b >> 6);
    ++n_alloc;
  }
  void clear_bit(int64_t b) {
    free_bits[b >> 6] &= ~(1ull << (b & 63));
    --n_alloc;
  }
  int32_t take_free() {   // caller checked n_alloc > 0
    int64_t w = hint;
    while (free_bits[w] == 0) ++w;
    hint = w;
    const int64_t b = (w << 6) + __builtin_ctzll(free_bits[w]);
    clear_bit(b);
    ref[b] = 1;
    --n_free;
    return (int32_t)b;
  }
  void release(int32_t b) {
    if (--ref[b] == 0) {
      ++n_free;
      if (!locked[b]) set_bit(b);
    }
  }
  void lock(int32_t b) {
    if (locked[b]) return;
    locked[b] = 1;
    if (ref[b] == 0) clear_bit(b);
  }
};

extern "C" {

pkv_block_manager* pkv_bm_create(int64_t num_blocks, int32_t block_size) {
  if (num_blocks <= 0) return nullptr;
  if (block_size != 16 && block_size != 32 && block_size != 64 && block_size != 128)
    return nullptr;
  if (num_blocks > (int64_t)INT32_MAX / block_size) return nullptr;
  pkv_block_manager* bm = new (std::nothrow) pkv_block_manager;
  if (!bm) return nullptr;
  try {
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->ref.assign(num_blocks, 0);
    bm->locked.assign(num_blocks, 0);
    bm->pending_dst.assign(num_blocks, 0);
    bm->free_bits.assign((num_blocks + 63) / 64, 0);
    for (int64_t b = 0; b < num_blocks; ++b) bm->free_bits[b >> 6] |= 1ull << (b & 63);
    bm->n_free = bm->n_alloc = num_blocks;
  } catch (...) {
    delete bm;
    return nullptr;
  }
  return bm;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id) {
  if (!bm) return PKV_ERR_NULL;
  if (bm->seqs.count(seq_id)) return PKV_ERR_SHAPE;
  bm->seqs.emplace(seq_id, pkv_block_manager::Seq{});
  return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager* bm, int64_t parent_id, int64_t child_id) {
  if (!bm) return PKV_ERR_NULL;
  auto it = bm->seqs.find(parent_id);
  if (it == bm->seqs.end() || bm->seqs.count(child_id)) return PKV_ERR_SHAPE;
  pkv_block_manager::Seq child = it->second;   // copy before inserting (rehash)
  for (int32_t b : child.blocks) ++bm->ref[b];
  bm->seqs.emplace(child_id, std::move(child));
  return PKV_OK;
}

int pkv_bm_append(pkv_block_manager* bm, int64_t seq_id, int64_t num_tokens, int32_t* slots_out) {
  if (!bm) return PKV_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end() || num_tokens < 0) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!slots_out) return PKV_ERR_NULL;
  auto& s = it->second;
  const int64_t bs = bm->block_size;
  const bool cow = (s.len % bs) != 0 && bm->ref[s.blocks.back()] > 1;
  if (cow && bm->pending_dst[s.blocks.back()]) return PKV_ERR_PENDING_COPY;
  if (num_tokens > bm->num_blocks * bs) return PKV_ERR_NO_BLOCKS;   // (keeps the sum below in range)
  const int64_t need_total = (s.len + num_tokens + bs - 1) / bs;
  const int64_t new_blocks = need_total - (int64_t)s.blocks.size();
  if (new_blocks + (cow ? 1 : 0) > bm->n_alloc) return PKV_ERR_NO_BLOCKS;
  if (cow) {
    const int32_t old = s.blocks.back();
    const int32_t fresh = bm->take_free();
    bm->pending.emplace_back(old, fresh);
    bm->pending_dst[fresh] = 1;
    bm->lock(old);
    bm->lock(fresh);
    s.blocks.back() = fresh;
    bm->release(old);
  }
  for (int64_t i = 0; i < new_blocks; ++i) s.blocks.push_back(bm->take_free());
  for (int64_t p = s.len, i = 0; i < num_tokens; ++p, ++i)
    slots_out[i] = (int32_t)(s.blocks[p / bs] * bs + p % bs);
  s.len += num_tokens;
  return PKV_OK;
}

int64_t pkv_bm_append_each(pkv_block_manager* bm, const int64_t* seq_ids, int64_t num_seqs,
                           int64_t tokens_each, int32_t* slots_out) {
  if (!bm) return PKV_ERR_NULL;
  if (num_seqs < 0 || tokens_each < 0) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return 0;
  if (!seq_ids || (tokens_each > 0 && !slots_out)) return PKV_ERR_NULL;
  for (int64_t i = 0; i < num_seqs; ++i) {
    if (pkv_bm_append(bm, seq_ids[i], tokens_each, slots_out + i * tokens_each) != PKV_OK)
      return i;
  }
  return num_seqs;
}

int pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq_id) {
  if (!bm) return PKV_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PKV_ERR_SHAPE;
  for (int32_t b : it->second.blocks) bm->release(b);
  bm->seqs.erase(it);
  return PKV_OK;
}

int64_t pkv_bm_num_free_blocks(const pkv_block_manager* bm) { return bm ? bm->n_free : -1; }

int64_t pkv_bm_sequence_length(const pkv_block_manager* bm, int64_t seq_id) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq_id);
  return it == bm->seqs.end() ? -1 : it->second.len;
}

int32_t pkv_bm_ref_count(const pkv_block_manager* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[block];
}

int pkv_bm_block_table(const pkv_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs,
                       int32_t max_blocks_per_seq, int32_t* table_out, int32_t* lens_out) {
  if (!bm) return PKV_ERR_NULL;
  if (num_seqs < 0 || max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!seq_ids || !table_out || !lens_out) return PKV_ERR_NULL;
  std::vector<const pkv_block_manager::Seq*> rows(num_seqs);
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end() || (int64_t)it->second.blocks.size() > max_blocks_per_seq)
      return PKV_ERR_SHAPE;
    rows[i] = &it->second;
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    int32_t* row = table_out + (int64_t)i * max_blocks_per_seq;
    const auto& b = rows[i]->blocks;
    std::copy(b.begin(), b.end(), row);
    std::fill(row + b.size(), row + max_blocks_per_seq, -1);
    lens_out[i] = (int32_t)rows[i]->len;
  }
  return PKV_OK;
}

int64_t pkv_bm_num_pending_copies(const pkv_block_manager* bm) {
  return bm ? (int64_t)bm->pending.size() : -1;
}

int64_t pkv_bm_take_copies(pkv_block_manager* bm, int32_t* pairs_out, int64_t max_pairs) {
  if (!bm) return PKV_ERR_NULL;
  const int64_t n = (int64_t)bm->pending.size();
  if (n > max_pairs) return PKV_ERR_SHAPE;
  if (n && !pairs_out) return PKV_ERR_NULL;
  for (int64_t i = 0; i < n; ++i) {
    const auto [src, dst] = bm->pending[i];
    pairs_out[2 * i] = src;
    pairs_out[2 * i + 1] = dst;
    for (int32_t b : {src, dst}) {
      if (!bm->locked[b]) continue;
      bm->locked[b] = 0;
      if (bm->ref[b] == 0) bm->set_bit(b);
    }
    bm->pending_dst[dst] = 0;
  }
  bm->pending.clear();
  return n;
}

}  // extern "C"
