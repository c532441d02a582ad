// Host-side block manager for the paged KV cache (PagedAttention, tutorial
// "Chapter 3 Advanced principles", section 3.0 and its sections on sharing:
// the cache is cut into fixed-size physical blocks, each sequence has a
// table of block ids, sequences forked for parallel sampling or beam search
// share their prefix blocks, and a shared block is copied before it is
// written -- copy-on-write).
//
// The manager only does the bookkeeping: it hands out physical slots for new
// tokens, counts references per block and tells the caller which block copies
// to run (paged_kv_copy_blocks) before writing (paged_kv_write).  Full blocks
// stay shared after a fork; only a partially filled last block that is shared
// is copied when a sequence appends to it.  Free blocks are reused last-freed
// first, so the same calls give the same block ids.
#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/attn.h"

namespace attn {
int set_error(int code, const std::string& msg);   // attn_api.hip
}

struct attn_block_manager {
  int num_blocks = 0, block_size = 0;
  std::vector<int32_t> free_list;   // stack of free block ids
  std::vector<int32_t> refs;        // references per block
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t len = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;

  int32_t take() {
    const int32_t b = free_list.back();
    free_list.pop_back();
    refs[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--refs[b] == 0) free_list.push_back(b);
  }
};

namespace {
int bad(const char* fn, int code, const std::string& msg) {
  return attn::set_error(code, std::string(fn) + ": " + msg);
}
}  // namespace

extern "C" {

int attn_bm_create(int num_blocks, int block_size, attn_block_manager** out) {
  if (out == nullptr) return bad("attn_bm_create", ATTN_ERR_NULL, "out must not be NULL");
  *out = nullptr;
  if (num_blocks < 0 || block_size <= 0 || (int64_t)num_blocks * block_size > INT32_MAX)
    return bad("attn_bm_create", ATTN_ERR_SHAPE,
               "num_blocks >= 0, block_size > 0 and num_blocks * block_size < 2^31 required");
  try {
    auto* m = new attn_block_manager();
    m->num_blocks = num_blocks;
    m->block_size = block_size;
    m->refs.assign(num_blocks, 0);
    m->free_list.reserve(num_blocks);
    for (int b = num_blocks - 1; b >= 0; --b) m->free_list.push_back(b);   // block 0 first
    *out = m;
    return attn::set_error(ATTN_OK, "");
  } catch (...) {
    return bad("attn_bm_create", ATTN_ERR_NO_BLOCKS, "host allocation failed");
  }
}

void attn_bm_destroy(attn_block_manager* m) { delete m; }

int attn_bm_num_free(const attn_block_manager* m) {
  return m == nullptr ? -1 : (int)m->free_list.size();
}

int attn_bm_ref_count(const attn_block_manager* m, int block) {
  if (m == nullptr || block < 0 || block >= m->num_blocks) return -1;
  return m->refs[block];
}

int64_t attn_bm_length(const attn_block_manager* m, int64_t seq_id) {
  if (m == nullptr) return -1;
  auto it = m->seqs.find(seq_id);
  return it == m->seqs.end() ? -1 : it->second.len;
}

int attn_bm_add_sequence(attn_block_manager* m, int64_t seq_id) {
  const char* fn = "attn_bm_add_sequence";
  if (m == nullptr) return bad(fn, ATTN_ERR_NULL, "manager must not be NULL");
  try {
    if (!m->seqs.emplace(seq_id, attn_block_manager::Seq{}).second)
      return bad(fn, ATTN_ERR_SHAPE, "sequence " + std::to_string(seq_id) + " already exists");
  } catch (...) {
    return bad(fn, ATTN_ERR_NO_BLOCKS, "host allocation failed");
  }
  return attn::set_error(ATTN_OK, "");
}

int attn_bm_fork(attn_block_manager* m, int64_t parent, int64_t child) {
  const char* fn = "attn_bm_fork";
  if (m == nullptr) return bad(fn, ATTN_ERR_NULL, "manager must not be NULL");
  auto it = m->seqs.find(parent);
  if (it == m->seqs.end()) return bad(fn, ATTN_ERR_SHAPE, "unknown parent sequence");
  if (m->seqs.count(child)) return bad(fn, ATTN_ERR_SHAPE, "child sequence already exists");
  try {
    attn_block_manager::Seq s = it->second;   // copy before inserting (rehash)
    for (int32_t b : s.blocks) ++m->refs[b];
    m->seqs.emplace(child, std::move(s));
  } catch (...) {
    return bad(fn, ATTN_ERR_NO_BLOCKS, "host allocation failed");
  }
  return attn::set_error(ATTN_OK, "");
}

int attn_bm_append(attn_block_manager* m, int64_t seq_id, int n_tokens, int32_t* slots,
                   int32_t* copy_src, int32_t* copy_dst, int* n_copies) {
  const char* fn = "attn_bm_append";
  if (m == nullptr || n_copies == nullptr || copy_src == nullptr || copy_dst == nullptr ||
      (n_tokens > 0 && slots == nullptr))
    return bad(fn, ATTN_ERR_NULL, "manager, slots and copy outputs must not be NULL");
  *n_copies = 0;
  if (n_tokens < 0) return bad(fn, ATTN_ERR_SHAPE, "n_tokens must be non-negative");
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return bad(fn, ATTN_ERR_SHAPE, "unknown sequence");
  auto& s = it->second;
  const int64_t bs = m->block_size, len = s.len;
  if (n_tokens == 0) return attn::set_error(ATTN_OK, "");
  // blocks needed: new ones past the current table, plus one copy when the
  // partially filled last block is shared
  const bool cow = (len % bs) != 0 && m->refs[s.blocks.back()] > 1;
  const int64_t have = (int64_t)s.blocks.size();
  const int64_t after = (len + n_tokens + bs - 1) / bs;
  const int64_t need = (after - have) + (cow ? 1 : 0);
  if (need > (int64_t)m->free_list.size())
    return bad(fn, ATTN_ERR_NO_BLOCKS,
               "needs " + std::to_string(need) + " free blocks, " +
                   std::to_string(m->free_list.size()) + " left");
  try {
    s.blocks.reserve(after);
  } catch (...) {
    return bad(fn, ATTN_ERR_NO_BLOCKS, "host allocation failed");
  }
  if (cow) {
    const int32_t old = s.blocks.back(), fresh = m->take();
    copy_src[0] = old;
    copy_dst[0] = fresh;
    *n_copies = 1;
    m->drop(old);
    s.blocks.back() = fresh;
  }
  for (int i = 0; i < n_tokens; ++i) {
    const int64_t pos = len + i, lb = pos / bs;
    if (lb == (int64_t)s.blocks.size()) s.blocks.push_back(m->take());
    slots[i] = (int32_t)(s.blocks[lb] * bs + pos % bs);
  }
  s.len = len + n_tokens;
  return attn::set_error(ATTN_OK, "");
}

int attn_bm_free_sequence(attn_block_manager* m, int64_t seq_id) {
  const char* fn = "attn_bm_free_sequence";
  if (m == nullptr) return bad(fn, ATTN_ERR_NULL, "manager must not be NULL");
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return bad(fn, ATTN_ERR_SHAPE, "unknown sequence");
  for (int32_t b : it->second.blocks) m->drop(b);
  m->seqs.erase(it);
  return attn::set_error(ATTN_OK, "");
}

int attn_bm_block_table(const attn_block_manager* m, const int64_t* seq_ids, int n,
                        int max_blocks, int32_t* table, int32_t* context_lens) {
  const char* fn = "attn_bm_block_table";
  if (m == nullptr || (n > 0 && (seq_ids == nullptr || table == nullptr || context_lens == nullptr)))
    return bad(fn, ATTN_ERR_NULL, "arguments must not be NULL");
  if (n < 0 || max_blocks < 0) return bad(fn, ATTN_ERR_SHAPE, "sizes must be non-negative");
  for (int i = 0; i < n; ++i) {
    auto it = m->seqs.find(seq_ids[i]);
    if (it == m->seqs.end()) return bad(fn, ATTN_ERR_SHAPE, "unknown sequence");
    if ((int64_t)it->second.blocks.size() > max_blocks)
      return bad(fn, ATTN_ERR_SHAPE, "a sequence has more than max_blocks blocks");
    if (it->second.len > INT32_MAX) return bad(fn, ATTN_ERR_SHAPE, "sequence too long");
  }
  for (int i = 0; i < n; ++i) {
    const auto& s = m->seqs.find(seq_ids[i])->second;
    int32_t* row = table + (int64_t)i * max_blocks;
    for (int j = 0; j < max_blocks; ++j) row[j] = j < (int)s.blocks.size() ? s.blocks[j] : -1;
    context_lens[i] = (int32_t)s.len;
  }
  return attn::set_error(ATTN_OK, "");
}

}  // extern "C"
