// block_manager.cpp - host-side block manager of the paged KV cache: a
// free list, reference counts and per-sequence block tables, with
// copy-on-write of a shared block about to be written, and swapping of
// whole sequences between the device pool and a host pool.  Plain C++; it
// never touches the device.
#include <stdint.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "pkv_blocks.h"

struct pkv_block_manager {
  struct Seq {
    std::vector<int32_t> table;  // logical block -> physical block
    int32_t tokens = 0;
    bool swapped = false;        // the table holds host blocks
  };
  // One pool of blocks: a free stack (top = back()) and reference counts.
  struct Pool {
    std::vector<int32_t> free_stack;
    std::vector<int32_t> ref;
    void init(int32_t n) {
      ref.assign(n, 0);
      free_stack.clear();
      free_stack.reserve(n);
      for (int32_t b = n - 1; b >= 0; --b) free_stack.push_back(b);
    }
    int32_t pop() {
      const int32_t b = free_stack.back();
      free_stack.pop_back();
      ref[b] = 1;
      return b;
    }
  };
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  Pool dev, host;
  std::unordered_map<int64_t, Seq> seqs;

  int32_t pop_free() { return dev.pop(); }
};

namespace {

int64_t slot_of(const pkv_block_manager::Seq &s, int32_t t, int32_t bs) {
  return (int64_t)s.table[t / bs] * bs + t % bs;
}

}  // namespace

extern "C" {

int pkv_bm_create_with_host(int32_t num_blocks, int32_t num_host_blocks, int32_t block_size,
                            pkv_block_manager **out) {
  if (!out) return PKV_ERR_NULL;
  if (num_blocks < 0 || num_host_blocks < 0 || block_size < 1) return PKV_ERR_SHAPE;
  pkv_block_manager *bm = new (std::nothrow) pkv_block_manager();
  if (!bm) return PKV_ERR_SHAPE;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->dev.init(num_blocks);
  bm->host.init(num_host_blocks);
  *out = bm;
  return PKV_OK;
}

int pkv_bm_create(int32_t num_blocks, int32_t block_size, pkv_block_manager **out) {
  return pkv_bm_create_with_host(num_blocks, 0, block_size, out);
}

void pkv_bm_destroy(pkv_block_manager *bm) { delete bm; }

int pkv_bm_add_sequence(pkv_block_manager *bm, int64_t seq_id, int32_t num_tokens,
                        int64_t *slots_out) {
  if (!bm) return PKV_ERR_NULL;
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  if (bm->seqs.count(seq_id)) return PKV_ERR_SEQ_EXISTS;
  const int32_t bs = bm->block_size;
  const int64_t need = ((int64_t)num_tokens + bs - 1) / bs;
  if (need > (int64_t)bm->dev.free_stack.size()) return PKV_ERR_NO_BLOCKS;
  pkv_block_manager::Seq s;
  s.table.reserve((size_t)need);
  for (int64_t i = 0; i < need; ++i) s.table.push_back(bm->pop_free());
  s.tokens = num_tokens;
  if (slots_out)
    for (int32_t t = 0; t < num_tokens; ++t) slots_out[t] = slot_of(s, t, bs);
  bm->seqs.emplace(seq_id, std::move(s));
  return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager *bm, int64_t parent, int64_t child) {
  if (!bm) return PKV_ERR_NULL;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
  if (bm->seqs.count(child)) return PKV_ERR_SEQ_EXISTS;
  if (it->second.swapped) return PKV_ERR_SWAPPED;
  pkv_block_manager::Seq c = it->second;
  for (int32_t b : c.table) ++bm->dev.ref[b];
  bm->seqs.emplace(child, std::move(c));
  return PKV_OK;
}

int pkv_bm_append_tokens(pkv_block_manager *bm, const int64_t *seq_ids, int32_t n,
                         int64_t *slots_out, int64_t *copy_pairs_out,
                         int32_t *num_copies_out) {
  if (!bm || (n > 0 && (!seq_ids || !slots_out || !copy_pairs_out)) || !num_copies_out)
    return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  const int32_t bs = bm->block_size;
  // Dry run: how many fresh blocks does the batch take?  A sequence's last
  // block is private once it got a fresh block earlier in the batch; a
  // shared block's count drops by one with every copy taken from it.
  std::unordered_map<int64_t, int32_t> extra_tokens;
  std::unordered_map<int64_t, bool> last_private;
  std::unordered_map<int32_t, int32_t> ref_drop;
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
    if (it->second.swapped) return PKV_ERR_SWAPPED;
    const int32_t t = it->second.tokens + extra_tokens[seq_ids[i]];
    if (t % bs == 0) {
      ++need;
      last_private[seq_ids[i]] = true;
    } else if (!last_private[seq_ids[i]]) {
      const int32_t last = it->second.table.back();
      if (bm->dev.ref[last] - ref_drop[last] > 1) {
        ++need;
        ++ref_drop[last];
      }
      last_private[seq_ids[i]] = true;
    }
    ++extra_tokens[seq_ids[i]];
  }
  if (need > (int64_t)bm->dev.free_stack.size()) return PKV_ERR_NO_BLOCKS;

  int32_t copies = 0;
  for (int32_t i = 0; i < n; ++i) {
    pkv_block_manager::Seq &s = bm->seqs.find(seq_ids[i])->second;
    const int32_t t = s.tokens;
    if (t % bs == 0) {
      s.table.push_back(bm->pop_free());
    } else {
      const int32_t last = s.table.back();
      if (bm->dev.ref[last] > 1) {
        const int32_t fresh = bm->pop_free();
        --bm->dev.ref[last];
        s.table.back() = fresh;
        copy_pairs_out[2 * copies] = last;
        copy_pairs_out[2 * copies + 1] = fresh;
        ++copies;
      }
    }
    slots_out[i] = slot_of(s, t, bs);
    s.tokens = t + 1;
  }
  *num_copies_out = copies;
  return PKV_OK;
}

int pkv_bm_free_sequence(pkv_block_manager *bm, int64_t seq_id) {
  if (!bm) return PKV_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
  const std::vector<int32_t> &table = it->second.table;
  pkv_block_manager::Pool &pool = it->second.swapped ? bm->host : bm->dev;
  for (auto b = table.rbegin(); b != table.rend(); ++b)
    if (--pool.ref[*b] == 0) pool.free_stack.push_back(*b);
  bm->seqs.erase(it);
  return PKV_OK;
}

namespace {

// Move the listed sequences between the pools (to_host: device to host,
// else host to device).  See pkv_bm_swap_out.
int move_sequences(pkv_block_manager *bm, const int64_t *seq_ids, int32_t n, int64_t *pairs_out,
                   int32_t max_pairs, int32_t *num_pairs_out, bool to_host) {
  if (!bm || !num_pairs_out || (n > 0 && !seq_ids)) return PKV_ERR_NULL;
  if (n < 0 || max_pairs < 0) return PKV_ERR_SHAPE;
  pkv_block_manager::Pool &from = to_host ? bm->dev : bm->host;
  pkv_block_manager::Pool &to = to_host ? bm->host : bm->dev;
  // distinct sequences in list order
  std::vector<int64_t> ids;
  std::unordered_map<int64_t, bool> seen;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
    if (it->second.swapped == to_host) return PKV_ERR_SWAPPED;
    if (!seen[seq_ids[i]]) {
      seen[seq_ids[i]] = true;
      ids.push_back(seq_ids[i]);
    }
  }
  // distinct blocks in order of first appearance, with their holder counts
  std::vector<int32_t> blocks;
  std::unordered_map<int32_t, int32_t> holders;
  for (int64_t id : ids)
    for (int32_t b : bm->seqs.find(id)->second.table)
      if (holders[b]++ == 0) blocks.push_back(b);
  for (int32_t b : blocks)
    if (holders[b] != from.ref[b]) return PKV_ERR_SHARED;
  if (blocks.size() > to.free_stack.size()) return PKV_ERR_NO_BLOCKS;
  if ((int64_t)blocks.size() > (int64_t)max_pairs) return PKV_ERR_CAPACITY;
  if (!blocks.empty() && !pairs_out) return PKV_ERR_NULL;

  std::unordered_map<int32_t, int32_t> moved;
  for (size_t i = 0; i < blocks.size(); ++i) {
    const int32_t b = blocks[i], nb = to.pop();
    to.ref[nb] = from.ref[b];
    moved[b] = nb;
    pairs_out[2 * i] = b;
    pairs_out[2 * i + 1] = nb;
  }
  for (int64_t id : ids) {
    pkv_block_manager::Seq &s = bm->seqs.find(id)->second;
    for (int32_t &b : s.table) b = moved[b];
    s.swapped = to_host;
  }
  // the old blocks return to their free stack so that the first one moved
  // is the next one handed out
  for (auto b = blocks.rbegin(); b != blocks.rend(); ++b) {
    from.ref[*b] = 0;
    from.free_stack.push_back(*b);
  }
  *num_pairs_out = (int32_t)blocks.size();
  return PKV_OK;
}

}  // namespace

int pkv_bm_swap_out(pkv_block_manager *bm, const int64_t *seq_ids, int32_t n, int64_t *pairs_out,
                    int32_t max_pairs, int32_t *num_pairs_out) {
  return move_sequences(bm, seq_ids, n, pairs_out, max_pairs, num_pairs_out, true);
}

int pkv_bm_swap_in(pkv_block_manager *bm, const int64_t *seq_ids, int32_t n, int64_t *pairs_out,
                   int32_t max_pairs, int32_t *num_pairs_out) {
  return move_sequences(bm, seq_ids, n, pairs_out, max_pairs, num_pairs_out, false);
}

int pkv_bm_batch_tables(const pkv_block_manager *bm, const int64_t *seq_ids, int32_t n,
                        int32_t max_blocks, int32_t *tables_out,
                        int32_t *context_lens_out) {
  if (!bm || (n > 0 && (!seq_ids || !tables_out || !context_lens_out))) return PKV_ERR_NULL;
  if (n < 0 || max_blocks < 0) return PKV_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
    if (it->second.swapped) return PKV_ERR_SWAPPED;
    if ((int64_t)it->second.table.size() > max_blocks) return PKV_ERR_CAPACITY;
  }
  for (int32_t i = 0; i < n; ++i) {
    const pkv_block_manager::Seq &s = bm->seqs.find(seq_ids[i])->second;
    int32_t *row = tables_out + (size_t)i * max_blocks;
    for (int32_t j = 0; j < max_blocks; ++j)
      row[j] = j < (int32_t)s.table.size() ? s.table[j] : -1;
    context_lens_out[i] = s.tokens;
  }
  return PKV_OK;
}

int32_t pkv_bm_num_free_blocks(const pkv_block_manager *bm) {
  return bm ? (int32_t)bm->dev.free_stack.size() : -1;
}

int32_t pkv_bm_num_free_host_blocks(const pkv_block_manager *bm) {
  return bm ? (int32_t)bm->host.free_stack.size() : -1;
}

int32_t pkv_bm_refcount(const pkv_block_manager *bm, int32_t block) {
  if (!bm || block < 0 || block >= (int32_t)bm->dev.ref.size()) return -1;
  return bm->dev.ref[block];
}

int32_t pkv_bm_host_refcount(const pkv_block_manager *bm, int32_t block) {
  if (!bm || block < 0 || block >= (int32_t)bm->host.ref.size()) return -1;
  return bm->host.ref[block];
}

int32_t pkv_bm_is_swapped(const pkv_block_manager *bm, int64_t seq_id) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq_id);
  return it == bm->seqs.end() ? -1 : (it->second.swapped ? 1 : 0);
}

int pkv_bm_block_table(const pkv_block_manager *bm, int64_t seq_id, int32_t *table_out,
                       int32_t max_blocks, int32_t *num_blocks_out) {
  if (!bm || !num_blocks_out) return PKV_ERR_NULL;
  if (max_blocks < 0) return PKV_ERR_SHAPE;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
  const std::vector<int32_t> &t = it->second.table;
  if ((int64_t)t.size() > max_blocks) return PKV_ERR_CAPACITY;
  if (!t.empty() && !table_out) return PKV_ERR_NULL;
  for (size_t j = 0; j < t.size(); ++j) table_out[j] = t[j];
  *num_blocks_out = (int32_t)t.size();
  return PKV_OK;
}

int32_t pkv_bm_num_tokens(const pkv_block_manager *bm, int64_t seq_id) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq_id);
  return it == bm->seqs.end() ? -1 : it->second.tokens;
}

}  // extern "C"
