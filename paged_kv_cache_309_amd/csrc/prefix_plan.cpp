// prefix_plan.cpp - host-side search for sets of sequences that share their
// leading blocks (pkv_prefix_plan, declared in pkv_prefix.h).
//
// A prefix shared through the block tables - forks of one prompt, requests
// with the same system prompt - maps the same leading logical blocks of
// every sharer to the same physical blocks ("PagedAttention: how vLLM
// manages the KV cache", section "Copy-on-write makes shared prefixes
// practical").  Sequences are grouped by their first physical block; a
// group's shared prefix is the longest run of leading entries that all its
// members map alike and that lies wholly inside every member's context.
#include <stddef.h>
#include <stdint.h>

#include <unordered_map>
#include <vector>

#include "pkv_blocks.h"
#include "pkv_prefix.h"

extern "C" int pkv_prefix_plan(const int32_t *block_tables, const int32_t *context_lens,
                               int num_seqs, int max_blocks_per_seq, int block_size,
                               int min_sharers, int32_t *plan, size_t plan_capacity,
                               pkv_prefix_info *info) {
  if (!info || !plan || (num_seqs > 0 && (!block_tables || !context_lens)))
    return PKV_ERR_NULL;
  if (block_size <= 0) return PKV_ERR_BLOCK_SIZE;
  if (num_seqs < 0 || max_blocks_per_seq < 0 || min_sharers < 2) return PKV_ERR_SHAPE;
  const size_t S = (size_t)num_seqs, MB = (size_t)max_blocks_per_seq;

  // full blocks of sequence s inside its context (and its table)
  auto full_blocks = [&](size_t s) -> int64_t {
    int64_t L = context_lens[s];
    if (L < 0) L = 0;
    const int64_t f = L / block_size;
    return f < (int64_t)MB ? f : (int64_t)MB;
  };

  // sets keyed by the first physical block, in order of first appearance
  std::unordered_map<int32_t, size_t> set_of_block;
  std::vector<std::vector<int32_t>> sets;
  for (size_t s = 0; s < S; ++s) {
    if (full_blocks(s) < 1) continue;
    const int32_t first = block_tables[s * MB];
    auto it = set_of_block.find(first);
    if (it == set_of_block.end()) {
      set_of_block.emplace(first, sets.size());
      sets.push_back({(int32_t)s});
    } else {
      sets[it->second].push_back((int32_t)s);
    }
  }

  // each kept set's prefix: the shortest common run with its first member
  std::vector<int32_t> seq_prefix(S, 0), starts{0}, tokens, members;
  int32_t max_members = 0, max_tokens = 0;
  for (const auto &set : sets) {
    if ((int)set.size() < min_sharers) continue;
    const size_t r = (size_t)set[0];
    int64_t k = full_blocks(r);
    const int32_t *rep = block_tables + r * MB;
    for (size_t i = 1; i < set.size() && k > 0; ++i) {
      const size_t m = (size_t)set[i];
      const int64_t lim = k < full_blocks(m) ? k : full_blocks(m);
      const int32_t *row = block_tables + m * MB;
      int64_t j = 0;
      while (j < lim && row[j] == rep[j]) ++j;
      k = j;
    }
    const int64_t tok = k * block_size;
    for (int32_t s : set) {
      seq_prefix[(size_t)s] = (int32_t)tok;
      members.push_back(s);
    }
    starts.push_back((int32_t)members.size());
    tokens.push_back((int32_t)tok);
    if ((int32_t)set.size() > max_members) max_members = (int32_t)set.size();
    if (tok > max_tokens) max_tokens = (int32_t)tok;
  }

  const size_t G = tokens.size(), M = members.size();
  const size_t need = S + (G + 1) + G + M;
  if (need > plan_capacity) return PKV_ERR_CAPACITY;
  int32_t *p = plan;
  for (size_t s = 0; s < S; ++s) *p++ = seq_prefix[s];
  for (int32_t v : starts) *p++ = v;
  for (int32_t v : tokens) *p++ = v;
  for (int32_t v : members) *p++ = v;
  info->num_seqs = (int32_t)S;
  info->num_groups = (int32_t)G;
  info->num_members = (int32_t)M;
  info->max_members = max_members;
  info->max_prefix_tokens = max_tokens;
  return PKV_OK;
}
