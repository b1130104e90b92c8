/*
 * pkv_prefix.h - decode attention that computes a shared prefix once per
 * set of sharers.
 *
 * Sequences forked from one prompt, or requests that begin with the same
 * system prompt, map the same leading logical blocks to the same physical
 * blocks: the prefix is stored once and a reference count tracks its
 * sharers ("Why vLLM Uses PagedAttention", section "The bonus";
 * "PagedAttention: how vLLM manages the KV cache", section "Copy-on-write
 * makes shared prefixes practical"; "Paged Attention" placement notes,
 * section "Benefits": shared prefixes point to the same physical blocks).
 * paged_attention_decode still reads such a prefix once per sharer.  The
 * call below reads it once per set: every sharer's queries meet the
 * prefix's keys and values in one dense product on the matrix cores, which
 * leaves a partial softmax state (maximum, sum of exponentials, weighted
 * sum of values) per (sequence, head, prefix chunk); the decode kernels then
 * walk only each sequence's own tokens after the prefix and merge those
 * partial states into their result.  The result is the same attention as
 * paged_attention_decode's, up to rounding.
 *
 * Conventions, layouts, dtypes and error behaviour are those of pkv.h.
 */
#ifndef PKV_PREFIX_H
#define PKV_PREFIX_H

#include <stddef.h>
#include <stdint.h>

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Sizes of a prefix plan (host memory). */
typedef struct pkv_prefix_info {
  int32_t num_seqs;          /* S the plan was built for */
  int32_t num_groups;        /* sharer sets */
  int32_t num_members;       /* sequences in all sets together */
  int32_t max_members;       /* members of the largest set */
  int32_t max_prefix_tokens; /* longest shared prefix, in tokens */
} pkv_prefix_info;

/* Entries of the plan array for S sequences: at most 4*S + 1 int32. */
#define PKV_PREFIX_PLAN_MAX_ENTRIES(S) (4 * (size_t)(S) + 1)

/*
 * pkv_prefix_plan - find the sets of sequences that share leading blocks
 * (host code; no device call).
 *
 * block_tables [num_seqs, max_blocks_per_seq] and context_lens [num_seqs]
 * are HOST copies of the arrays the decode call will get.  Sequences whose
 * first block is the same physical block form one set (sets in the order of
 * their first member; members in sequence order; a sequence of fewer than
 * block_size tokens joins none).  A set's shared prefix is the longest run
 * of leading table entries that every member maps to the same blocks and
 * that lies wholly inside every member's context; sets of fewer than
 * min_sharers members (min_sharers >= 2) are dropped.
 *
 * Writes the plan (int32, to be copied to the device as is) to `plan`,
 * which holds plan_capacity entries (PKV_PREFIX_PLAN_MAX_ENTRIES(num_seqs)
 * always suffice), and its sizes to *info.  Layout, with G = num_groups and
 * M = num_members:
 *   [0, S)                seq_prefix[s]: tokens of sequence s that its set's
 *                         prefix covers (0: none), a multiple of block_size
 *   [S, S+G+1)            group_start[j]: first member of set j (member
 *                         offsets; group_start[G] = M)
 *   [S+G+1, S+2G+1)       group_tokens[j]: tokens of set j's prefix
 *   [S+2G+1, S+2G+1+M)    members: sequence indices, set after set
 * Returns PKV_OK, PKV_ERR_NULL, PKV_ERR_BLOCK_SIZE, PKV_ERR_SHAPE (negative
 * sizes, min_sharers < 2) or PKV_ERR_CAPACITY (plan too small).
 */
int pkv_prefix_plan(const int32_t *block_tables, const int32_t *context_lens,
                    int num_seqs, int max_blocks_per_seq, int block_size,
                    int min_sharers, int32_t *plan, size_t plan_capacity,
                    pkv_prefix_info *info);

/*
 * paged_attention_shared_prefix_workspace_bytes - fp32 workspace the
 * shared-prefix decode needs for these sizes and this plan.  Writes it to
 * *bytes (0 when the plan has no set).
 */
int paged_attention_shared_prefix_workspace_bytes(const pkv_dims *dims, int block_size,
                                                  const pkv_prefix_info *info,
                                                  size_t *bytes);

/*
 * paged_attention_decode_shared_prefix - paged_attention_decode with each
 * set's shared prefix computed once for all its members.
 *
 * prefix_plan: DEVICE copy of the array pkv_prefix_plan wrote for these
 * block tables and context lengths; info: its sizes (host).  Preconditions
 * (device data, not checked): the plan was built from the same tables and
 * lengths (every member's first group_tokens / block_size entries map the
 * blocks of the set's first member, and its context holds them).  Plan
 * entries out of range never make a kernel address outside the buffers
 * described here, but give unspecified results.
 *
 * Two launches: the prefix products on the matrix cores (for multi-head
 * attention, blocks of 32 members of a set as the columns of the products,
 * one partial per (member, head, chunk of the prefix); for grouped-query
 * attention, blocks of 128 (member, query head) rows against chunks of the
 * prefix staged in LDS, one partial per chunk), then the decode kernel over
 * each sequence's tokens after its prefix, which starts from the prefix
 * partials.  In the prefix products the probabilities enter the value
 * product rounded to the query type and the sums add exactly those rounded
 * weights; accumulation is fp32.  fp32 queries are refused
 * (PKV_ERR_DTYPE): use paged_attention_decode.  workspace: device memory of at least
 * paged_attention_shared_prefix_workspace_bytes (contents on entry do not
 * matter; it must not overlap any other argument).  A plan with no set
 * runs paged_attention_decode.  Everything else as paged_attention_decode.
 */
int paged_attention_decode_shared_prefix(void *out, const void *q, const void *k_cache,
                                         const void *v_cache, const int32_t *block_tables,
                                         const int32_t *context_lens, float scale,
                                         int block_size, const int32_t *prefix_plan,
                                         const pkv_prefix_info *info, void *workspace,
                                         size_t workspace_bytes, const pkv_dims *dims,
                                         pkv_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PREFIX_H */
