/*
 * pkv_blocks.h - copy-on-write support for the paged KV cache: the device
 * block copy, and a host-side block manager (free list, reference counts,
 * per-sequence block tables).
 *
 * A block manager hands out fixed-size blocks on demand: a sequence gets a
 * new block only when its token count crosses a block boundary ("Why vLLM
 * Uses PagedAttention", section "The mechanism"; "PagedAttention: how vLLM
 * manages the KV cache", section "Walk one request through the allocator"),
 * and returns its blocks to a global free list when it ends ("Paged
 * Attention" placement notes, section "Paged Attention's Approach").
 * Sequences forked from one another share physical blocks; a reference
 * count tracks the sharers, and a shared block about to be written is first
 * copied into a private block - only that block ("Why vLLM Uses
 * PagedAttention", section "The bonus"; "PagedAttention: how vLLM manages
 * the KV cache", section "Copy-on-write makes shared prefixes practical").
 *
 * Status codes are those of pkv.h, plus the ones below.
 */
#ifndef PKV_BLOCKS_H
#define PKV_BLOCKS_H

#include <stddef.h>
#include <stdint.h>

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PKV_ERR_NO_BLOCKS = 12,   /* not enough free blocks; nothing changed */
  PKV_ERR_UNKNOWN_SEQ = 13, /* no sequence with this id */
  PKV_ERR_SEQ_EXISTS = 14,  /* a sequence with this id already exists */
  PKV_ERR_CAPACITY = 15     /* an output buffer is too small */
};

/*
 * copy_blocks - device copy of whole blocks in both pools.
 *
 * For each pair i, block block_mapping[2i+1] of k_cache and of v_cache
 * becomes a copy of block block_mapping[2i] (all KV heads, all slots, raw
 * bits).  block_mapping: device int64 [num_pairs, 2] (source, destination).
 * Uses dims->num_kv_heads, head_dim, num_blocks, dtype (PKV_E4M3 for the
 * 8-bit caches).
 * Preconditions (device data, not checked): destinations pairwise distinct
 * and none of them a source.  A pair with an index outside the pool copies
 * nothing.  Asynchronous on `stream`; returns a pkv_status.
 */
int copy_blocks(void *k_cache, void *v_cache, const int64_t *block_mapping,
                int num_pairs, int block_size, const pkv_dims *dims,
                pkv_stream_t stream);

/* ---- host block manager ------------------------------------------------
 * All functions are host-only, touch no device, and are not thread-safe on
 * one manager.  Allocation pops the free list as a stack: a fresh manager
 * hands out blocks 0, 1, 2, ...; a finished sequence pushes its blocks back
 * in reverse table order, so its first block is the next one handed out. */
typedef struct pkv_block_manager pkv_block_manager;

/* A manager of num_blocks blocks of block_size tokens (block_size >= 1). */
int pkv_bm_create(int32_t num_blocks, int32_t block_size,
                  pkv_block_manager **out);
void pkv_bm_destroy(pkv_block_manager *bm);

/* Register sequence seq_id holding num_tokens (>= 0) prompt tokens: it gets
 * ceil(num_tokens / block_size) fresh blocks.  If slots_out is not NULL it
 * receives the slot of every token (int64 [num_tokens]). */
int pkv_bm_add_sequence(pkv_block_manager *bm, int64_t seq_id,
                        int32_t num_tokens, int64_t *slots_out);

/* child becomes a copy of parent that shares all of parent's blocks
 * (every shared block's reference count goes up by one). */
int pkv_bm_fork(pkv_block_manager *bm, int64_t parent, int64_t child);

/* Reserve the slot of one new token for each listed sequence (a sequence
 * may appear several times; items are served in order).  For item i the
 * new token t (the sequence's token count) goes to
 *   - a fresh block when t is a multiple of block_size,
 *   - otherwise the last block; if that block is shared (reference count
 *     > 1) the sequence first gets a fresh private block and the pair
 *     (shared, fresh) is appended to copy_pairs_out - the caller copies it
 *     (copy_blocks) before writing the token.
 * slots_out: int64 [n]; copy_pairs_out: int64 [n, 2] (at most n copies);
 * *num_copies_out: the number of pairs written.  If the free list cannot
 * serve the whole batch, PKV_ERR_NO_BLOCKS is returned and nothing
 * changes. */
int pkv_bm_append_tokens(pkv_block_manager *bm, const int64_t *seq_ids,
                         int32_t n, int64_t *slots_out,
                         int64_t *copy_pairs_out, int32_t *num_copies_out);

/* The sequence ends: every block's reference count goes down by one, and
 * blocks no longer referenced return to the free list. */
int pkv_bm_free_sequence(pkv_block_manager *bm, int64_t seq_id);

/* Block tables and lengths of a batch, ready for the decode calls:
 * tables_out int32 [n, max_blocks] (unused entries -1), context_lens_out
 * int32 [n].  PKV_ERR_CAPACITY if a sequence holds more than max_blocks
 * blocks. */
int pkv_bm_batch_tables(const pkv_block_manager *bm, const int64_t *seq_ids,
                        int32_t n, int32_t max_blocks, int32_t *tables_out,
                        int32_t *context_lens_out);

int32_t pkv_bm_num_free_blocks(const pkv_block_manager *bm);
/* Reference count of a block, or -1 for an index outside the pool. */
int32_t pkv_bm_refcount(const pkv_block_manager *bm, int32_t block);
/* Token count of a sequence, or -1 if unknown. */
int32_t pkv_bm_num_tokens(const pkv_block_manager *bm, int64_t seq_id);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BLOCKS_H */
