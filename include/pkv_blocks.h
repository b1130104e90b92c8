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
 * Under memory pressure a sequence can leave the device: its blocks are
 * copied to host memory and the device blocks freed, and later copied back
 * into whatever device blocks are free then ("PagedAttention - Virtual
 * Memory for the KV Cache" explainer, chapter 05 "vLLM - The Engine", card
 * "Preemption & swapping", and deep dive "Indirection Is the Universal
 * Unlock", card "What Indirection Buys"; "PagedAttention: how vLLM manages
 * the KV cache", section "PagedAttention does not solve admission
 * control").  swap_blocks is the copy; the block manager's swap calls do
 * the bookkeeping.
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
  PKV_ERR_CAPACITY = 15,    /* an output buffer is too small */
  PKV_ERR_SWAPPED = 17,     /* the sequence is (or is not) swapped out */
  PKV_ERR_SHARED = 18,      /* a block is shared with a sequence not listed */
  PKV_ERR_MEMORY = 19       /* a pointer is neither device memory nor pinned
                               host memory */
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

/*
 * swap_blocks - copy whole blocks from one pair of pools to another, where
 * each pool is device memory or pinned host memory (hipHostMalloc, or a
 * torch tensor made with pin_memory=True); the copy runs as one kernel that
 * reads and writes host memory directly over the host link.
 *
 * For each pair i, block block_mapping[2i+1] of dst_k_cache and of
 * dst_v_cache becomes a copy of block block_mapping[2i] of src_k_cache and
 * src_v_cache (raw bits; a block is Hkv * block_size * head_dim elements,
 * the same in every layout).  block_mapping: int64 [num_pairs, 2] (source,
 * destination), in device or pinned host memory.  The source pools hold
 * src_num_blocks blocks, the destination pools dst_num_blocks; dims gives
 * num_kv_heads, head_dim and dtype (PKV_E4M3 for the 8-bit caches) - its
 * num_blocks is not used.
 * Every pointer is checked with the HIP runtime: one that is neither device
 * memory nor pinned host memory returns PKV_ERR_MEMORY before any launch.
 * Preconditions (data, not checked): destinations pairwise distinct and,
 * when source and destination are the same pools, none of them a source.
 * A pair with an index outside its pool copies nothing.  Asynchronous on
 * `stream`: host memory is complete once the stream has been synchronised.
 */
int swap_blocks(const void *src_k_cache, const void *src_v_cache,
                void *dst_k_cache, void *dst_v_cache,
                const int64_t *block_mapping, int num_pairs,
                int32_t src_num_blocks, int32_t dst_num_blocks, int block_size,
                const pkv_dims *dims, pkv_stream_t stream);

/* ---- host block manager ------------------------------------------------
 * All functions are host-only, touch no device, and are not thread-safe on
 * one manager.  Allocation pops the free list as a stack: a fresh manager
 * hands out blocks 0, 1, 2, ...; a finished sequence pushes its blocks back
 * in reverse table order, so its first block is the next one handed out. */
typedef struct pkv_block_manager pkv_block_manager;

/* A manager of num_blocks device blocks of block_size tokens (block_size
 * >= 1) and no host blocks. */
int pkv_bm_create(int32_t num_blocks, int32_t block_size,
                  pkv_block_manager **out);
/* The same, with a second pool of num_host_blocks host blocks that swapped
 * out sequences occupy (its own free stack: 0, 1, 2, ... first). */
int pkv_bm_create_with_host(int32_t num_blocks, int32_t num_host_blocks,
                            int32_t block_size, pkv_block_manager **out);
void pkv_bm_destroy(pkv_block_manager *bm);

/* Register sequence seq_id holding num_tokens (>= 0) prompt tokens: it gets
 * ceil(num_tokens / block_size) fresh blocks.  If slots_out is not NULL it
 * receives the slot of every token (int64 [num_tokens]). */
int pkv_bm_add_sequence(pkv_block_manager *bm, int64_t seq_id,
                        int32_t num_tokens, int64_t *slots_out);

/* child becomes a copy of parent that shares all of parent's blocks
 * (every shared block's reference count goes up by one).  PKV_ERR_SWAPPED
 * if the parent is swapped out. */
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
 * changes; a swapped-out sequence in the batch gives PKV_ERR_SWAPPED. */
int pkv_bm_append_tokens(pkv_block_manager *bm, const int64_t *seq_ids,
                         int32_t n, int64_t *slots_out,
                         int64_t *copy_pairs_out, int32_t *num_copies_out);

/* The sequence ends: every block's reference count goes down by one, and
 * blocks no longer referenced return to the free list (the host free list
 * for a swapped-out sequence). */
int pkv_bm_free_sequence(pkv_block_manager *bm, int64_t seq_id);

/* Swap the listed sequences out to the host pool (a sequence listed twice
 * counts once).  Each distinct device block they hold gets one fresh host
 * block, which inherits its reference count; the pairs (device, host) go
 * to pairs_out (int64 [max_pairs, 2]) in order of first appearance (list
 * order, then table order), and *num_pairs_out says how many.  The device
 * blocks then return to the free list - the caller runs swap_blocks on the
 * pairs before anything writes to them.  Nothing changes on an error:
 * PKV_ERR_UNKNOWN_SEQ; PKV_ERR_SWAPPED (one is out already);
 * PKV_ERR_SHARED (a block is also held by a sequence not listed);
 * PKV_ERR_NO_BLOCKS (too few free host blocks); PKV_ERR_CAPACITY (more
 * than max_pairs pairs). */
int pkv_bm_swap_out(pkv_block_manager *bm, const int64_t *seq_ids, int32_t n,
                    int64_t *pairs_out, int32_t max_pairs,
                    int32_t *num_pairs_out);

/* The reverse: swapped-out sequences come back into fresh device blocks;
 * pairs are (host, device).  Same rules, with PKV_ERR_SWAPPED for a
 * sequence that is not swapped out and PKV_ERR_NO_BLOCKS for too few free
 * device blocks. */
int pkv_bm_swap_in(pkv_block_manager *bm, const int64_t *seq_ids, int32_t n,
                   int64_t *pairs_out, int32_t max_pairs,
                   int32_t *num_pairs_out);

/* Block tables and lengths of a batch, ready for the decode calls:
 * tables_out int32 [n, max_blocks] (unused entries -1), context_lens_out
 * int32 [n].  PKV_ERR_CAPACITY if a sequence holds more than max_blocks
 * blocks; PKV_ERR_SWAPPED if one is swapped out. */
int pkv_bm_batch_tables(const pkv_block_manager *bm, const int64_t *seq_ids,
                        int32_t n, int32_t max_blocks, int32_t *tables_out,
                        int32_t *context_lens_out);

int32_t pkv_bm_num_free_blocks(const pkv_block_manager *bm);
int32_t pkv_bm_num_free_host_blocks(const pkv_block_manager *bm);
/* Reference count of a block, or -1 for an index outside the pool. */
int32_t pkv_bm_refcount(const pkv_block_manager *bm, int32_t block);
/* Reference count of a host block, or -1 for an index outside that pool. */
int32_t pkv_bm_host_refcount(const pkv_block_manager *bm, int32_t block);
/* Token count of a sequence, or -1 if unknown. */
int32_t pkv_bm_num_tokens(const pkv_block_manager *bm, int64_t seq_id);
/* 1 if the sequence is swapped out, 0 if on the device, -1 if unknown. */
int32_t pkv_bm_is_swapped(const pkv_block_manager *bm, int64_t seq_id);
/* A sequence's block table (device or host block numbers) into
 * table_out (int32 [max_blocks]); *num_blocks_out its length. */
int pkv_bm_block_table(const pkv_block_manager *bm, int64_t seq_id,
                       int32_t *table_out, int32_t max_blocks,
                       int32_t *num_blocks_out);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BLOCKS_H */
