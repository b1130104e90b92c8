/*
 * pkv.h - paged decode attention for AMD MI355X (gfx950): the C ABI.
 *
 * A KV cache is cut into fixed-size blocks of `block_size` tokens that may
 * sit anywhere in a pool; each sequence owns a block table that maps its
 * logical blocks (tokens 0..15, 16..31, ...) to physical blocks of the pool,
 * like a page table ("Why vLLM Uses PagedAttention", sections "The insight"
 * and "The mechanism").  This library provides the device side of one
 * decode step over such a cache:
 *
 *   reshape_and_cache             writes every new token's K and V into the
 *                                 slot it was given;
 *   paged_attention_decode        single-query attention for every
 *                                 (sequence, query head), walking the block
 *                                 table, in one kernel launch;
 *   paged_attention_decode_split  the same result for long contexts: the
 *                                 context is cut into partitions that are
 *                                 processed independently, then a second
 *                                 kernel merges the partial results.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All data pointers are DEVICE pointers (HBM), owned by the caller.  The
 *   library allocates nothing and may be called from several host threads;
 *   the one state it keeps is the static scratch of
 *   paged_attention_decode_split_static (one array per device, its address
 *   looked up once per device).
 * - Calls are asynchronous: work is enqueued on `stream` (a hipStream_t;
 *   NULL means the default stream) and the call returns before it runs.
 * - One element type covers q, out, k, v and both caches (pkv_dims.dtype).
 * - Every base pointer must be 16-byte aligned.
 * - Return value: PKV_OK (0) or a positive pkv_status.  On an error nothing
 *   is enqueued.  The library never aborts and never prints.  Only values
 *   the host can see are validated; device-resident indices are
 *   preconditions (see each call), and a kernel never reads or writes
 *   outside the buffers described here whatever those indices hold.
 *
 * Memory layouts (row-major, contiguous; Hq = num_heads, Hkv = num_kv_heads,
 * D = head_dim, bs = block_size, NB = num_blocks, S = num_seqs)
 * ---------------------------------------------------------------------------
 *   q, out        [S, Hq, D]
 *   k, v          [num_tokens, Hkv, D]            (reshape_and_cache input)
 *   k_cache       [NB, Hkv, bs, D]
 *                 element (p, g, o, d) at ((p*Hkv + g)*bs + o)*D + d
 *   v_cache       [NB, Hkv, bs/4, D, 4]
 *                 element (p, g, o, d) at
 *                 (p*Hkv + g)*bs*D + (o/4)*4*D + d*4 + o%4
 *                 (runs of four consecutive tokens of one dimension are
 *                 adjacent, so that the token axis - the contraction axis of
 *                 the probability-times-value product - is contiguous)
 *   block_tables  int32 [S, max_blocks_per_seq]; entry j of row s is the
 *                 physical block holding tokens j*bs .. j*bs+bs-1
 *   context_lens  int32 [S]
 *   slot_mapping  int64 [num_tokens]; slot = physical_block*bs + offset
 *
 * Query head h reads KV head h / (Hq / Hkv) (consecutive groups).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Compatible with hipStream_t (which is `struct ihipStream_t *`). */
typedef struct ihipStream_t *pkv_stream_t;

typedef enum pkv_dtype {
  PKV_F32 = 0,  /* IEEE binary32 */
  PKV_F16 = 1,  /* IEEE binary16 */
  PKV_BF16 = 2, /* bfloat16 */
  PKV_E4M3 = 3  /* 8-bit E4M3 cache elements: only copy_blocks takes it in
                   dims->dtype (the *_fp8 calls imply it for their caches) */
} pkv_dtype;

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,        /* a required pointer is NULL */
  PKV_ERR_DTYPE = 2,       /* dtype not one of pkv_dtype */
  PKV_ERR_BLOCK_SIZE = 3,  /* block_size not 16 or 32 */
  PKV_ERR_HEAD_DIM = 4,    /* head_dim not 64 or 128 */
  PKV_ERR_HEADS = 5,       /* heads <= 0, or num_heads % num_kv_heads != 0 */
  PKV_ERR_SHAPE = 6,       /* a negative size, or a size too large to index */
  PKV_ERR_ALIGN = 7,       /* a base pointer not 16-byte aligned */
  PKV_ERR_PARTITION = 8,   /* partition_size not a positive multiple of
                              block_size */
  PKV_ERR_WORKSPACE = 9,   /* workspace NULL or smaller than required */
  PKV_ERR_LAUNCH = 10,     /* the HIP runtime rejected a kernel launch */
  PKV_ERR_ALIAS = 11,      /* out (or a workspace) overlaps an input */
  PKV_ERR_SCALE = 16,      /* a dequantisation scale not finite and > 0 */
  PKV_ERR_SCRATCH = 20     /* the split partials would not fit the static
                              scratch of paged_attention_decode_split_static */
} pkv_status;

/* Sizes of one call.  Fields a call does not use are ignored. */
typedef struct pkv_dims {
  int32_t num_seqs;           /* S */
  int32_t num_heads;          /* Hq, query heads */
  int32_t num_kv_heads;       /* Hkv, key/value heads */
  int32_t head_dim;           /* D: 64 or 128 */
  int32_t num_blocks;         /* NB, blocks in the pool */
  int32_t max_blocks_per_seq; /* row length of block_tables */
  int32_t dtype;              /* a pkv_dtype */
} pkv_dims;

/*
 * reshape_and_cache - write new tokens' keys and values into the cache.
 *
 * For every token i with slot = slot_mapping[i] >= 0: p = slot / block_size,
 * o = slot % block_size, and for every KV head g the vectors k[i, g, :] and
 * v[i, g, :] are copied bit for bit to k_cache[p, g, o, :] and
 * v_cache[p, g, o, :].  Nothing else in the pools changes.  The write goes
 * into the block a sequence is currently filling, or into a freshly
 * allocated block when the last one is full ("Inside vLLM: How PagedAttention
 * Eliminates KV-Cache Memory Waste", section "How It Works During
 * Generation"; "PagedAttention: how vLLM manages the KV cache", section
 * "Walk one request through the allocator"); the attention kernels read the
 * cache through the same block tables ("PagedAttention - Virtual Memory for
 * the KV Cache" explainer, chapter "vLLM - The Engine": attention and copy
 * kernels traverse block tables).
 *
 * Uses dims->num_kv_heads, head_dim, num_blocks, dtype.
 * Preconditions (device data, not checked): the non-negative slots are
 * pairwise distinct.  A negative slot writes nothing (a padding token); a
 * slot >= num_blocks*block_size writes nothing.
 * k_cache and v_cache must not overlap k or v.
 */
int reshape_and_cache(const void *k, const void *v, void *k_cache,
                      void *v_cache, const int64_t *slot_mapping,
                      int num_tokens, int block_size, const pkv_dims *dims,
                      pkv_stream_t stream);

/*
 * paged_attention_decode - single-query attention over a paged KV cache.
 *
 * For every sequence s and query head h, with L = context_lens[s] and
 * g = h / (Hq/Hkv):
 *     out[s, h, :] = sum_t softmax_t(scale * q[s,h,:] . K_t) * V_t,
 * over tokens t = 0 .. L-1, where K_t and V_t are read from physical block
 * block_tables[s][t / block_size] at offset t % block_size.  This is the
 * computation of ordinary attention; only the addressing goes through the
 * block table ("PagedAttention: how vLLM manages the KV cache", section
 * "PagedAttention changes addressing inside attention"; "Paged Attention"
 * placement notes, section "Paged Attention's Approach": the kernel reads
 * the table and walks the blocks of a request).  L counts the token being
 * decoded, whose K/V were written by reshape_and_cache before this call.
 * L = 0 gives an all-zero output row.
 *
 * Arithmetic: products and sums in fp32 whatever the storage type; the
 * result is rounded to nearest-even into the storage type.  The result is
 * deterministic and depends only on the logical contents, not on which
 * physical blocks hold them.
 *
 * Preconditions (device data, not checked): 0 <= L <= max_blocks_per_seq *
 * block_size (larger L is treated as that bound), and
 * 0 <= block_tables[s][j] < num_blocks for j < ceil(L / block_size) (an
 * entry outside the pool is read as block 0).  Table entries past
 * ceil(L / block_size), and slots past L-1 in the last block, are never read.
 * `out` must not overlap any input.
 */
int paged_attention_decode(void *out, const void *q, const void *k_cache,
                           const void *v_cache, const int32_t *block_tables,
                           const int32_t *context_lens, float scale,
                           int block_size, const pkv_dims *dims,
                           pkv_stream_t stream);

/*
 * paged_attention_split_workspace_bytes - size of the fp32 workspace
 * paged_attention_decode_split needs for these sizes.  Writes it to *bytes.
 */
int paged_attention_split_workspace_bytes(const pkv_dims *dims, int block_size,
                                          int partition_size, size_t *bytes);

/*
 * paged_attention_decode_split - the same result as paged_attention_decode,
 * computed in two launches for long contexts.
 *
 * Launch 1 cuts every sequence's context into partitions of partition_size
 * tokens and, for every (sequence, head, partition), writes to `workspace`
 * the partition's maximum logit, its sum of exponentials and its
 * un-normalised weighted sum of values (fp32).  Launch 2 merges the
 * partitions of each (sequence, head) by rescaling every partial to the
 * largest maximum, and writes `out`.  The merge is an exact re-association
 * of the softmax sum, so the two entry points agree up to rounding.
 *
 * partition_size: a positive multiple of block_size (512 is the usual
 * choice).  workspace: device memory of at least the size returned by
 * paged_attention_split_workspace_bytes; its contents on entry do not
 * matter, and after the call it holds scratch data.  Arguments and
 * preconditions are otherwise those of paged_attention_decode.
 */
int paged_attention_decode_split(void *out, const void *q, const void *k_cache,
                                 const void *v_cache,
                                 const int32_t *block_tables,
                                 const int32_t *context_lens, float scale,
                                 int block_size, int partition_size,
                                 void *workspace, size_t workspace_bytes,
                                 const pkv_dims *dims, pkv_stream_t stream);

/*
 * paged_attention_prefill - multi-query attention over the paged cache for
 * chunked prefill.
 *
 * A long prompt is processed in chunks interleaved with decode steps
 * ("Inside vLLM: How PagedAttention Eliminates KV-Cache Memory Waste",
 * section "Continuous Batching and Chunked Prefill").  Before this call the
 * chunk's keys and values are written with reshape_and_cache, so sequence s
 * holds context_lens[s] tokens of which its chunk is the last
 * C_s = query_start_loc[s+1] - query_start_loc[s].  Chunk token j (row
 * query_start_loc[s] + j of q) sits at position context_lens[s] - C_s + j
 * and attends, through the block table, to every token up to and including
 * itself (causal within the chunk); the result is ordinary attention over
 * that prefix ("PagedAttention: how vLLM manages the KV cache", section
 * "PagedAttention changes addressing inside attention").  A one-token chunk
 * is a decode step.
 *
 *   out, q            [num_query_tokens, num_heads, head_dim], dims->dtype
 *   query_start_loc   int32 [num_seqs + 1]: 0 = start[0] <= ... <=
 *                     start[num_seqs] = num_query_tokens (device)
 *   max_query_len     an upper bound of every C_s (host-side; sizes the grid)
 *   k_cache, v_cache, block_tables, context_lens: as for decode.
 * fp16 and bf16 run on the matrix cores: probabilities enter the value
 * product rounded to dims->dtype, accumulation is fp32.  fp32 runs on the
 * vector ALUs (one workgroup per query token and head, fp32 throughout;
 * num_query_tokens * num_heads must fit in an int).  Preconditions (device
 * data, not checked): C_s <= max_query_len and C_s <= context_lens[s]; rows
 * of a query token whose position would be negative are written as zeros.
 * Asynchronous on `stream`; returns a pkv_status.
 */
int paged_attention_prefill(void *out, const void *q, const void *k_cache,
                            const void *v_cache, const int32_t *block_tables,
                            const int32_t *context_lens,
                            const int32_t *query_start_loc, float scale,
                            int block_size, int num_query_tokens,
                            int max_query_len, const pkv_dims *dims,
                            pkv_stream_t stream);

/* ---- 8-bit (E4M3) caches ----------------------------------------------
 * Lower-precision cache formats reduce the bytes per element ("PagedAttention:
 * how vLLM manages the KV cache", section "Keep the tensor formula beside the
 * allocator model"); on this bandwidth-bound path that halves the bytes read
 * per decode step.  The caches then hold one byte per element - the OCP
 * 8-bit float E4M3 (sign, 4 exponent bits with bias 7, 3 fraction bits, no
 * infinity, 0x7f/0xff NaN, largest finite 448) - in the same layouts as
 * above, and each pool has one per-tensor scale: a stored code c stands for
 * the value e4m3(c) * scale.  q, out, k and v keep dims->dtype.
 *
 * reshape_and_cache_fp8: element x is stored as the E4M3 value nearest to
 * x / scale (the quotient in IEEE single precision; ties to the even
 * fraction; magnitudes of 448 and beyond saturate to +-448; NaN stays NaN).
 * paged_attention_decode_fp8 / _split_fp8: attention over the dequantised
 * keys and values; the key scale multiplies the logits and the value scale
 * the output, both in fp32.  fp16/bf16 queries with Hq/Hkv in 2..16 run on
 * the matrix cores (codes widened exactly to the query's type); every
 * other case, fp32 queries with any Hq/Hkv included, runs on the vector
 * ALUs with the codes widened to fp32.  Scales must be finite and > 0
 * (else PKV_ERR_SCALE).  Everything else is as for the calls above. */
int reshape_and_cache_fp8(const void *k, const void *v, void *k_cache,
                          void *v_cache, const int64_t *slot_mapping,
                          int num_tokens, int block_size, float k_scale,
                          float v_scale, const pkv_dims *dims,
                          pkv_stream_t stream);

int paged_attention_decode_fp8(void *out, const void *q, const void *k_cache,
                               const void *v_cache, const int32_t *block_tables,
                               const int32_t *context_lens, float scale,
                               int block_size, float k_scale, float v_scale,
                               const pkv_dims *dims, pkv_stream_t stream);

/* Chunked prefill over 8-bit caches (same rows and causality as
 * paged_attention_prefill).  fp16 and bf16 run on the matrix cores, the
 * codes widened exactly to dims->dtype; fp32 runs on the vector ALUs. */
int paged_attention_prefill_fp8(void *out, const void *q, const void *k_cache,
                                const void *v_cache, const int32_t *block_tables,
                                const int32_t *context_lens,
                                const int32_t *query_start_loc, float scale,
                                int block_size, int num_query_tokens,
                                int max_query_len, float k_scale, float v_scale,
                                const pkv_dims *dims, pkv_stream_t stream);

int paged_attention_decode_split_fp8(void *out, const void *q,
                                     const void *k_cache, const void *v_cache,
                                     const int32_t *block_tables,
                                     const int32_t *context_lens, float scale,
                                     int block_size, int partition_size,
                                     void *workspace, size_t workspace_bytes,
                                     float k_scale, float v_scale,
                                     const pkv_dims *dims, pkv_stream_t stream);

/*
 * paged_attention_decode_split_static - paged_attention_decode_split with no
 * workspace argument and no allocation of any kind, for callers that cannot
 * allocate device memory: code being captured into a HIP graph, serving
 * loops that forbid hipMalloc, harnesses that do not allow it.
 *
 * The partials live in a scratch array of PKV_STATIC_SCRATCH_BYTES (32 MiB)
 * that the library holds on every device it runs on, from the first such
 * call on that device until the process ends; the call uses the copy of the
 * current device (the stream must belong to it).  Sizes whose partials need
 * more (paged_attention_split_workspace_bytes > PKV_STATIC_SCRATCH_BYTES)
 * return PKV_ERR_SCRATCH before anything is enqueued: 8 sequences x 32 heads
 * x 32768 tokens at 512-token partitions need 8.1 MiB, 8 x 64 heads 16.3 MiB.
 * No scratch byte needs a particular value on entry (every partial the
 * merge reads is written by the same call), so the contents left by earlier
 * calls do not matter.  Every call on one device shares its array: calls
 * that overlap in time on one device (concurrent streams, or host threads
 * with different streams) race on it and may return wrong results; calls
 * ordered on one stream do not.  16-bit and fp32 caches only.  Arguments,
 * results and every other error are those of paged_attention_decode_split.
 */
#define PKV_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

int paged_attention_decode_split_static(void *out, const void *q, const void *k_cache,
                                        const void *v_cache, const int32_t *block_tables,
                                        const int32_t *context_lens, float scale,
                                        int block_size, int partition_size,
                                        const pkv_dims *dims, pkv_stream_t stream);

/* A static, human-readable description of a status code. */
const char *pkv_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
