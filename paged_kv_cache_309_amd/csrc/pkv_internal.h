// pkv_internal.h - what the C-ABI layer and the kernel translation units
// share: the launch arguments and the launchers each kernel file exports.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_FP8 = 3 };

// Threads per workgroup of the decode kernels: four wave64 wavefronts.
constexpr int kDecodeThreads = 256;
constexpr int kDecodeWaves = 4;
// Most partitions one wave of the vector kernel's split launch computes.
constexpr int kMaxPartsPerWave = 4;
// Multi-head shared-prefix partials: blocks of 16 members (matrix-core
// columns) one workgroup computes against each prefix tile it loads.
constexpr int kPrefixColTiles = 2;
constexpr int kPrefixMembersPerWorkgroup = 16 * kPrefixColTiles;

// Compute units of the current device (256 if the query fails; a failed
// query's error is cleared so that it cannot read as a failed launch).
inline int device_compute_units() {
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  return cus;
}

// Consecutive partitions one wavefront of a split launch computes: enough
// that every wavefront of the grid (units = partitions to compute) is
// resident at once, at most kMaxPartsPerWave, and at most a quarter of the
// partitions so that each of a workgroup's four wavefronts gets some.
inline int split_parts_per_wave(int64_t units, int64_t resident_waves, int num_parts) {
  int64_t k = (units + resident_waves - 1) / resident_waves;
  k = k < (int64_t)(num_parts / kDecodeWaves) ? k : (int64_t)(num_parts / kDecodeWaves);
  k = k < (int64_t)kMaxPartsPerWave ? k : (int64_t)kMaxPartsPerWave;
  return k < 1 ? 1 : (int)k;
}

struct DecodeArgs {
  void *out;              // [S, Hq, D] storage type (single pass, reduce)
  float *ws_o;            // [S, Hq, P, D] partial weighted sums (split)
  float *ws_m;            // [S, Hq, P] partial maxima, log2 units (split)
  float *ws_l;            // [S, Hq, P] partial sums of exponentials (split)
  const void *q;          // [S, Hq, D]
  const void *k_cache;    // [NB, Hkv, bs, D]
  const void *v_cache;    // [NB, Hkv, bs/4, D, 4]
  const int32_t *block_tables;  // [S, max_blocks]
  const int32_t *context_lens;  // [S]
  float scale_log2;       // softmax scale times log2(e) times the key scale
  float v_scale;          // value dequantisation scale (1 for 16/32-bit caches)
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int num_blocks;
  int max_blocks;
  int block_size;
  int part_tokens;        // tokens per partition (split); unused otherwise
  int num_parts;          // partitions per sequence (1 for single pass)
  int parts_per_wave = 1; // split on the vector kernel: consecutive
                          // partitions one wavefront computes (1 .. 4)
  // multi-query (chunked prefill) on the vector kernel: q / out hold
  // num_query_tokens rows; sequence s's rows are query_start_loc[s] ..
  // query_start_loc[s+1]-1, the last tokens of its context (causal).
  // nullptr for decode.
  const int32_t *query_start_loc;
  int num_query_tokens;
  // shared-prefix decode (single pass): tokens [0, seq_prefix[s]) of
  // sequence s were computed by the prefix kernel, which left the partial
  // states of its chunks of pchunk_tokens tokens in pws_* ([S, Hq,
  // n_pchunks, D] weighted sums, [S, Hq, n_pchunks] maxima in log2 units
  // and sums); the walk starts after them and the final merge takes them
  // in.  nullptr otherwise.
  const int32_t *seq_prefix;
  const float *pws_o;
  const float *pws_m;
  const float *pws_l;
  int pchunk_tokens;
  int n_pchunks;
  // shared-prefix partials on the grouped-query kernel's structure (one
  // KV head per query head): the plan of pkv_prefix_plan, its set count,
  // member count and member blocks (kPrefixMembersPerWorkgroup) per set;
  // the partials go to ws_* ([S, Hq, n_pchunks] rows, one per chunk of
  // pchunk_tokens)
  const int32_t *plan;
  int num_groups;
  int num_members;
  int member_blocks;
};

struct CacheWriteArgs {
  const void *k;          // [T, Hkv, D]
  const void *v;          // [T, Hkv, D]
  void *k_cache;
  void *v_cache;
  const int64_t *slot_mapping;  // [T]
  int64_t num_tokens;
  int num_kv_heads;
  int num_blocks;
  float k_scale;          // 8-bit caches: stored = encode(x / scale)
  float v_scale;
};

// Block copies between pools (the same pools for copy-on-write; a device
// and a pinned host pool for swapping).  Pointers are device addresses.
struct CopyBlocksArgs {
  const void *src_k;
  const void *src_v;
  void *dst_k;
  void *dst_v;
  const int64_t *block_mapping;  // [num_pairs, 2] (source, destination)
  int64_t block_bytes;           // bytes of one block in one pool
  int src_num_blocks;
  int dst_num_blocks;
};

// Multi-query (chunked prefill) attention: query rows of sequence s are
// query_start_loc[s] .. query_start_loc[s+1]-1 of q / out, the last C_s of
// its context_lens[s] tokens, attending causally.
struct PrefillArgs {
  void *out;
  const void *q;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  const int32_t *query_start_loc;
  float scale_log2;  // scale * k_scale * log2(e)
  float v_scale;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int num_blocks;
  int max_blocks;
  int num_query_tokens;
  int q_blocks;      // grid extent over the query rows of one (seq, KV head)
  // shared-prefix partials (prefix mode): the plan of pkv_prefix_plan, the
  // partial states of every (member, head, chunk) and the chunking of the
  // prefixes.  q_blocks is then the grid extent over the rows of one (set,
  // KV head, chunk).
  const int32_t *plan;
  float *ws_o;       // [S, Hq, n_chunks, D]
  float *ws_m;       // [S, Hq, n_chunks], log2 units
  float *ws_l;       // [S, Hq, n_chunks]
  int num_groups;
  int num_members;
  int chunk_tokens;  // a multiple of 32
  int n_chunks;
};

// Each returns the launch error (hipSuccess when enqueued).
// dtype: of q and out; cache_dtype: of the two pools (dtype, or DT_FP8)
hipError_t launch_decode_vector(const DecodeArgs &a, int dtype, int cache_dtype,
                                int head_dim, int block_size, bool split,
                                hipStream_t st);
hipError_t launch_decode_mfma(const DecodeArgs &a, int dtype, int cache_dtype,
                              int head_dim, int block_size, bool split,
                              hipStream_t st);
hipError_t launch_partition_reduce(const DecodeArgs &a, int dtype,
                                   int head_dim, hipStream_t st);
hipError_t launch_reshape_and_cache(const CacheWriteArgs &a, int dtype,
                                    int cache_dtype, int head_dim,
                                    int block_size, hipStream_t st);
// Multi-query attention on the vector kernel, one workgroup per (query
// row, query head): the prefill path for fp32 and for 8-bit caches.
hipError_t launch_prefill_vector(const DecodeArgs &a, int dtype, int cache_dtype,
                                 int head_dim, int block_size, hipStream_t st);
hipError_t launch_prefill_mfma(const PrefillArgs &a, int dtype, int cache_dtype,
                               int head_dim, int block_size, int max_query_len,
                               hipStream_t st);
// rows of one (sequence, KV head) a prefill workgroup covers, and the
// number of workgroups a prefill launch takes
int prefill_rows_per_workgroup();
int64_t prefill_grid(int num_seqs, int num_kv_heads, int q_blocks);
// Shared-prefix partials: every (set, KV head, chunk) of the plan, its
// member rows times the group's query heads in row blocks of
// prefill_rows_per_workgroup(); workgroups a launch takes.
hipError_t launch_prefix_mfma(const PrefillArgs &a, int dtype, int cache_dtype,
                              int head_dim, int block_size, hipStream_t st);
// Shared-prefix partials for multi-head attention: one workgroup per
// (KV head, set and block of kPrefixMembersPerWorkgroup members, chunk)
// walks the chunk, its four wavefronts splitting the tiles, and writes one
// partial per (member, head, chunk).
hipError_t launch_prefix_mha(const DecodeArgs &a, int dtype, int head_dim,
                             int block_size, hipStream_t st);
int64_t prefix_grid(int num_groups, int num_kv_heads, int n_chunks, int q_blocks);
hipError_t launch_copy_blocks(const CopyBlocksArgs &a, int num_pairs,
                              hipStream_t st);

}  // namespace pkv
