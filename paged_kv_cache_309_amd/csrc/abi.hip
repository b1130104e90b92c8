// abi.hip - the exported C ABI: argument validation, kernel choice and
// launch.  Every check on plain arguments runs before the first HIP call, so
// a call rejected by one touches no device; swap_blocks then asks the
// runtime what its pointers are.
#include <limits.h>
#include <stdint.h>

#include <mutex>

#include "pkv.h"
#include "pkv_blocks.h"
#include "pkv_internal.h"
#include "pkv_prefix.h"

namespace {

using u128 = unsigned __int128;

constexpr int kMaxGridYZ = 65535;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int elem_bytes(int dtype) { return dtype == PKV_F32 ? 4 : (dtype == PKV_E4M3 ? 1 : 2); }

constexpr int kCacheSame = -1;  // the caches hold dims->dtype

bool scale_ok(float x) { return x > 0.f && x <= 3.0e38f; }  // finite, positive

// The address a kernel uses for p: p itself for device (or managed)
// memory; for pinned host memory, the device-side address of the same byte.
// False for anything else (pageable host memory, unknown pointers).
bool device_address(const void *p, void **out) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the error this query leaves behind
    return false;
  }
  switch (at.type) {
    case hipMemoryTypeDevice:
    case hipMemoryTypeManaged:
      *out = const_cast<void *>(p);
      return true;
    case hipMemoryTypeHost: {
      void *d = nullptr;
      if (hipHostGetDevicePointer(&d, const_cast<void *>(p), 0) != hipSuccess || !d) {
        (void)hipGetLastError();
        return false;
      }
      *out = d;
      return true;
    }
    default:
      return false;
  }
}

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  if (na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Checks shared by the decode entry points; fills the byte sizes.
// cache_elem: bytes of one cache element (dtype's size, or 1 for E4M3).
int check_decode(const pkv_dims *d, int block_size, size_t *q_bytes,
                 size_t *cache_bytes, int cache_elem = 0) {
  if (!d) return PKV_ERR_NULL;
  if (d->dtype < PKV_F32 || d->dtype > PKV_BF16) return PKV_ERR_DTYPE;
  if (block_size != 16 && block_size != 32) return PKV_ERR_BLOCK_SIZE;
  if (d->head_dim != 64 && d->head_dim != 128) return PKV_ERR_HEAD_DIM;
  if (d->num_heads <= 0 || d->num_kv_heads <= 0 || d->num_heads % d->num_kv_heads != 0)
    return PKV_ERR_HEADS;
  if (d->num_seqs < 0 || d->num_blocks < 0 || d->max_blocks_per_seq < 0)
    return PKV_ERR_SHAPE;
  if (d->num_seqs > kMaxGridYZ) return PKV_ERR_SHAPE;
  if ((int64_t)d->max_blocks_per_seq * block_size > INT_MAX / 2) return PKV_ERR_SHAPE;
  const u128 e = (u128)elem_bytes(d->dtype);
  const u128 qb = (u128)d->num_seqs * (u128)d->num_heads * (u128)d->head_dim * e;
  const u128 ce = cache_elem ? (u128)cache_elem : e;
  const u128 cb = (u128)d->num_blocks * (u128)d->num_kv_heads * (u128)block_size *
                  (u128)d->head_dim * ce;
  if (qb > ((u128)1 << 62) || cb > ((u128)1 << 62)) return PKV_ERR_SHAPE;
  *q_bytes = (size_t)qb;
  *cache_bytes = (size_t)cb;
  return PKV_OK;
}

int check_decode_ptrs(void *out, const void *q, const void *k_cache,
                      const void *v_cache, const int32_t *block_tables,
                      const int32_t *context_lens, const pkv_dims *d,
                      size_t q_bytes, size_t cache_bytes) {
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PKV_ERR_ALIGN;
  const size_t tb = (size_t)d->num_seqs * (size_t)d->max_blocks_per_seq * 4;
  const size_t lb = (size_t)d->num_seqs * 4;
  if (overlap(out, q_bytes, q, q_bytes) || overlap(out, q_bytes, k_cache, cache_bytes) ||
      overlap(out, q_bytes, v_cache, cache_bytes) || overlap(out, q_bytes, block_tables, tb) ||
      overlap(out, q_bytes, context_lens, lb))
    return PKV_ERR_ALIAS;
  return PKV_OK;
}

pkv::DecodeArgs make_args(void *out, const void *q, const void *k_cache,
                          const void *v_cache, const int32_t *block_tables,
                          const int32_t *context_lens, float scale,
                          int block_size, const pkv_dims *d,
                          float k_scale = 1.f, float v_scale = 1.f) {
  pkv::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  // the softmax runs in base 2: exp(x * scale) = 2^(x * scale * log2 e); an
  // 8-bit cache's key scale multiplies every logit and is folded in too
  a.scale_log2 = (float)((double)scale * (double)k_scale * 1.4426950408889634074);
  a.v_scale = v_scale;
  a.num_seqs = d->num_seqs;
  a.num_heads = d->num_heads;
  a.num_kv_heads = d->num_kv_heads;
  a.num_blocks = d->num_blocks;
  // an empty pool holds no token: every context is then treated as empty,
  // so no block (not even the clamped block 0) is ever read
  a.max_blocks = d->num_blocks > 0 ? d->max_blocks_per_seq : 0;
  a.block_size = block_size;
  a.part_tokens = 0;
  a.num_parts = 1;
  return a;
}

// Matrix cores when a KV head serves 2..16 query heads in fp16/bf16; the
// vector kernel otherwise: multi-head attention, wider groups, and fp32
// queries over any cache (fp32 arithmetic throughout, 8-bit caches too).
bool use_mfma(const pkv_dims *d) {
  const int G = d->num_heads / d->num_kv_heads;
  return d->dtype != PKV_F32 && G >= 2 && G <= 16;
}

int num_partitions(const pkv_dims *d, int block_size, int partition_size) {
  const int64_t ctx = (int64_t)d->max_blocks_per_seq * block_size;
  return (int)((ctx + partition_size - 1) / partition_size);
}

int split_ws_bytes(const pkv_dims *d, int block_size, int partition_size,
                   size_t *bytes) {
  if (partition_size <= 0 || partition_size % block_size != 0) return PKV_ERR_PARTITION;
  const int P = num_partitions(d, block_size, partition_size);
  if (P > kMaxGridYZ) return PKV_ERR_PARTITION;
  const u128 n = (u128)d->num_seqs * (u128)d->num_heads * (u128)(P > 0 ? P : 1);
  const u128 b = n * (u128)(d->head_dim + 2) * 4;
  if (b > ((u128)1 << 62)) return PKV_ERR_SHAPE;
  *bytes = (size_t)b;
  return PKV_OK;
}

}  // namespace

namespace {

int cache_write(const void *k, const void *v, void *k_cache, void *v_cache,
                const int64_t *slot_mapping, int num_tokens, int block_size,
                const pkv_dims *dims, pkv_stream_t stream, int cache_dtype,
                float k_scale, float v_scale) {
  if (!dims) return PKV_ERR_NULL;
  if (dims->dtype < PKV_F32 || dims->dtype > PKV_BF16) return PKV_ERR_DTYPE;
  if (block_size != 16 && block_size != 32) return PKV_ERR_BLOCK_SIZE;
  if (dims->head_dim != 64 && dims->head_dim != 128) return PKV_ERR_HEAD_DIM;
  if (dims->num_kv_heads <= 0) return PKV_ERR_HEADS;
  if (num_tokens < 0 || dims->num_blocks < 0) return PKV_ERR_SHAPE;
  if (!scale_ok(k_scale) || !scale_ok(v_scale)) return PKV_ERR_SCALE;
  const u128 e = (u128)elem_bytes(dims->dtype);
  const u128 ce = cache_dtype == kCacheSame ? e : 1;
  const u128 tb = (u128)num_tokens * (u128)dims->num_kv_heads * (u128)dims->head_dim * e;
  const u128 cb = (u128)dims->num_blocks * (u128)dims->num_kv_heads * (u128)block_size *
                  (u128)dims->head_dim * ce;
  if (tb > ((u128)1 << 62) || cb > ((u128)1 << 62)) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PKV_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned(slot_mapping, 8))
    return PKV_ERR_ALIGN;
  if (overlap(k_cache, (size_t)cb, k, (size_t)tb) || overlap(k_cache, (size_t)cb, v, (size_t)tb) ||
      overlap(v_cache, (size_t)cb, k, (size_t)tb) || overlap(v_cache, (size_t)cb, v, (size_t)tb) ||
      overlap(k_cache, (size_t)cb, v_cache, (size_t)cb))
    return PKV_ERR_ALIAS;
  pkv::CacheWriteArgs a{};
  a.k = k;
  a.v = v;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_kv_heads = dims->num_kv_heads;
  a.num_blocks = dims->num_blocks;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  const int ct = cache_dtype == kCacheSame ? dims->dtype : cache_dtype;
  const hipError_t err = pkv::launch_reshape_and_cache(
      a, dims->dtype, ct, dims->head_dim, block_size, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int decode(void *out, const void *q, const void *k_cache, const void *v_cache,
           const int32_t *block_tables, const int32_t *context_lens, float scale,
           int block_size, const pkv_dims *dims, pkv_stream_t stream,
           int cache_dtype, float k_scale, float v_scale) {
  size_t qb = 0, cb = 0;
  int rc = check_decode(dims, block_size, &qb, &cb, cache_dtype == kCacheSame ? 0 : 1);
  if (rc != PKV_OK) return rc;
  if (!scale_ok(k_scale) || !scale_ok(v_scale)) return PKV_ERR_SCALE;
  if (dims->num_seqs == 0) return PKV_OK;
  rc = check_decode_ptrs(out, q, k_cache, v_cache, block_tables, context_lens, dims, qb, cb);
  if (rc != PKV_OK) return rc;
  const pkv::DecodeArgs a = make_args(out, q, k_cache, v_cache, block_tables,
                                      context_lens, scale, block_size, dims, k_scale,
                                      v_scale);
  const int ct = cache_dtype == kCacheSame ? dims->dtype : cache_dtype;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const hipError_t err =
      use_mfma(dims)
          ? pkv::launch_decode_mfma(a, dims->dtype, ct, dims->head_dim, block_size, false, st)
          : pkv::launch_decode_vector(a, dims->dtype, ct, dims->head_dim, block_size, false, st);
  return err == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int prefill(void *out, const void *q, const void *k_cache, const void *v_cache,
            const int32_t *block_tables, const int32_t *context_lens,
            const int32_t *query_start_loc, float scale, int block_size, int num_query_tokens,
            int max_query_len, const pkv_dims *dims, pkv_stream_t stream, int cache_dtype,
            float k_scale, float v_scale) {
  size_t sb = 0, cb = 0;
  int rc = check_decode(dims, block_size, &sb, &cb, cache_dtype == kCacheSame ? 0 : 1);
  if (rc != PKV_OK) return rc;
  if (!scale_ok(k_scale) || !scale_ok(v_scale)) return PKV_ERR_SCALE;
  if (num_query_tokens < 0 || max_query_len < 0) return PKV_ERR_SHAPE;
  // fp16/bf16 queries run on the matrix cores (16-bit or 8-bit caches);
  // fp32 on the vector kernel, one workgroup per (query row, head)
  const bool on_mfma = dims->dtype != PKV_F32;
  if (!on_mfma && (int64_t)num_query_tokens * dims->num_heads > INT_MAX) return PKV_ERR_SHAPE;
  const int G = dims->num_heads / dims->num_kv_heads;
  const u128 qb = (u128)num_query_tokens * (u128)dims->num_heads * (u128)dims->head_dim *
                  (u128)elem_bytes(dims->dtype);
  if (qb > ((u128)1 << 62)) return PKV_ERR_SHAPE;
  // no chunk is longer than all query tokens together
  const int64_t rows = (int64_t)(max_query_len < num_query_tokens ? max_query_len
                                                                  : num_query_tokens) * G;
  const int64_t rpw = pkv::prefill_rows_per_workgroup();
  const int64_t q_blocks = (rows + rpw - 1) / rpw;
  if (q_blocks > INT_MAX ||
      pkv::prefill_grid(dims->num_seqs, dims->num_kv_heads, (int)q_blocks) > INT_MAX)
    return PKV_ERR_SHAPE;
  if (dims->num_seqs == 0 || num_query_tokens == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc)
    return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(query_start_loc, 4))
    return PKV_ERR_ALIGN;
  const size_t tb = (size_t)dims->num_seqs * (size_t)dims->max_blocks_per_seq * 4;
  const size_t lb = (size_t)dims->num_seqs * 4;
  const size_t ob = (size_t)qb;
  if (overlap(out, ob, q, ob) || overlap(out, ob, k_cache, cb) || overlap(out, ob, v_cache, cb) ||
      overlap(out, ob, block_tables, tb) || overlap(out, ob, context_lens, lb) ||
      overlap(out, ob, query_start_loc, lb + 4))
    return PKV_ERR_ALIAS;
  const int ct = cache_dtype == kCacheSame ? dims->dtype : cache_dtype;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!on_mfma) {
    pkv::DecodeArgs d = make_args(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                  block_size, dims, k_scale, v_scale);
    d.query_start_loc = query_start_loc;
    d.num_query_tokens = num_query_tokens;
    const hipError_t err =
        pkv::launch_prefill_vector(d, dims->dtype, ct, dims->head_dim, block_size, st);
    return err == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
  }
  pkv::PrefillArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  a.scale_log2 = (float)((double)scale * (double)k_scale * 1.4426950408889634074);
  a.v_scale = v_scale;
  a.num_seqs = dims->num_seqs;
  a.num_heads = dims->num_heads;
  a.num_kv_heads = dims->num_kv_heads;
  a.num_blocks = dims->num_blocks;
  a.max_blocks = dims->num_blocks > 0 ? dims->max_blocks_per_seq : 0;
  a.num_query_tokens = num_query_tokens;
  a.q_blocks = (int)q_blocks;
  const hipError_t err =
      pkv::launch_prefill_mfma(a, dims->dtype, ct, dims->head_dim, block_size, max_query_len, st);
  return err == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int decode_split(void *out, const void *q, const void *k_cache, const void *v_cache,
                 const int32_t *block_tables, const int32_t *context_lens, float scale,
                 int block_size, int partition_size, void *workspace,
                 size_t workspace_bytes, const pkv_dims *dims, pkv_stream_t stream,
                 int cache_dtype, float k_scale, float v_scale) {
  size_t qb = 0, cb = 0, need = 0;
  int rc = check_decode(dims, block_size, &qb, &cb, cache_dtype == kCacheSame ? 0 : 1);
  if (rc != PKV_OK) return rc;
  if (!scale_ok(k_scale) || !scale_ok(v_scale)) return PKV_ERR_SCALE;
  rc = split_ws_bytes(dims, block_size, partition_size, &need);
  if (rc != PKV_OK) return rc;
  if (dims->num_seqs == 0) return PKV_OK;
  rc = check_decode_ptrs(out, q, k_cache, v_cache, block_tables, context_lens, dims, qb, cb);
  if (rc != PKV_OK) return rc;
  if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PKV_ERR_ALIGN;
  if (overlap(workspace, need, out, qb) || overlap(workspace, need, q, qb) ||
      overlap(workspace, need, k_cache, cb) || overlap(workspace, need, v_cache, cb) ||
      overlap(workspace, need, block_tables,
              (size_t)dims->num_seqs * (size_t)dims->max_blocks_per_seq * 4) ||
      overlap(workspace, need, context_lens, (size_t)dims->num_seqs * 4))
    return PKV_ERR_ALIAS;

  pkv::DecodeArgs a = make_args(out, q, k_cache, v_cache, block_tables,
                                context_lens, scale, block_size, dims, k_scale, v_scale);
  const int P = num_partitions(dims, block_size, partition_size);
  a.num_parts = P > 0 ? P : 1;  // P == 0: no token can be attended; the reduce writes zeros
  a.part_tokens = partition_size;
  const size_t n = (size_t)dims->num_seqs * dims->num_heads * a.num_parts;
  a.ws_o = static_cast<float *>(workspace);
  a.ws_m = a.ws_o + n * dims->head_dim;
  a.ws_l = a.ws_m + n;

  const int ct = cache_dtype == kCacheSame ? dims->dtype : cache_dtype;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t err = hipSuccess;
  if (P > 0) {
    err = use_mfma(dims)
              ? pkv::launch_decode_mfma(a, dims->dtype, ct, dims->head_dim, block_size, true, st)
              : pkv::launch_decode_vector(a, dims->dtype, ct, dims->head_dim, block_size, true, st);
  }
  if (err == hipSuccess) err = pkv::launch_partition_reduce(a, dims->dtype, dims->head_dim, st);
  return err == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

// ---- shared-prefix decode ------------------------------------------------
// Chunking of the prefixes: enough (set, KV head, chunk) units that the
// prefix launch fills the chip's 256 compute units once, in chunks of at
// least 128 tokens (a multiple of the 32-token super-tile).  Fixed by the
// sizes alone, so that the workspace size is known before any device call.
constexpr int kPrefixTargetWorkgroups = 256;
constexpr int kPrefixMinChunk = 128;
constexpr int kPrefixMaxChunks = 16;  // the vector decode kernel's row states
constexpr int kPrefixMemberTarget = 256;

struct PrefixChunks {
  int q_blocks;      // row blocks of the largest set (member blocks of
                     // kPrefixMembersPerWorkgroup for multi-head attention)
  int chunk_tokens;
  int n_chunks;
};

// Multi-head attention (one query head per KV head) takes its prefix on
// the grouped-query decode kernel's structure: 32 members of a set are the
// columns of the products (two 16-column tiles against every tile loaded),
// the four wavefronts split the prefix (or one chunk of it), and one
// partial per (member, head, chunk) comes out: a few MB where the 128-token
// chunks of the chunked products would write several times as much.  Grouped-query attention fills the
// columns with a member's heads instead, so it takes the chunked products,
// whose 128-row blocks read each chunk once for 128 / G members.
bool prefix_by_members(const pkv_dims *d) { return d->num_heads == d->num_kv_heads; }

int prefix_chunks(const pkv_dims *d, const pkv_prefix_info *info, PrefixChunks *pc) {
  if (prefix_by_members(d)) {
    // chunks (of at least 256 tokens) only when the (set, head, member
    // block) units leave compute units idle: each chunk adds a partial per
    // (member, head).  128 members x 32 heads over 1024 tokens, 32 members
    // per workgroup: one chunk 18.6 us, two 14.9 us (decode 90.7 / 90.9
    // us); 16 members per workgroup: one chunk 16.1 us, two 17.4, four 22.3
    pc->q_blocks = (info->max_members + pkv::kPrefixMembersPerWorkgroup - 1) /
                   pkv::kPrefixMembersPerWorkgroup;
    const int64_t base = (int64_t)info->num_groups * d->num_kv_heads * pc->q_blocks;
    const int64_t tok = info->max_prefix_tokens;
    int64_t n = base > 0 ? (kPrefixMemberTarget + base - 1) / base : 1;
    const int64_t most = (tok + 255) / 256;
    n = n < most ? n : most;
    n = n < kPrefixMaxChunks ? n : kPrefixMaxChunks;
    n = n < 1 ? 1 : n;
    int64_t ck = (tok + n - 1) / n;
    ck = (ck + 15) / 16 * 16;
    ck = ck < 16 ? 16 : ck;
    pc->chunk_tokens = (int)ck;
    pc->n_chunks = (int)((tok + ck - 1) / ck);
    if ((int64_t)info->num_groups * pc->q_blocks * pc->n_chunks > kMaxGridYZ)
      return PKV_ERR_SHAPE;
    return PKV_OK;
  }
  const int G = d->num_heads / d->num_kv_heads;
  const int rpw = pkv::prefill_rows_per_workgroup();
  const int64_t rows = (int64_t)info->max_members * G;
  pc->q_blocks = (int)((rows + rpw - 1) / rpw);
  const int64_t base = (int64_t)info->num_groups * d->num_kv_heads * pc->q_blocks;
  const int64_t tok = info->max_prefix_tokens;
  int64_t n = base > 0 ? (kPrefixTargetWorkgroups + base - 1) / base : 1;
  const int64_t most = (tok + kPrefixMinChunk - 1) / kPrefixMinChunk;
  n = n < most ? n : most;
  n = n < kPrefixMaxChunks ? n : kPrefixMaxChunks;
  n = n < 1 ? 1 : n;
  int64_t ck = (tok + n - 1) / n;
  ck = (ck + 31) / 32 * 32;
  if (ck < 32) ck = 32;
  pc->chunk_tokens = (int)ck;
  pc->n_chunks = (int)((tok + ck - 1) / ck);
  if (pkv::prefix_grid(info->num_groups, d->num_kv_heads, pc->n_chunks, pc->q_blocks) >
      INT_MAX)
    return PKV_ERR_SHAPE;
  return PKV_OK;
}

// The plan's sizes against the dims; fills the chunking and the workspace
// bytes (0 when no set is planned).
int check_prefix(const pkv_dims *d, int block_size, const pkv_prefix_info *info,
                 PrefixChunks *pc, size_t *ws_bytes) {
  if (!info) return PKV_ERR_NULL;
  if (info->num_seqs != d->num_seqs || info->num_groups < 0 || info->num_members < 0 ||
      info->max_members < 0 || info->max_prefix_tokens < 0 ||
      info->num_members > d->num_seqs || info->max_members > info->num_members ||
      2 * (int64_t)info->num_groups > info->num_members ||
      (int64_t)info->max_prefix_tokens > (int64_t)d->max_blocks_per_seq * block_size)
    return PKV_ERR_SHAPE;
  *ws_bytes = 0;
  *pc = PrefixChunks{0, 0, 0};
  if (info->num_groups == 0 || info->max_prefix_tokens == 0) return PKV_OK;
  const int rc = prefix_chunks(d, info, pc);
  if (rc != PKV_OK) return rc;
  const u128 b = (u128)d->num_seqs * (u128)d->num_heads * (u128)pc->n_chunks *
                 (u128)(d->head_dim + 2) * 4;
  if (b > ((u128)1 << 62)) return PKV_ERR_SHAPE;
  *ws_bytes = (size_t)b;
  return PKV_OK;
}

// ---- the allocation-free split decode's scratch ----------------------------
// For callers that cannot allocate device memory.  The split partials of
// paged_attention_decode_split_static live in this array; every device the
// library runs on holds its own copy (at its own address) until the process
// ends.  In host code `scratch` names a host-side stand-in, never the
// device memory: kernels and copies get the per-device address from
// hipGetSymbolAddress instead.
static __device__ __align__(256) unsigned char scratch[PKV_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];  // device address of `scratch` per device

// The current device's copy of `scratch` (looked up once per device, with
// that device current).
int static_scratch(void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return PKV_ERR_LAUNCH;
  }
  if (dev < 0 || dev >= kMaxDevices) return PKV_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return PKV_ERR_LAUNCH;
    }
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

int reshape_and_cache(const void *k, const void *v, void *k_cache,
                      void *v_cache, const int64_t *slot_mapping,
                      int num_tokens, int block_size, const pkv_dims *dims,
                      pkv_stream_t stream) {
  return cache_write(k, v, k_cache, v_cache, slot_mapping, num_tokens, block_size, dims,
                     stream, kCacheSame, 1.f, 1.f);
}

int reshape_and_cache_fp8(const void *k, const void *v, void *k_cache,
                          void *v_cache, const int64_t *slot_mapping,
                          int num_tokens, int block_size, float k_scale,
                          float v_scale, const pkv_dims *dims,
                          pkv_stream_t stream) {
  return cache_write(k, v, k_cache, v_cache, slot_mapping, num_tokens, block_size, dims,
                     stream, pkv::DT_FP8, k_scale, v_scale);
}

int paged_attention_decode(void *out, const void *q, const void *k_cache,
                           const void *v_cache, const int32_t *block_tables,
                           const int32_t *context_lens, float scale,
                           int block_size, const pkv_dims *dims,
                           pkv_stream_t stream) {
  return decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                dims, stream, kCacheSame, 1.f, 1.f);
}

int paged_attention_decode_fp8(void *out, const void *q, const void *k_cache,
                               const void *v_cache, const int32_t *block_tables,
                               const int32_t *context_lens, float scale,
                               int block_size, float k_scale, float v_scale,
                               const pkv_dims *dims, pkv_stream_t stream) {
  return decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                dims, stream, pkv::DT_FP8, k_scale, v_scale);
}

int paged_attention_prefill(void *out, const void *q, const void *k_cache,
                            const void *v_cache, const int32_t *block_tables,
                            const int32_t *context_lens, const int32_t *query_start_loc,
                            float scale, int block_size, int num_query_tokens,
                            int max_query_len, const pkv_dims *dims, pkv_stream_t stream) {
  return prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale,
                 block_size, num_query_tokens, max_query_len, dims, stream, kCacheSame, 1.f,
                 1.f);
}

int paged_attention_prefill_fp8(void *out, const void *q, const void *k_cache,
                                const void *v_cache, const int32_t *block_tables,
                                const int32_t *context_lens, const int32_t *query_start_loc,
                                float scale, int block_size, int num_query_tokens,
                                int max_query_len, float k_scale, float v_scale,
                                const pkv_dims *dims, pkv_stream_t stream) {
  return prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale,
                 block_size, num_query_tokens, max_query_len, dims, stream, pkv::DT_FP8, k_scale,
                 v_scale);
}

int paged_attention_split_workspace_bytes(const pkv_dims *dims, int block_size,
                                          int partition_size, size_t *bytes) {
  if (!bytes) return PKV_ERR_NULL;
  size_t qb = 0, cb = 0;
  const int rc = check_decode(dims, block_size, &qb, &cb);
  if (rc != PKV_OK) return rc;
  return split_ws_bytes(dims, block_size, partition_size, bytes);
}

int paged_attention_decode_split(void *out, const void *q, const void *k_cache,
                                 const void *v_cache,
                                 const int32_t *block_tables,
                                 const int32_t *context_lens, float scale,
                                 int block_size, int partition_size,
                                 void *workspace, size_t workspace_bytes,
                                 const pkv_dims *dims, pkv_stream_t stream) {
  return decode_split(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                      block_size, partition_size, workspace, workspace_bytes, dims, stream,
                      kCacheSame, 1.f, 1.f);
}

int paged_attention_decode_split_fp8(void *out, const void *q, const void *k_cache,
                                     const void *v_cache,
                                     const int32_t *block_tables,
                                     const int32_t *context_lens, float scale,
                                     int block_size, int partition_size,
                                     void *workspace, size_t workspace_bytes,
                                     float k_scale, float v_scale,
                                     const pkv_dims *dims, pkv_stream_t stream) {
  return decode_split(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                      block_size, partition_size, workspace, workspace_bytes, dims, stream,
                      pkv::DT_FP8, k_scale, v_scale);
}

int paged_attention_decode_split_static(void *out, const void *q, const void *k_cache,
                                        const void *v_cache, const int32_t *block_tables,
                                        const int32_t *context_lens, float scale,
                                        int block_size, int partition_size,
                                        const pkv_dims *dims, pkv_stream_t stream) {
  // every check on plain arguments first (no HIP call before them)
  size_t qb = 0, cb = 0, need = 0;
  int rc = check_decode(dims, block_size, &qb, &cb);
  if (rc != PKV_OK) return rc;
  rc = split_ws_bytes(dims, block_size, partition_size, &need);
  if (rc != PKV_OK) return rc;
  if (need > (size_t)PKV_STATIC_SCRATCH_BYTES) return PKV_ERR_SCRATCH;
  if (dims->num_seqs == 0) return PKV_OK;
  rc = check_decode_ptrs(out, q, k_cache, v_cache, block_tables, context_lens, dims, qb, cb);
  if (rc != PKV_OK) return rc;
  void *ws = nullptr;
  rc = static_scratch(&ws);
  if (rc != PKV_OK) return rc;
  return decode_split(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                      block_size, partition_size, ws, (size_t)PKV_STATIC_SCRATCH_BYTES, dims,
                      stream, kCacheSame, 1.f, 1.f);
}

int paged_attention_shared_prefix_workspace_bytes(const pkv_dims *dims, int block_size,
                                                  const pkv_prefix_info *info,
                                                  size_t *bytes) {
  if (!bytes) return PKV_ERR_NULL;
  size_t qb = 0, cb = 0;
  int rc = check_decode(dims, block_size, &qb, &cb);
  if (rc != PKV_OK) return rc;
  PrefixChunks pc{};
  return check_prefix(dims, block_size, info, &pc, bytes);
}

int paged_attention_decode_shared_prefix(void *out, const void *q, const void *k_cache,
                                         const void *v_cache, const int32_t *block_tables,
                                         const int32_t *context_lens, float scale,
                                         int block_size, const int32_t *prefix_plan,
                                         const pkv_prefix_info *info, void *workspace,
                                         size_t workspace_bytes, const pkv_dims *dims,
                                         pkv_stream_t stream) {
  size_t qb = 0, cb = 0, need = 0;
  int rc = check_decode(dims, block_size, &qb, &cb);
  if (rc != PKV_OK) return rc;
  if (dims->dtype == PKV_F32) return PKV_ERR_DTYPE;  // the prefix runs on the matrix cores
  PrefixChunks pc{};
  rc = check_prefix(dims, block_size, info, &pc, &need);
  if (rc != PKV_OK) return rc;
  if (need == 0)  // no shared prefix: the ordinary decode
    return decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                  dims, stream, kCacheSame, 1.f, 1.f);
  if (dims->num_seqs == 0) return PKV_OK;
  rc = check_decode_ptrs(out, q, k_cache, v_cache, block_tables, context_lens, dims, qb, cb);
  if (rc != PKV_OK) return rc;
  if (!prefix_plan) return PKV_ERR_NULL;
  if (!aligned(prefix_plan, 4)) return PKV_ERR_ALIGN;
  if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PKV_ERR_ALIGN;
  const size_t pb = 4 * ((size_t)dims->num_seqs + 2 * (size_t)info->num_groups + 1 +
                         (size_t)info->num_members);
  const size_t tb = (size_t)dims->num_seqs * (size_t)dims->max_blocks_per_seq * 4;
  const size_t lb = (size_t)dims->num_seqs * 4;
  if (overlap(out, qb, prefix_plan, pb) || overlap(workspace, need, out, qb) ||
      overlap(workspace, need, q, qb) || overlap(workspace, need, k_cache, cb) ||
      overlap(workspace, need, v_cache, cb) || overlap(workspace, need, block_tables, tb) ||
      overlap(workspace, need, context_lens, lb) || overlap(workspace, need, prefix_plan, pb))
    return PKV_ERR_ALIAS;

  const size_t n = (size_t)dims->num_seqs * dims->num_heads * pc.n_chunks;
  float *ws_o = static_cast<float *>(workspace);
  float *ws_m = ws_o + n * dims->head_dim;
  float *ws_l = ws_m + n;
  const float scale_log2 = (float)((double)scale * 1.4426950408889634074);

  pkv::PrefillArgs p{};
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.scale_log2 = scale_log2;
  p.v_scale = 1.f;
  p.num_seqs = dims->num_seqs;
  p.num_heads = dims->num_heads;
  p.num_kv_heads = dims->num_kv_heads;
  p.num_blocks = dims->num_blocks;
  p.max_blocks = dims->num_blocks > 0 ? dims->max_blocks_per_seq : 0;
  p.q_blocks = pc.q_blocks;
  p.plan = prefix_plan;
  p.ws_o = ws_o;
  p.ws_m = ws_m;
  p.ws_l = ws_l;
  p.num_groups = info->num_groups;
  p.num_members = info->num_members;
  p.chunk_tokens = pc.chunk_tokens;
  p.n_chunks = pc.n_chunks;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  pkv::DecodeArgs a = make_args(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                block_size, dims);
  hipError_t err = hipSuccess;
  if (prefix_by_members(dims)) {
    pkv::DecodeArgs b = a;
    b.plan = prefix_plan;
    b.num_groups = info->num_groups;
    b.num_members = info->num_members;
    b.member_blocks = pc.q_blocks;
    b.pchunk_tokens = pc.chunk_tokens;
    b.n_pchunks = pc.n_chunks;
    b.ws_o = ws_o;
    b.ws_m = ws_m;
    b.ws_l = ws_l;
    err = pkv::launch_prefix_mha(b, dims->dtype, dims->head_dim, block_size, st);
  } else {
    err = pkv::launch_prefix_mfma(p, dims->dtype, dims->dtype, dims->head_dim, block_size, st);
  }
  if (err != hipSuccess) return PKV_ERR_LAUNCH;

  a.seq_prefix = prefix_plan;  // its first S entries
  a.pws_o = ws_o;
  a.pws_m = ws_m;
  a.pws_l = ws_l;
  a.pchunk_tokens = pc.chunk_tokens;
  a.n_pchunks = pc.n_chunks;
  err = use_mfma(dims)
            ? pkv::launch_decode_mfma(a, dims->dtype, dims->dtype, dims->head_dim, block_size,
                                      false, st)
            : pkv::launch_decode_vector(a, dims->dtype, dims->dtype, dims->head_dim,
                                        block_size, false, st);
  return err == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int copy_blocks(void *k_cache, void *v_cache, const int64_t *block_mapping,
                int num_pairs, int block_size, const pkv_dims *dims,
                pkv_stream_t stream) {
  if (!dims) return PKV_ERR_NULL;
  if (dims->dtype < PKV_F32 || dims->dtype > PKV_E4M3) return PKV_ERR_DTYPE;
  if (block_size != 16 && block_size != 32) return PKV_ERR_BLOCK_SIZE;
  if (dims->head_dim != 64 && dims->head_dim != 128) return PKV_ERR_HEAD_DIM;
  if (dims->num_kv_heads <= 0) return PKV_ERR_HEADS;
  if (num_pairs < 0 || dims->num_blocks < 0) return PKV_ERR_SHAPE;
  const u128 bb = (u128)dims->num_kv_heads * (u128)block_size * (u128)dims->head_dim *
                  (u128)elem_bytes(dims->dtype);
  const u128 cb = bb * (u128)dims->num_blocks;
  if (cb > ((u128)1 << 62)) return PKV_ERR_SHAPE;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !block_mapping) return PKV_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned(block_mapping, 8))
    return PKV_ERR_ALIGN;
  if (overlap(k_cache, (size_t)cb, v_cache, (size_t)cb) ||
      overlap(block_mapping, (size_t)num_pairs * 16, k_cache, (size_t)cb) ||
      overlap(block_mapping, (size_t)num_pairs * 16, v_cache, (size_t)cb))
    return PKV_ERR_ALIAS;
  pkv::CopyBlocksArgs a{};
  a.src_k = k_cache;
  a.src_v = v_cache;
  a.dst_k = k_cache;
  a.dst_v = v_cache;
  a.block_mapping = block_mapping;
  a.block_bytes = (int64_t)bb;
  a.src_num_blocks = dims->num_blocks;
  a.dst_num_blocks = dims->num_blocks;
  const hipError_t err =
      pkv::launch_copy_blocks(a, num_pairs, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int swap_blocks(const void *src_k_cache, const void *src_v_cache, void *dst_k_cache,
                void *dst_v_cache, const int64_t *block_mapping, int num_pairs,
                int32_t src_num_blocks, int32_t dst_num_blocks, int block_size,
                const pkv_dims *dims, pkv_stream_t stream) {
  if (!dims) return PKV_ERR_NULL;
  if (dims->dtype < PKV_F32 || dims->dtype > PKV_E4M3) return PKV_ERR_DTYPE;
  if (block_size != 16 && block_size != 32) return PKV_ERR_BLOCK_SIZE;
  if (dims->head_dim != 64 && dims->head_dim != 128) return PKV_ERR_HEAD_DIM;
  if (dims->num_kv_heads <= 0) return PKV_ERR_HEADS;
  if (num_pairs < 0 || src_num_blocks < 0 || dst_num_blocks < 0) return PKV_ERR_SHAPE;
  const u128 bb = (u128)dims->num_kv_heads * (u128)block_size * (u128)dims->head_dim *
                  (u128)elem_bytes(dims->dtype);
  const u128 sb = bb * (u128)src_num_blocks, db = bb * (u128)dst_num_blocks;
  if (sb > ((u128)1 << 62) || db > ((u128)1 << 62)) return PKV_ERR_SHAPE;
  if (num_pairs == 0) return PKV_OK;
  if (!src_k_cache || !src_v_cache || !dst_k_cache || !dst_v_cache || !block_mapping)
    return PKV_ERR_NULL;
  if (!aligned16(src_k_cache) || !aligned16(src_v_cache) || !aligned16(dst_k_cache) ||
      !aligned16(dst_v_cache) || !aligned(block_mapping, 8))
    return PKV_ERR_ALIGN;
  const size_t mb = (size_t)num_pairs * 16;
  if (overlap(dst_k_cache, (size_t)db, dst_v_cache, (size_t)db) ||
      overlap(block_mapping, mb, dst_k_cache, (size_t)db) ||
      overlap(block_mapping, mb, dst_v_cache, (size_t)db))
    return PKV_ERR_ALIAS;
  // Every pointer must be one the device can address: device memory, or
  // pinned host memory (then its device-side address is used).
  const void *ptrs[5] = {src_k_cache, src_v_cache, dst_k_cache, dst_v_cache, block_mapping};
  void *dev[5];
  for (int i = 0; i < 5; ++i) {
    if (!device_address(ptrs[i], &dev[i])) return PKV_ERR_MEMORY;
  }
  pkv::CopyBlocksArgs a{};
  a.src_k = dev[0];
  a.src_v = dev[1];
  a.dst_k = dev[2];
  a.dst_v = dev[3];
  a.block_mapping = static_cast<const int64_t *>(dev[4]);
  a.block_bytes = (int64_t)bb;
  a.src_num_blocks = src_num_blocks;
  a.dst_num_blocks = dst_num_blocks;
  const hipError_t err =
      pkv::launch_copy_blocks(a, num_pairs, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

const char *pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_DTYPE: return "unsupported dtype";
    case PKV_ERR_BLOCK_SIZE: return "block_size must be 16 or 32";
    case PKV_ERR_HEAD_DIM: return "head_dim must be 64 or 128";
    case PKV_ERR_HEADS: return "num_heads must be a positive multiple of num_kv_heads";
    case PKV_ERR_SHAPE: return "a size is negative or too large";
    case PKV_ERR_ALIGN: return "a pointer is not aligned (16 bytes for data)";
    case PKV_ERR_PARTITION: return "partition_size must be a positive multiple of block_size";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_LAUNCH: return "kernel launch failed";
    case PKV_ERR_ALIAS: return "output overlaps an input";
    case PKV_ERR_NO_BLOCKS: return "not enough free blocks";
    case PKV_ERR_UNKNOWN_SEQ: return "unknown sequence id";
    case PKV_ERR_SEQ_EXISTS: return "sequence id already in use";
    case PKV_ERR_CAPACITY: return "output buffer too small";
    case PKV_ERR_SCALE: return "a dequantisation scale is not a finite positive number";
    case PKV_ERR_SWAPPED: return "sequence is swapped out (or, for swap_in, is not)";
    case PKV_ERR_SHARED: return "a block is shared with a sequence outside the list";
    case PKV_ERR_MEMORY: return "a pointer is neither device memory nor pinned host memory";
    case PKV_ERR_SCRATCH:
      return "the split partials need more than the library's static scratch "
             "(PKV_STATIC_SCRATCH_BYTES, 32 MiB per device)";
    default: return "unknown status";
  }
}

int pkv_version(void) { return 200; }

}  // extern "C"
