// reduce_and_cache.hip - the partition-reduce kernel of the split decode
// and the cache-write scatter.
#include "pkv_device.h"

namespace pkv {

// ---------------------------------------------------------------------------
// Partition reduce.  Partition p of (sequence s, head h) left its largest
// logit m_p (log2 units), its sum of exponentials l_p = sum 2^(x - m_p) and
// its un-normalised weighted sum o_p = sum 2^(x - m_p) v.  With M = max m_p:
//     out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,
// the same rescaling the online softmax uses inside a partition, so the
// result is the softmax over the whole context.  Partitions at or past
// ceil(L / part_tokens) were empty and are not read.
// One workgroup of 256 threads per (sequence, head): thread t takes the
// four dims 4 (t % (D/4)) .. +3 of the partitions p = t / (D/4) (mod
// 256 / (D/4)), as 16-byte loads of o_p, in one pass with a running maximum
// of its own (each partition's m_p, l_p and o_p are loaded together, the
// loop unrolled so that the loads of several partitions are in flight);
// the partition groups' states are merged through LDS, each rescaled to the
// largest maximum.
constexpr int kReduceThreads = 256;

template <int DT, int D>
__global__ void __launch_bounds__(kReduceThreads) partition_reduce_kernel(DecodeArgs a) {
  constexpr int Q = D / 4;                 // dim quads per row
  constexpr int PG = kReduceThreads / Q;   // partition groups
  __shared__ f32x4 sm_num[PG][Q];
  __shared__ float sm_den[PG];
  __shared__ float sm_m[PG];
  const int h = blockIdx.x, s = blockIdx.y, t = threadIdx.x;
  const int q = t % Q, pg = t / Q;
  const int Hq = a.num_heads;
  int L = a.context_lens[s];
  L = max(0, min(L, a.max_blocks * a.block_size));
  const int np = min(a.num_parts, (L + a.part_tokens - 1) / a.part_tokens);
  const size_t base = ((size_t)s * Hq + h) * a.num_parts;
  const size_t orow = ((size_t)s * Hq + h) * D;
  if (np <= 0) {  // the whole workgroup
    for (int i = t; i < D; i += kReduceThreads) store_elem<DT>(a.out, orow + i, 0.f);
    return;
  }
  // this thread's partitions, in one pass: (m, num, den) rescaled to the
  // running maximum m as partitions arrive (m = -inf: nothing yet, weight 0)
  float m = -INFINITY, den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int p = pg; p < np; p += PG) {
    const float mp = a.ws_m[base + p];
    const float lp = a.ws_l[base + p];
    const f32x4 o = *reinterpret_cast<const f32x4 *>(a.ws_o + (base + p) * D + 4 * q);
    const float mn = fmaxf(m, mp);
    const float r = fast_exp2(m - mn), f = fast_exp2(mp - mn);
    num = r * num + f * o;
    den = fmaf(r, den, f * lp);
    m = mn;
  }
  sm_num[pg][q] = num;
  if (q == 0) {
    sm_den[pg] = den;
    sm_m[pg] = m;
  }
  __syncthreads();
  if (pg == 0) {
    // M: the largest partition maximum (finite: np >= 1); a group without
    // partitions has m = -inf and weight 0
    float M = sm_m[0];
#pragma unroll
    for (int i = 1; i < PG; ++i) M = fmaxf(M, sm_m[i]);
    f32x4 n = {0.f, 0.f, 0.f, 0.f};
    float dd = 0.f;
#pragma unroll
    for (int i = 0; i < PG; ++i) {
      const float f = fast_exp2(sm_m[i] - M);
      n += f * sm_num[i][q];
      dd = fmaf(f, sm_den[i], dd);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) store_elem<DT>(a.out, orow + 4 * q + e, n[e] / dd);
  }
}

hipError_t launch_partition_reduce(const DecodeArgs &a, int dtype,
                                   int head_dim, hipStream_t st) {
  dim3 grid(a.num_heads, a.num_seqs);
#define PKV_REDUCE(DTV, DV) \
  hipLaunchKernelGGL((partition_reduce_kernel<DTV, DV>), grid, dim3(kReduceThreads), 0, st, a)
  if (head_dim == 128) {
    if (dtype == DT_F32) PKV_REDUCE(DT_F32, 128);
    else if (dtype == DT_F16) PKV_REDUCE(DT_F16, 128);
    else PKV_REDUCE(DT_BF16, 128);
  } else {
    if (dtype == DT_F32) PKV_REDUCE(DT_F32, 64);
    else if (dtype == DT_F16) PKV_REDUCE(DT_F16, 64);
    else PKV_REDUCE(DT_BF16, 64);
  }
#undef PKV_REDUCE
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Cache write.  Token i goes to slot = slot_mapping[i]: block slot / BS,
// offset slot % BS.  One thread moves one 16-byte chunk of one (token,
// KV head) key row - a single 16-byte store into the K tile - and the same
// dims of the value row, which the token-grouped V layout spreads with a
// stride of four elements: when four consecutive tokens of the batch fill a
// whole group of four slots (a prompt or a chunk written in order), the
// first of them writes the group's values as 16-byte units, otherwise every
// token writes its own elements.  Negative or out-of-pool slots write
// nothing.  All cache stores are non-temporal: lines this kernel left
// dirty in L2 slowed the attention launch that follows it.  Decode steps,
// same GPU: 64 tokens x 40 heads 232.0 -> 229.9 us, 256 tokens x 8 KV
// heads 266.7 -> 263.5 us; the gain comes from the per-token value
// stores.  The cost: 128 sequences over one shared 1024-token prefix
// (served from cache) 200.8 -> 208.3 us, the same value stores again.
// Group of four consecutive slots of one block that token i's slot falls
// in, if the four tokens b .. b+3 of the batch (b = i - slot % 4) fill
// exactly those slots in order: then one thread (token b's) writes the
// whole group's values as 16-byte units.  Returns b, or -1 when token i's
// group is only partly written by this batch.  The slots are distinct (a
// precondition), so a full group has exactly one such leader.
__device__ __forceinline__ int64_t full_group_leader(const int64_t *slots, int64_t i,
                                                     int64_t num_tokens, int64_t slot) {
  const int64_t b = i - (slot & 3);
  if (b < 0 || b + 3 >= num_tokens) return -1;
  const int64_t s0 = slot - (slot & 3);
  for (int j = 0; j < 4; ++j)
    if (slots[b + j] != s0 + j) return -1;
  return b;
}

template <int DT, int D, int BS>
__global__ void __launch_bounds__(256) reshape_and_cache_kernel(CacheWriteArgs a) {
  constexpr int E = Elem<DT>::bytes;
  constexpr int EPC = 16 / E;      // elements per 16-byte chunk
  constexpr int CPR = D / EPC;     // chunks per (token, head) row
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = a.num_tokens * a.num_kv_heads * CPR;
  if (idx >= total) return;
  const int chunk = (int)(idx % CPR);
  const int64_t row = idx / CPR;          // token * Hkv + head
  const int g = (int)(row % a.num_kv_heads);
  const int64_t i = row / a.num_kv_heads;
  const int64_t slot = a.slot_mapping[i];
  if (slot < 0 || slot >= (int64_t)a.num_blocks * BS) return;
  const int64_t p = slot / BS;
  const int o = (int)(slot % BS);
  const size_t src = (size_t)row * D + chunk * EPC;
  const size_t tile = ((size_t)p * a.num_kv_heads + g) * BS * D;

  const u32x4 kx = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.k) + src * E);
  __builtin_nontemporal_store(
      kx, reinterpret_cast<u32x4 *>(static_cast<char *>(a.k_cache) +
                                    (tile + (size_t)o * D + chunk * EPC) * E));

  // values: the token-grouped layout keeps four consecutive slots of one
  // dim together, elements (o/4)*4*D + d*4 + o%4 of the tile
  const size_t vg = tile + (size_t)(o / 4) * 4 * D;  // the slot group
  const int64_t lead = full_group_leader(a.slot_mapping, i, a.num_tokens, slot);
  if (lead == i) {
    // four tokens' EPC dims: EPC x 4 elements, contiguous, as 16-byte stores
    const size_t vrow = (size_t)a.num_kv_heads * D;  // elements between tokens
    u32x4 vt[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      vt[t] = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.v) +
                                               (src + t * vrow) * E);
    char *dst = static_cast<char *>(a.v_cache) + (vg + (size_t)chunk * EPC * 4) * E;
    if constexpr (E == 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        __builtin_nontemporal_store(u32x4{vt[0][e], vt[1][e], vt[2][e], vt[3][e]},
                                    reinterpret_cast<u32x4 *>(dst) + e);
    } else {
      // 16 bytes = two dims x four tokens; word w of dim pair q
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo[4] = {vt[0][q] & 0xffffu, vt[1][q] & 0xffffu, vt[2][q] & 0xffffu,
                                vt[3][q] & 0xffffu};
        const uint32_t hi[4] = {vt[0][q] >> 16, vt[1][q] >> 16, vt[2][q] >> 16, vt[3][q] >> 16};
        __builtin_nontemporal_store(
            u32x4{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), hi[0] | (hi[1] << 16),
                  hi[2] | (hi[3] << 16)},
            reinterpret_cast<u32x4 *>(dst) + q);
      }
    }
    return;
  }
  if (lead >= 0) return;  // the group's leader writes this token's values

  const u32x4 vx = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.v) + src * E);
  const size_t vb = vg + (o % 4);
  if constexpr (E == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      __builtin_nontemporal_store(
          vx[e], static_cast<uint32_t *>(a.v_cache) + vb + (size_t)(chunk * EPC + e) * 4);
  } else {
    uint16_t *vp = static_cast<uint16_t *>(a.v_cache);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t wd = vx[e >> 1];
      __builtin_nontemporal_store((e & 1) ? (uint16_t)(wd >> 16) : (uint16_t)wd,
                                  vp + vb + (size_t)(chunk * EPC + e) * 4);
    }
  }
}

template <int DT, int D>
static hipError_t launch_rac_d(const CacheWriteArgs &a, int block_size, hipStream_t st) {
  constexpr int CPR = D / (16 / Elem<DT>::bytes);
  const int64_t total = a.num_tokens * a.num_kv_heads * CPR;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (block_size == 16)
    hipLaunchKernelGGL((reshape_and_cache_kernel<DT, D, 16>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((reshape_and_cache_kernel<DT, D, 32>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// Cache write into 8-bit E4M3 pools ("PagedAttention: how vLLM manages the
// KV cache", section "Keep the tensor formula beside the allocator model":
// lower-precision cache formats reduce the bytes per element).  Every
// element x is stored as e4m3(x / scale), the quotient computed in IEEE
// single precision.  One thread converts eight consecutive dims of one
// (token, KV head) row: one 8-byte K store, and eight V bytes four apart -
// or, for the first token of four that fill a whole slot group, the
// group's 32 value bytes of those dims as two 16-byte stores.
template <int IT, int D, int BS>
__global__ void __launch_bounds__(256) reshape_and_cache_fp8_kernel(CacheWriteArgs a) {
  constexpr int EI = Elem<IT>::bytes;
  constexpr int CPR = D / 8;  // 8-element groups per row
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = a.num_tokens * a.num_kv_heads * CPR;
  if (idx >= total) return;
  const int chunk = (int)(idx % CPR);
  const int64_t row = idx / CPR;
  const int g = (int)(row % a.num_kv_heads);
  const int64_t i = row / a.num_kv_heads;
  const int64_t slot = a.slot_mapping[i];
  if (slot < 0 || slot >= (int64_t)a.num_blocks * BS) return;
  const int64_t p = slot / BS;
  const int o = (int)(slot % BS);
  const size_t src = (size_t)row * D + chunk * 8;
  const size_t tile = ((size_t)p * a.num_kv_heads + g) * BS * D;

  uint32_t kw[8 * EI / 4], vw[8 * EI / 4];
#pragma unroll
  for (int u = 0; u < 8 * EI / 16; ++u) {
    const u32x4 x = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.k) + src * EI + 16 * u);
    const u32x4 y = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.v) + src * EI + 16 * u);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kw[4 * u + e] = x[e];
      vw[4 * u + e] = y[e];
    }
  }
  uint32_t kq[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    kq[e / 4] |= e4m3_from_f32(elem<IT>(kw, e) / a.k_scale) << (8 * (e % 4));
  __builtin_nontemporal_store(
      u32x2{kq[0], kq[1]},
      reinterpret_cast<u32x2 *>(static_cast<char *>(a.k_cache) + tile + (size_t)o * D + chunk * 8));

  uint8_t *vc = static_cast<uint8_t *>(a.v_cache);
  const size_t vg = tile + (size_t)(o / 4) * 4 * D;
  const int64_t lead = full_group_leader(a.slot_mapping, i, a.num_tokens, slot);
  if (lead == i) {
    // the group's four tokens, eight dims: one word (four tokens) per dim
    uint32_t word[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    const size_t vrow = (size_t)a.num_kv_heads * D;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t tw[8 * EI / 4];
#pragma unroll
      for (int u = 0; u < 8 * EI / 16; ++u) {
        const u32x4 y = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.v) +
                                                         (src + t * vrow) * EI + 16 * u);
#pragma unroll
        for (int e = 0; e < 4; ++e) tw[4 * u + e] = y[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        word[e] |= e4m3_from_f32(elem<IT>(tw, e) / a.v_scale) << (8 * t);
    }
    u32x4 *dst = reinterpret_cast<u32x4 *>(vc + vg + (size_t)chunk * 8 * 4);
    __builtin_nontemporal_store(u32x4{word[0], word[1], word[2], word[3]}, dst);
    __builtin_nontemporal_store(u32x4{word[4], word[5], word[6], word[7]}, dst + 1);
    return;
  }
  if (lead >= 0) return;  // the group's leader writes this token's values
  const size_t vb = vg + (o % 4);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    __builtin_nontemporal_store(
        static_cast<uint8_t>(e4m3_from_f32(elem<IT>(vw, e) / a.v_scale)),
        vc + vb + (size_t)(chunk * 8 + e) * 4);
}

template <int DT, int CT>
static hipError_t launch_rac_dt(const CacheWriteArgs &a, int head_dim, int block_size,
                                hipStream_t st) {
  if constexpr (CT == DT_FP8) {
    const int64_t total = a.num_tokens * a.num_kv_heads * (head_dim / 8);
    const dim3 grid((unsigned)((total + 255) / 256));
#define PKV_RAC8(DV, BV) \
  hipLaunchKernelGGL((reshape_and_cache_fp8_kernel<DT, DV, BV>), grid, dim3(256), 0, st, a)
    if (head_dim == 128) {
      if (block_size == 16) PKV_RAC8(128, 16); else PKV_RAC8(128, 32);
    } else {
      if (block_size == 16) PKV_RAC8(64, 16); else PKV_RAC8(64, 32);
    }
#undef PKV_RAC8
    return hipGetLastError();
  } else {
    return head_dim == 128 ? launch_rac_d<DT, 128>(a, block_size, st)
                           : launch_rac_d<DT, 64>(a, block_size, st);
  }
}

hipError_t launch_reshape_and_cache(const CacheWriteArgs &a, int dtype,
                                    int cache_dtype, int head_dim, int block_size,
                                    hipStream_t st) {
  if (a.num_tokens == 0) return hipSuccess;
  if (cache_dtype == DT_FP8) {
    switch (dtype) {
      case DT_F32: return launch_rac_dt<DT_F32, DT_FP8>(a, head_dim, block_size, st);
      case DT_F16: return launch_rac_dt<DT_F16, DT_FP8>(a, head_dim, block_size, st);
      default: return launch_rac_dt<DT_BF16, DT_FP8>(a, head_dim, block_size, st);
    }
  }
  switch (dtype) {
    case DT_F32: return launch_rac_dt<DT_F32, DT_F32>(a, head_dim, block_size, st);
    case DT_F16: return launch_rac_dt<DT_F16, DT_F16>(a, head_dim, block_size, st);
    default: return launch_rac_dt<DT_BF16, DT_BF16>(a, head_dim, block_size, st);
  }
}

}  // namespace pkv
