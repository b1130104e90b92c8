// decode_mfma.hip - paged decode attention for grouped-query attention on
// the matrix cores (fp16 / bf16).
//
// With G = Hq / Hkv query heads sharing one KV head, the G queries of a
// (sequence, KV head) meet every key and value of that head, so the two
// products are small dense GEMMs: S^T[16 tokens x G] = K[16 x D] . Q^T and
// O^T[D x G] += V^T[D x 16 tokens] . P^T.  Grouped-query attention shrinks
// the KV-head term of the cache ("PagedAttention: how vLLM manages the KV
// cache", section "Keep the tensor formula beside the allocator model"); the
// walk through the block table and the online softmax are those of the
// vector kernel ("Paged Attention" placement notes, section "Paged
// Attention's Approach").
//
// One workgroup (4 wavefronts) per (sequence, KV head[, partition]); each
// K/V tile is read from HBM once for all G heads.  Per 16-token tile a
// wavefront issues D/32 v_mfma_f32_16x16x32 (keys as the A operand, 16
// tokens x 32 dims per lane-group, queries as B, one head per column) and
// 2*D/16 v_mfma_f32_16x16x16 (values as A: each lane holds 4 consecutive
// tokens of one dim, which is what the token-grouped V layout stores
// contiguously; probabilities as B).  The probabilities go in as a
// high and a low half-precision part (p = hi + lo to about 16 bits), so the
// value product keeps near-fp32 weights.
//
// The output of the QK product leaves lane l holding tokens 4*(l/16)+i of
// head l%16, which is exactly the layout the PV product wants for its B
// operand, so the probabilities never move between lanes.  Heads >= G are
// padding: their logits are masked to -inf.
#include "pkv_device.h"

namespace pkv {

template <int DT> struct MfmaOps;

template <> struct MfmaOps<DT_BF16> {
  __device__ static __forceinline__ f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
        __builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
  }
  // p -> (hi, lo) bit patterns with hi + lo ~= p
  __device__ static __forceinline__ void split(float p, uint32_t &hi, uint32_t &lo) {
    hi = from_f32<DT_BF16>(p);
    lo = from_f32<DT_BF16>(p - __uint_as_float(hi << 16));
  }
};

template <> struct MfmaOps<DT_F16> {
  __device__ static __forceinline__ f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(
        __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(
        __builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ void split(float p, uint32_t &hi, uint32_t &lo) {
    const _Float16 h = static_cast<_Float16>(p);
    hi = __builtin_bit_cast(uint16_t, h);
    lo = __builtin_bit_cast(uint16_t, static_cast<_Float16>(p - static_cast<float>(h)));
  }
};

template <int D>
struct MfmaTile {
  u32x4 k[D / 32];  // A operand of the QK products
  u32x2 v[D / 16];  // A operand of the PV products
};

template <int DT, int D, int BS>
__device__ __forceinline__ void load_mfma_tile(MfmaTile<D> &t, const char *kc,
                                               const char *vc, size_t tile_elem,
                                               int col, int grp) {
  constexpr int E = 2;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    t.k[kk] = *reinterpret_cast<const u32x4 *>(
        kc + (tile_elem + (size_t)col * D + (kk * 4 + grp) * 8) * E);
#pragma unroll
  for (int nt = 0; nt < D / 16; ++nt)
    t.v[nt] = *reinterpret_cast<const u32x2 *>(
        vc + (tile_elem + (size_t)grp * 4 * D + (nt * 16 + col) * 4) * E);
}

template <int DT, int D, int BS, bool SPLIT>
__global__ void __launch_bounds__(kDecodeThreads)
decode_mfma_kernel(DecodeArgs a) {
  using Ops = MfmaOps<DT>;
  constexpr int SUBS = BS / 16;
  constexpr int NT = D / 16;

  const int g = blockIdx.x, s = blockIdx.y, part = blockIdx.z;
  const int Hq = a.num_heads, Hkv = a.num_kv_heads;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, col = lane & 15, grp = lane >> 4;

  int L = a.context_lens[s];
  L = max(0, min(L, a.max_blocks * BS));
  const int tok_begin = SPLIT ? part * a.part_tokens : 0;
  const int tok_end = SPLIT ? min(L, tok_begin + a.part_tokens) : L;

  if (tok_begin >= tok_end) {
    if (!SPLIT) {
      for (int i = tid; i < G * D; i += kDecodeThreads)
        store_elem<DT>(a.out, ((size_t)s * Hq + g * G) * D + i, 0.f);
    }
    return;
  }

  // Q^T operand: lane holds head `col`, dims (kk*4+grp)*8 .. +8
  u32x4 qop[D / 32];
  {
    const char *qp = static_cast<const char *>(a.q) + ((size_t)s * Hq + g * G + col) * D * 2;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      qop[kk] = col < G ? *reinterpret_cast<const u32x4 *>(qp + (kk * 4 + grp) * 16)
                        : u32x4{0u, 0u, 0u, 0u};
  }

  const char *kc = static_cast<const char *>(a.k_cache);
  const char *vc = static_cast<const char *>(a.v_cache);
  const int32_t *trow = a.block_tables + (size_t)s * a.max_blocks;
  const unsigned nb = (unsigned)a.num_blocks;

  const int st_begin = tok_begin >> 4;
  const int st_end = (tok_end + 15) >> 4;
  const int n_tiles = st_end - st_begin;
  const int n_mine = n_tiles > w ? (n_tiles - w + 3) >> 2 : 0;

  auto fetch_entries = [&](int n0) -> int {
    const int n = n0 + lane;
    if (n >= n_mine) return 0;
    return trow[(st_begin + w + 4 * n) / SUBS];
  };
  auto tile_base = [&](int ent, int n) -> size_t {
    const int phys = (unsigned)ent < nb ? ent : 0;
    const int k = st_begin + w + 4 * n;
    return ((size_t)phys * Hkv + g) * BS * D + (size_t)(k % SUBS) * 16 * D;
  };

  float m = -INFINITY, l = 0.f;  // head `col`; l is this lane's share
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (n_mine > 0) {
    int ent_cur = fetch_entries(0);
    int ent_nxt = n_mine > 64 ? fetch_entries(64) : 0;
    MfmaTile<D> cur, nxt;
    load_mfma_tile<DT, D, BS>(cur, kc, vc,
                              tile_base(__builtin_amdgcn_readlane(ent_cur, 0), 0), col, grp);
    for (int n = 0; n < n_mine; ++n) {
      const int n1 = n + 1;
      if (n1 < n_mine) {
        if ((n1 & 63) == 0) {
          ent_cur = ent_nxt;
          if (n1 + 64 < n_mine) ent_nxt = fetch_entries(n1 + 64);
        }
        load_mfma_tile<DT, D, BS>(
            nxt, kc, vc, tile_base(__builtin_amdgcn_readlane(ent_cur, n1 & 63), n1), col, grp);
      }

      // S^T[token 4*grp+i][head col]
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) sacc = Ops::qk(cur.k[kk], qop[kk], sacc);

      const int t0 = (st_begin + w + 4 * n) * 16 + 4 * grp;
      const bool tail = (st_begin + w + 4 * n) * 16 + 16 > tok_end;
      const int nvalid = tail ? max(0, min(4, tok_end - t0)) : 4;
      float sc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sc[i] = (i < nvalid && col < G) ? sacc[i] * a.scale_log2 : -INFINITY;
      if (tail) {
        const uint32_t m01 = nvalid >= 2 ? 0xffffffffu : (nvalid == 1 ? 0x0000ffffu : 0u);
        const uint32_t m23 = nvalid >= 4 ? 0xffffffffu : (nvalid == 3 ? 0x0000ffffu : 0u);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          cur.v[nt][0] &= m01;
          cur.v[nt][1] &= m23;
        }
      }

      // running max of head `col` over the 4 lanes that share it
      float mb = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      mb = fmaxf(mb, __shfl_xor(mb, 16));
      mb = fmaxf(mb, __shfl_xor(mb, 32));
      const float m_new = fmaxf(m, mb);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sc[i] - m_use);
      l = fmaf(l, alpha, (p[0] + p[1]) + (p[2] + p[3]));
      m = m_new;

      uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
      Ops::split(p[0], h0, l0);
      Ops::split(p[1], h1, l1);
      Ops::split(p[2], h2, l2);
      Ops::split(p[3], h3, l3);
      const u32x2 phi = {h0 | (h1 << 16), h2 | (h3 << 16)};
      const u32x2 plo = {l0 | (l1 << 16), l2 | (l3 << 16)};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4 x = acc[nt] * alpha;
        x = Ops::pv(cur.v[nt], phi, x);
        x = Ops::pv(cur.v[nt], plo, x);
        acc[nt] = x;
      }
      cur = nxt;
    }
  }

  // ---- merge the 4 wavefronts through LDS ----
  __shared__ float sm_o[kDecodeWaves][16][D + 4];
  __shared__ float sm_m[kDecodeWaves][16], sm_l[kDecodeWaves][16];
  float lt = l + __shfl_xor(l, 16);
  lt += __shfl_xor(lt, 32);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_o[w][col][nt * 16 + 4 * grp + i] = acc[nt][i];
  if (grp == 0) {
    sm_m[w][col] = m;
    sm_l[w][col] = lt;
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kDecodeThreads) {
    const int hh = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < kDecodeWaves; ++i) M = fmaxf(M, sm_m[i][hh]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int i = 0; i < kDecodeWaves; ++i) {
      const float f = fast_exp2(sm_m[i][hh] - M);
      num = fmaf(f, sm_o[i][hh][d], num);
      den = fmaf(f, sm_l[i][hh], den);
    }
    const int h = g * G + hh;
    if constexpr (SPLIT) {
      const size_t pi = ((size_t)s * Hq + h) * a.num_parts + part;
      a.ws_o[pi * D + d] = num;
      if (d == 0) {
        a.ws_m[pi] = M;
        a.ws_l[pi] = den;
      }
    } else {
      store_elem<DT>(a.out, ((size_t)s * Hq + h) * D + d, num / den);
    }
  }
}

template <int DT, int D, int BS>
static hipError_t launch_mfma(const DecodeArgs &a, bool split, hipStream_t st) {
  dim3 grid(a.num_kv_heads, a.num_seqs, split ? a.num_parts : 1);
  if (split)
    hipLaunchKernelGGL((decode_mfma_kernel<DT, D, BS, true>), grid,
                       dim3(kDecodeThreads), 0, st, a);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<DT, D, BS, false>), grid,
                       dim3(kDecodeThreads), 0, st, a);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_mfma_dt(const DecodeArgs &a, int head_dim,
                                 int block_size, bool split, hipStream_t st) {
  if (head_dim == 128)
    return block_size == 16 ? launch_mfma<DT, 128, 16>(a, split, st)
                            : launch_mfma<DT, 128, 32>(a, split, st);
  return block_size == 16 ? launch_mfma<DT, 64, 16>(a, split, st)
                          : launch_mfma<DT, 64, 32>(a, split, st);
}

hipError_t launch_decode_mfma(const DecodeArgs &a, int dtype, int head_dim,
                              int block_size, bool split, hipStream_t st) {
  if (dtype == DT_F16) return launch_mfma_dt<DT_F16>(a, head_dim, block_size, split, st);
  return launch_mfma_dt<DT_BF16>(a, head_dim, block_size, split, st);
}

}  // namespace pkv
