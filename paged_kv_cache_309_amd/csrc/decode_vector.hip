// decode_vector.hip - paged decode attention, one query head per workgroup,
// on the vector ALUs.
//
// What it computes: for one (sequence, query head[, partition]),
// softmax(scale * q . K_t) weighted sum of V_t over the tokens t of the
// sequence (or of the partition), with K_t and V_t gathered block by block
// through the sequence's block table ("Paged Attention" placement notes,
// section "Paged Attention's Approach": the kernel reads the block table and
// walks the request's blocks; "PagedAttention: how vLLM manages the KV
// cache", section "PagedAttention changes addressing inside attention").
// The softmax is the online form (running maximum and running sum, rescaled
// when the maximum grows), which the sketch on the placement-notes page also
// keeps as max_score / sum_exp.
//
// Used for multi-head attention (one KV head per query head), and for fp32
// or very wide query groups, where every query head re-reads its KV head.
//
// Work decomposition (gfx950, wave64):
//  * a workgroup is 4 wavefronts; the sequence's context is cut into
//    16-token tiles, dealt round-robin to the wavefronts;
//  * inside a wavefront, row r (lanes 16r..16r+15) owns tokens 4r..4r+3 of
//    the tile; lane c of the row holds dims c*D/16 .. of each of those keys
//    and, for the values, the D/16 dims it accumulates;
//  * a K tile of one (block, head) is 16 tokens x D contiguous elements, a V
//    tile the same bytes in the token-grouped layout; every row loads whole
//    16-byte chunks, and one load instruction of the wave covers four
//    256-byte runs;
//  * q.k is a per-lane partial dot product reduced over the row with four
//    DPP adds; each row keeps its own running max / sum / accumulator, so no
//    lane talks to another row inside the loop;
//  * the next tile's loads are issued before the current tile is computed,
//    and block-table entries are fetched 64 tiles at a time, one per lane,
//    then broadcast with readlane;
//  * at the end the 16 partial states (4 rows x 4 waves) are merged through
//    LDS, each rescaled to the largest maximum.
#include "pkv_device.h"

namespace pkv {

template <int DT, int D, int BS>
struct VecTile {
  static constexpr int E = Elem<DT>::bytes;
  static constexpr int DQ = D / 16;          // dims per lane on the K side
  static constexpr int KW = DQ * E / 4;      // words per lane per key
  static constexpr int VI = 4 * D * E / 256; // 16-byte V chunks per lane
  static constexpr int VW = VI * 4;          // words per lane for V
  static constexpr int DPV = 4 / E;          // dims per V chunk
  uint32_t k[4][KW];
  uint32_t v[VW];
};

template <int DT, int D, int BS>
__device__ __forceinline__ void load_vec_tile(VecTile<DT, D, BS> &t,
                                              const char *kc, const char *vc,
                                              size_t tile_elem, int r, int c) {
  using Tl = VecTile<DT, D, BS>;
  constexpr int E = Tl::E;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const char *p = kc + (tile_elem + (size_t)(4 * r + i) * D + c * Tl::DQ) * E;
    if constexpr (Tl::KW == 2) {
      const u32x2 x = *reinterpret_cast<const u32x2 *>(p);
      t.k[i][0] = x[0];
      t.k[i][1] = x[1];
    } else {
#pragma unroll
      for (int u = 0; u < Tl::KW / 4; ++u) {
        const u32x4 x = *reinterpret_cast<const u32x4 *>(p + 16 * u);
        t.k[i][4 * u + 0] = x[0];
        t.k[i][4 * u + 1] = x[1];
        t.k[i][4 * u + 2] = x[2];
        t.k[i][4 * u + 3] = x[3];
      }
    }
  }
  const char *pv = vc + (tile_elem + (size_t)r * 4 * D) * E + c * 16;
#pragma unroll
  for (int ii = 0; ii < Tl::VI; ++ii) {
    const u32x4 x = *reinterpret_cast<const u32x4 *>(pv + ii * 256);
    t.v[4 * ii + 0] = x[0];
    t.v[4 * ii + 1] = x[1];
    t.v[4 * ii + 2] = x[2];
    t.v[4 * ii + 3] = x[3];
  }
}

template <int DT, int D, int BS, bool SPLIT>
__global__ void __launch_bounds__(kDecodeThreads)
decode_vector_kernel(DecodeArgs a) {
  using Tl = VecTile<DT, D, BS>;
  constexpr int E = Tl::E;
  constexpr int SUBS = BS / 16;
  constexpr int NACC = Tl::VI * Tl::DPV;  // == D / 16

  const int h = blockIdx.x, s = blockIdx.y, part = blockIdx.z;
  const int Hq = a.num_heads, Hkv = a.num_kv_heads;
  const int g = h / (Hq / Hkv);
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane >> 4, c = lane & 15;

  int L = a.context_lens[s];
  L = max(0, min(L, a.max_blocks * BS));
  const int tok_begin = SPLIT ? part * a.part_tokens : 0;
  const int tok_end = SPLIT ? min(L, tok_begin + a.part_tokens) : L;
  const size_t orow = ((size_t)s * Hq + h) * D;

  if (tok_begin >= tok_end) {
    if (!SPLIT) {
      for (int d = tid; d < D; d += kDecodeThreads) store_elem<DT>(a.out, orow + d, 0.f);
    }
    return;  // an empty partition leaves its workspace entry unused
  }

  // q for this lane's dims, pre-multiplied by scale * log2(e)
  float qv[Tl::DQ];
  {
    uint32_t qw[Tl::KW];
    const char *qp = static_cast<const char *>(a.q) + (orow + c * Tl::DQ) * E;
#pragma unroll
    for (int u = 0; u < Tl::KW; ++u) qw[u] = reinterpret_cast<const uint32_t *>(qp)[u];
#pragma unroll
    for (int e = 0; e < Tl::DQ; ++e) qv[e] = elem<DT>(qw, e) * a.scale_log2;
  }

  const char *kc = static_cast<const char *>(a.k_cache);
  const char *vc = static_cast<const char *>(a.v_cache);
  const int32_t *trow = a.block_tables + (size_t)s * a.max_blocks;
  const unsigned nb = (unsigned)a.num_blocks;

  const int st_begin = tok_begin >> 4;
  const int st_end = (tok_end + 15) >> 4;
  const int n_tiles = st_end - st_begin;
  const int n_mine = n_tiles > w ? (n_tiles - w + 3) >> 2 : 0;

  // block-table entry of this wave's n-th tile, one n per lane
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

  float m = -INFINITY, l = 0.f;
  float acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i) acc[i] = 0.f;

  if (n_mine > 0) {
    int ent_cur = fetch_entries(0);
    int ent_nxt = n_mine > 64 ? fetch_entries(64) : 0;
    Tl cur, nxt;
    load_vec_tile<DT, D, BS>(cur, kc, vc,
                             tile_base(__builtin_amdgcn_readlane(ent_cur, 0), 0), r, c);
    for (int n = 0; n < n_mine; ++n) {
      const int n1 = n + 1;
      if (n1 < n_mine) {
        if ((n1 & 63) == 0) {
          ent_cur = ent_nxt;
          if (n1 + 64 < n_mine) ent_nxt = fetch_entries(n1 + 64);
        }
        load_vec_tile<DT, D, BS>(
            nxt, kc, vc, tile_base(__builtin_amdgcn_readlane(ent_cur, n1 & 63), n1), r, c);
      }

      // ---- logits of this row's four tokens (log2 units) ----
      float sc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < Tl::DQ; ++e) d = fmaf(qv[e], elem<DT>(cur.k[i], e), d);
        sc[i] = row_sum16(d);
      }
      const int t0 = (st_begin + w + 4 * n) * 16 + 4 * r;  // first token of this row
      if ((st_begin + w + 4 * n) * 16 + 16 > tok_end) {
        // last tile: tokens at or past tok_end are masked; their V words
        // may hold anything (NaN included) and are zeroed, not multiplied
        const int nvalid = max(0, min(4, tok_end - t0));
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i >= nvalid) sc[i] = -INFINITY;
        if constexpr (E == 2) {
          const uint32_t m01 = nvalid >= 2 ? 0xffffffffu : (nvalid == 1 ? 0x0000ffffu : 0u);
          const uint32_t m23 = nvalid >= 4 ? 0xffffffffu : (nvalid == 3 ? 0x0000ffffu : 0u);
#pragma unroll
          for (int u = 0; u < Tl::VW; u += 2) {
            cur.v[u] &= m01;
            cur.v[u + 1] &= m23;
          }
        } else {
#pragma unroll
          for (int u = 0; u < Tl::VW; ++u)
            if ((u & 3) >= nvalid) cur.v[u] = 0u;
        }
      }

      // ---- online softmax update of this row's state ----
      const float mb = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      const float m_new = fmaxf(m, mb);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sc[i] - m_use);
      l = fmaf(l, alpha, (p[0] + p[1]) + (p[2] + p[3]));
      m = m_new;

      // ---- weighted values ----
#pragma unroll
      for (int ii = 0; ii < Tl::VI; ++ii) {
        if constexpr (E == 2) {
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const uint32_t *wv = &cur.v[4 * ii + 2 * k2];
            float x = acc[2 * ii + k2] * alpha;
            x = fmaf(p[0], elem<DT>(wv, 0), x);
            x = fmaf(p[1], elem<DT>(wv, 1), x);
            x = fmaf(p[2], elem<DT>(wv, 2), x);
            x = fmaf(p[3], elem<DT>(wv, 3), x);
            acc[2 * ii + k2] = x;
          }
        } else {
          const uint32_t *wv = &cur.v[4 * ii];
          float x = acc[ii] * alpha;
          x = fmaf(p[0], elem<DT>(wv, 0), x);
          x = fmaf(p[1], elem<DT>(wv, 1), x);
          x = fmaf(p[2], elem<DT>(wv, 2), x);
          x = fmaf(p[3], elem<DT>(wv, 3), x);
          acc[ii] = x;
        }
      }
      cur = nxt;
    }
  }

  // ---- merge the 16 partial states (4 rows x 4 waves) through LDS ----
  __shared__ float sm_acc[16][D];
  __shared__ float sm_m[16], sm_l[16];
  const int si = w * 4 + r;
#pragma unroll
  for (int ii = 0; ii < Tl::VI; ++ii)
#pragma unroll
    for (int k2 = 0; k2 < Tl::DPV; ++k2)
      sm_acc[si][(ii * 256 + c * 16) / (4 * E) + k2] = acc[ii * Tl::DPV + k2];
  if (c == 0) {
    sm_m[si] = m;
    sm_l[si] = l;
  }
  __syncthreads();
  for (int d = tid; d < D; d += kDecodeThreads) {
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) M = fmaxf(M, sm_m[i]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float f = fast_exp2(sm_m[i] - M);  // a row that saw no token: m = -inf
      num = fmaf(f, sm_acc[i][d], num);
      den = fmaf(f, sm_l[i], den);
    }
    if constexpr (SPLIT) {
      const size_t pi = ((size_t)s * Hq + h) * a.num_parts + part;
      a.ws_o[pi * D + d] = num;
      if (d == 0) {
        a.ws_m[pi] = M;
        a.ws_l[pi] = den;
      }
    } else {
      store_elem<DT>(a.out, orow + d, num / den);
    }
  }
}

template <int DT, int D, int BS>
static hipError_t launch_vec(const DecodeArgs &a, bool split, hipStream_t st) {
  dim3 grid(a.num_heads, a.num_seqs, split ? a.num_parts : 1);
  if (split)
    hipLaunchKernelGGL((decode_vector_kernel<DT, D, BS, true>), grid,
                       dim3(kDecodeThreads), 0, st, a);
  else
    hipLaunchKernelGGL((decode_vector_kernel<DT, D, BS, false>), grid,
                       dim3(kDecodeThreads), 0, st, a);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_vec_dt(const DecodeArgs &a, int head_dim,
                                int block_size, bool split, hipStream_t st) {
  if (head_dim == 128)
    return block_size == 16 ? launch_vec<DT, 128, 16>(a, split, st)
                            : launch_vec<DT, 128, 32>(a, split, st);
  return block_size == 16 ? launch_vec<DT, 64, 16>(a, split, st)
                          : launch_vec<DT, 64, 32>(a, split, st);
}

hipError_t launch_decode_vector(const DecodeArgs &a, int dtype, int head_dim,
                                int block_size, bool split, hipStream_t st) {
  switch (dtype) {
    case DT_F32: return launch_vec_dt<DT_F32>(a, head_dim, block_size, split, st);
    case DT_F16: return launch_vec_dt<DT_F16>(a, head_dim, block_size, split, st);
    default: return launch_vec_dt<DT_BF16>(a, head_dim, block_size, split, st);
  }
}

}  // namespace pkv
