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
// With MQ the same kernel serves chunked prefill where the matrix-core
// kernel does not (fp32, 8-bit caches): a workgroup then takes one (query
// token, query head) and attends to the token's causal prefix ("Inside
// vLLM: How PagedAttention Eliminates KV-Cache Memory Waste", section
// "Continuous Batching and Chunked Prefill").
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
//  * the next tile's loads are issued before the current tile is computed;
//    the tile's address is a scalar, each lane's offset inside a tile is
//    fixed for the whole loop;
//  * tiles are streamed (non-temporal loads), except the leading blocks the
//    neighbouring sequence's table maps to the same physical blocks - a
//    shared prefix, which every sharer reads - whose plain loads keep them
//    in cache.  The two kinds of tile are two walks, so the waits of each
//    stay exact (a branch between load kinds per tile makes the compiler
//    merge them or drain the next tile's loads).  128 sequences over one
//    1024-token prefix, 32 heads: 201.8 -> 154.5 us;
//  * at the end the 16 partial states (4 rows x 4 waves) are merged through
//    LDS, each rescaled to the largest maximum;
//  * split launches instead give each wave partitions of its own: wave w of
//    workgroup z walks every tile of partitions (4z + w) * k .. + k - 1 as
//    one stream (k = parts_per_wave, 1 to 4).  At the last tile of each
//    partition every row parks its own state in LDS with plain stores (no
//    cross-lane step, nothing to wait for inside the walk) and starts
//    afresh; after the walk the wave merges each partition's four row
//    states and writes the partials to the workspace.  The host picks k so
//    that the whole grid is resident at once.
#include <algorithm>
#include <type_traits>

#include "pkv_device.h"

namespace pkv {

template <int DT, int D>
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

// Sequence of query row r: the s with query_start_loc[s] <= r <
// query_start_loc[s+1] (binary search over the nondecreasing starts).
__device__ __forceinline__ int seq_of_row(const int32_t *qsl, int num_seqs, int r) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qsl[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// QT: element type of q and out; CT: of the caches (QT, or 8-bit E4M3)
template <int QT, int CT, int D, int BS, bool SPLIT, bool MQ = false>
__global__ void __launch_bounds__(kDecodeThreads)
decode_vector_kernel(DecodeArgs a) {
  using Tl = VecTile<CT, D>;
  constexpr int E = Tl::E;
  constexpr int KWQ = Tl::DQ * Elem<QT>::bytes / 4;  // words of q per lane
  constexpr int NACC = Tl::VI * Tl::DPV;  // == D / 16

  static_assert(!(MQ && SPLIT), "multi-query runs single-pass");
  const int Hq = a.num_heads, Hkv = a.num_kv_heads;
  // multi-query: one workgroup per (query row, head), flattened on x
  const int h = MQ ? (int)(blockIdx.x % Hq) : (int)blockIdx.x;
  const int qrow = MQ ? (int)(blockIdx.x / Hq) : 0;
  const int g = h / (Hq / Hkv);
  const int tid = threadIdx.x;

  // LDS: the final merge of partial states; before the loop it holds the
  // length histogram of the longest-first order
  // (split: the parked row states, four per partition of each wave)
  constexpr int kStates = SPLIT ? kDecodeWaves * kMaxPartsPerWave * 4 : 16;
  __shared__ float sm_acc[kStates][D];
  __shared__ float sm_m[kStates], sm_l[kStates];
  static_assert(sizeof(sm_acc) >= kOrderScratchInts * sizeof(int), "order scratch");
  const int s = MQ ? seq_of_row(a.query_start_loc, a.num_seqs, qrow)
               : SPLIT ? (int)blockIdx.y
                       : longest_first_seq<kDecodeThreads>(
                             a.context_lens, a.num_seqs, a.max_blocks * BS, blockIdx.y,
                             reinterpret_cast<int *>(&sm_acc[0][0]));
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63, r = lane >> 4, c = lane & 15;
  constexpr int kWaves = kDecodeWaves;
  // split: this wave's first partition and how many it takes (the split
  // path has no workgroup barrier, so a wave with nothing to do leaves)
  const int ppw = SPLIT ? a.parts_per_wave : 1;
  const int part0 = SPLIT ? ((int)blockIdx.z * kWaves + w) * ppw : 0;
  if (SPLIT && part0 >= a.num_parts) return;

  int L = a.context_lens[s];
  L = max(0, min(L, a.max_blocks * BS));
  if constexpr (MQ) {
    // the chunk is the last C tokens of the context; row qrow attends to
    // the tokens up to and including its own position
    const int q0 = a.query_start_loc[s];
    const int C = a.query_start_loc[s + 1] - q0;
    L = max(0, min(L, L - C + (qrow - q0) + 1));
  }
  // shared-prefix decode: the prefix kernel computed tokens [0, ptok) in
  // n_pre chunks; the walk starts after them (ptok is a multiple of the
  // block size, so of the 16-token tile)
  int ptok = 0, n_pre = 0;
  if (!SPLIT && !MQ && a.seq_prefix) {
    ptok = max(0, min(a.seq_prefix[s], L)) & ~15;
    // at most one chunk per row state (the library plans at most 16 chunks)
    n_pre = min(min(a.n_pchunks, 16), (ptok + a.pchunk_tokens - 1) / a.pchunk_tokens);
  }
  const int tok_begin = SPLIT ? part0 * a.part_tokens : ptok;
  const int tok_end = SPLIT ? min(L, min(a.num_parts, part0 + ppw) * a.part_tokens) : L;
  const size_t orow = ((size_t)(MQ ? qrow : s) * Hq + h) * D;

  if (tok_begin >= tok_end && n_pre == 0) {
    if (!SPLIT) {
      for (int d = tid; d < D; d += kDecodeThreads) store_elem<QT>(a.out, orow + d, 0.f);
    }
    return;  // empty partitions leave their workspace entries unused
  }

  // q for this lane's dims, pre-multiplied by scale * log2(e) (and the
  // key dequantisation scale of an 8-bit cache)
  float qv[Tl::DQ];
  {
    uint32_t qw[KWQ];
    const char *qp = static_cast<const char *>(a.q) + (orow + c * Tl::DQ) * Elem<QT>::bytes;
#pragma unroll
    for (int u = 0; u < KWQ; ++u) qw[u] = reinterpret_cast<const uint32_t *>(qp)[u];
#pragma unroll
    for (int e = 0; e < Tl::DQ; ++e) qv[e] = elem<QT>(qw, e) * a.scale_log2;
  }

  const char *kc = static_cast<const char *>(a.k_cache);
  const char *vc = static_cast<const char *>(a.v_cache);
  const int32_t *trow = a.block_tables + (size_t)s * a.max_blocks;

  const int st_begin = tok_begin >> 4;
  const int st_end = (tok_end + 15) >> 4;
  const int n_tiles = st_end - st_begin;
  // the wave's tiles: tile0 + kStride * n for n < n_mine -- every tile of
  // its partitions (split), or every fourth tile of the context
  constexpr int kStride = SPLIT ? 1 : kWaves;
  const int tile0 = SPLIT ? st_begin : st_begin + w;
  const int n_mine = SPLIT ? n_tiles : (n_tiles > w ? (n_tiles - w + kWaves - 1) / kWaves : 0);
  // split: tiles per partition, the last tile of the current partition and
  // how many partitions have been parked in LDS (all wave-uniform)
  const int tpp = a.part_tokens >> 4;
  int flush_at = min(st_end, st_begin + tpp) - 1;
  int n_flushed = 0;

  // lane offsets inside a tile, in bytes
  const uint32_t koff = (uint32_t)((4 * r * D + c * Tl::DQ) * E);
  const uint32_t voff = (uint32_t)(r * 4 * D * E + c * 16);

  float m = -INFINITY, l = 0.f;
  float acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i) acc[i] = 0.f;
  if (n_pre > 0) {
    // shared-prefix decode: row state 4w + r starts as the partial state of
    // prefix chunk 4w + r, so the final merge takes the prefix in with the
    // rest, and these loads overlap the first tiles' instead of trailing
    // the walk
    const int si = w * 4 + r;
    if (si < n_pre) {
      const size_t pc = ((size_t)s * Hq + h) * a.n_pchunks + si;
      m = a.pws_m[pc];
      l = a.pws_l[pc];
#pragma unroll
      for (int ii = 0; ii < Tl::VI; ++ii)
#pragma unroll
        for (int k2 = 0; k2 < Tl::DPV; ++k2)
          acc[ii * Tl::DPV + k2] = a.pws_o[pc * D + (ii * 256 + c * 16) / (4 * E) + k2];
    }
  }

  // one tile's loads: non-temporal (streamed), or plain for a block the
  // neighbouring sequence shares, which the other sharers read too
  auto load_with = [&](Tl &t, size_t tile_bytes, auto keep) {
    constexpr bool KEEP = decltype(keep)::value;
    const char *kp = kc + tile_bytes + koff;
    const char *vp = vc + tile_bytes + voff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (Tl::KW == 1) {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(kp + i * D * E);
        if constexpr (KEEP) t.k[i][0] = *p;
        else t.k[i][0] = __builtin_nontemporal_load(p);
      } else if constexpr (Tl::KW == 2) {
        const u32x2 x = KEEP ? load_keep8(kp + i * D * E) : load_stream8(kp + i * D * E);
        t.k[i][0] = x[0];
        t.k[i][1] = x[1];
      } else {
#pragma unroll
        for (int u = 0; u < Tl::KW / 4; ++u) {
          const char *p = kp + i * D * E + 16 * u;
          const u32x4 x = KEEP ? load_keep16(p) : load_stream16(p);
          t.k[i][4 * u + 0] = x[0];
          t.k[i][4 * u + 1] = x[1];
          t.k[i][4 * u + 2] = x[2];
          t.k[i][4 * u + 3] = x[3];
        }
      }
    }
#pragma unroll
    for (int ii = 0; ii < Tl::VI; ++ii) {
      const u32x4 x = KEEP ? load_keep16(vp + ii * 256) : load_stream16(vp + ii * 256);
      t.v[4 * ii + 0] = x[0];
      t.v[4 * ii + 1] = x[1];
      t.v[4 * ii + 2] = x[2];
      t.v[4 * ii + 3] = x[3];
    }
  };
  auto load = [&](Tl &t, size_t tile_bytes) { load_with(t, tile_bytes, std::false_type{}); };
  auto load_keep = [&](Tl &t, size_t tile_bytes) { load_with(t, tile_bytes, std::true_type{}); };

  auto compute = [&](Tl &t, int n) {
    // ---- logits of this row's four tokens (log2 units) ----
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < Tl::DQ; ++e) d = fmaf(qv[e], elem<CT>(t.k[i], e), d);
      sc[i] = row_sum16(d);
    }
    const int tile_tok = (tile0 + kStride * n) * 16;
    if (tile_tok + 16 > tok_end) {
      // last tile: tokens at or past tok_end are masked; their V words may
      // hold anything (NaN included) and are zeroed, not multiplied
      const int nvalid = max(0, min(4, tok_end - tile_tok - 4 * r));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i >= nvalid) sc[i] = -INFINITY;
      if constexpr (E == 1) {
        // one word = one dim's four tokens, one byte each
        const uint32_t mk = nvalid >= 4 ? 0xffffffffu : ((1u << (8 * nvalid)) - 1u);
#pragma unroll
        for (int u = 0; u < Tl::VW; ++u) t.v[u] &= mk;
      } else if constexpr (E == 2) {
        const uint32_t m01 = nvalid >= 2 ? 0xffffffffu : (nvalid == 1 ? 0x0000ffffu : 0u);
        const uint32_t m23 = nvalid >= 4 ? 0xffffffffu : (nvalid == 3 ? 0x0000ffffu : 0u);
#pragma unroll
        for (int u = 0; u < Tl::VW; u += 2) {
          t.v[u] &= m01;
          t.v[u + 1] &= m23;
        }
      } else {
#pragma unroll
        for (int u = 0; u < Tl::VW; ++u)
          if ((u & 3) >= nvalid) t.v[u] = 0u;
      }
    }

    // ---- online softmax: move the row's maximum only when a logit
    //      exceeds it by more than the slack (wave-uniform branch) ----
    const float mb = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    if (wave_any(mb > m + kRescaleSlack)) {
      const float m_new = fmaxf(m, mb);
      const float alpha = fast_exp2(m - (m_new == -INFINITY ? 0.f : m_new));
      l *= alpha;
#pragma unroll
      for (int i = 0; i < NACC; ++i) acc[i] *= alpha;
      m = m_new;
    }
    const float m_use = m == -INFINITY ? 0.f : m;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sc[i] - m_use);
    l += (p[0] + p[1]) + (p[2] + p[3]);

    // ---- weighted values ----
#pragma unroll
    for (int ii = 0; ii < Tl::VI; ++ii) {
#pragma unroll
      for (int k2 = 0; k2 < Tl::DPV; ++k2) {
        // the four tokens of one dim: k2*E words into the 16-byte chunk
        const uint32_t *wv = &t.v[4 * ii + k2 * E];
        float x = acc[ii * Tl::DPV + k2];
        x = fmaf(p[0], elem<CT>(wv, 0), x);
        x = fmaf(p[1], elem<CT>(wv, 1), x);
        x = fmaf(p[2], elem<CT>(wv, 2), x);
        x = fmaf(p[3], elem<CT>(wv, 3), x);
        acc[ii * Tl::DPV + k2] = x;
      }
    }

    if constexpr (SPLIT) {
      if (tile0 + n == flush_at) {
        // ---- the partition's last tile: each row parks its state (slot
        //      4 * (partition of the wave) + row) and starts afresh ----
        const int slot = (w * kMaxPartsPerWave + n_flushed) * 4 + r;
#pragma unroll
        for (int ii = 0; ii < Tl::VI; ++ii)
#pragma unroll
          for (int k2 = 0; k2 < Tl::DPV; ++k2) {
            sm_acc[slot][(ii * 256 + c * 16) / (4 * E) + k2] = acc[ii * Tl::DPV + k2];
            acc[ii * Tl::DPV + k2] = 0.f;
          }
        if (c == 0) {
          sm_m[slot] = m;
          sm_l[slot] = l;
        }
        m = -INFINITY;
        l = 0.f;
        ++n_flushed;
        flush_at = min(st_end - 1, flush_at + tpp);
      }
    }
  };

  if (n_mine > 0) {
    // tiles of a prefix the neighbouring sequence shares (none to look for
    // when the prefix kernel took the shared prefix)
    const int shared_tiles =
        a.seq_prefix ? 0
                     : shared_prefix_blocks<BS>(a.block_tables, a.max_blocks, a.num_seqs, s,
                                                tok_end, lane) *
                           (BS / 16);
    // the wave's tiles in front of shared_tiles are read with plain loads,
    // the rest streamed; two walks, each with its own exact waits
    const int n_keep =
        min(n_mine, shared_tiles > tile0 ? (shared_tiles - tile0 + kStride - 1) / kStride : 0);
    constexpr size_t tile_elems = (size_t)16 * D;
    if (n_keep > 0)
      walk_tiles<Tl, kStride>(trow, tile0, n_keep, BS / 16, (unsigned)a.num_blocks,
                              (size_t)g * BS * D * E, (size_t)Hkv * BS * D * E,
                              tile_elems * E, load_keep, compute);
    if (n_mine > n_keep)
      walk_tiles<Tl, kStride>(trow, tile0 + kStride * n_keep, n_mine - n_keep, BS / 16,
                              (unsigned)a.num_blocks, (size_t)g * BS * D * E,
                              (size_t)Hkv * BS * D * E, tile_elems * E, load,
                              [&](Tl &t, int n) { compute(t, n + n_keep); });
  }

  if constexpr (SPLIT) {
    // ---- each parked partition: merge its four row states, rescaled to
    //      their largest maximum, into the workspace.  LDS written and read
    //      by this wave only, so ordering inside the wave is all it needs.
    //      Row 0 saw the partition's first token, so M is finite; a row
    //      that saw none has m = -inf and weight 0.  The partials are
    //      written through L2 (8.5 MB at 512-token partitions of 8 x 32768
    //      tokens x 32 heads: 11.6 us less than plain stores). ----
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int j = 0; j < n_flushed; ++j) {
      const int base = (w * kMaxPartsPerWave + j) * 4;
      float M = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) M = fmaxf(M, sm_m[base + i]);
      float f[4], den = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[i] = fast_exp2(sm_m[base + i] - M);
        den = fmaf(f[i], sm_l[base + i], den);
      }
      const size_t pi = ((size_t)s * Hq + h) * a.num_parts + part0 + j;
      for (int d = lane; d < D; d += 64) {
        float num = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) num = fmaf(f[i], sm_acc[base + i][d], num);
        store_through(&a.ws_o[pi * D + d], num * a.v_scale);
      }
      if (lane == 0) {
        store_through(&a.ws_m[pi], M);
        store_through(&a.ws_l[pi], den);
      }
    }
    return;
  }

  // ---- merge the 16 partial states (4 rows x 4 waves) through LDS ----
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
    num *= a.v_scale;  // value dequantisation (1 for 16/32-bit caches)
    store_elem<QT>(a.out, orow + d, num / den);
  }
}

template <int QT, int CT, int D, int BS>
static hipError_t launch_vec(const DecodeArgs &a, bool split, hipStream_t st) {
  if (split) {
    // every wave of the grid resident at once: 16 waves per compute unit
    const int64_t units = (int64_t)a.num_seqs * a.num_heads * a.num_parts;
    const int64_t resident = (int64_t)device_compute_units() * 4 * kDecodeWaves;
    DecodeArgs b = a;
    b.parts_per_wave = split_parts_per_wave(units, resident, a.num_parts);
    const int per_wg = kDecodeWaves * b.parts_per_wave;
    const dim3 grid(a.num_heads, a.num_seqs, (a.num_parts + per_wg - 1) / per_wg);
    hipLaunchKernelGGL((decode_vector_kernel<QT, CT, D, BS, true>), grid,
                       dim3(kDecodeThreads), 0, st, b);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((decode_vector_kernel<QT, CT, D, BS, false>),
                     dim3(a.num_heads, a.num_seqs, 1), dim3(kDecodeThreads), 0, st, a);
  return hipGetLastError();
}

template <int QT, int CT, int D, int BS>
static hipError_t launch_vec_mq(const DecodeArgs &a, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)a.num_query_tokens * a.num_heads));
  hipLaunchKernelGGL((decode_vector_kernel<QT, CT, D, BS, false, true>), grid,
                     dim3(kDecodeThreads), 0, st, a);
  return hipGetLastError();
}

template <int QT, int CT>
static hipError_t launch_vec_mq_dt(const DecodeArgs &a, int head_dim, int block_size,
                                   hipStream_t st) {
  if (head_dim == 128)
    return block_size == 16 ? launch_vec_mq<QT, CT, 128, 16>(a, st)
                            : launch_vec_mq<QT, CT, 128, 32>(a, st);
  return block_size == 16 ? launch_vec_mq<QT, CT, 64, 16>(a, st)
                          : launch_vec_mq<QT, CT, 64, 32>(a, st);
}

hipError_t launch_prefill_vector(const DecodeArgs &a, int dtype, int cache_dtype, int head_dim,
                                 int block_size, hipStream_t st) {
  if (a.num_query_tokens == 0 || a.num_seqs == 0) return hipSuccess;
  if (cache_dtype == DT_FP8) {
    switch (dtype) {
      case DT_F32: return launch_vec_mq_dt<DT_F32, DT_FP8>(a, head_dim, block_size, st);
      case DT_F16: return launch_vec_mq_dt<DT_F16, DT_FP8>(a, head_dim, block_size, st);
      default: return launch_vec_mq_dt<DT_BF16, DT_FP8>(a, head_dim, block_size, st);
    }
  }
  switch (dtype) {
    case DT_F32: return launch_vec_mq_dt<DT_F32, DT_F32>(a, head_dim, block_size, st);
    case DT_F16: return launch_vec_mq_dt<DT_F16, DT_F16>(a, head_dim, block_size, st);
    default: return launch_vec_mq_dt<DT_BF16, DT_BF16>(a, head_dim, block_size, st);
  }
}

template <int QT, int CT>
static hipError_t launch_vec_dt(const DecodeArgs &a, int head_dim,
                                int block_size, bool split, hipStream_t st) {
  if (head_dim == 128)
    return block_size == 16 ? launch_vec<QT, CT, 128, 16>(a, split, st)
                            : launch_vec<QT, CT, 128, 32>(a, split, st);
  return block_size == 16 ? launch_vec<QT, CT, 64, 16>(a, split, st)
                          : launch_vec<QT, CT, 64, 32>(a, split, st);
}

hipError_t launch_decode_vector(const DecodeArgs &a, int dtype, int cache_dtype,
                                int head_dim, int block_size, bool split,
                                hipStream_t st) {
  if (cache_dtype == DT_FP8) {
    switch (dtype) {
      case DT_F32: return launch_vec_dt<DT_F32, DT_FP8>(a, head_dim, block_size, split, st);
      case DT_F16: return launch_vec_dt<DT_F16, DT_FP8>(a, head_dim, block_size, split, st);
      default: return launch_vec_dt<DT_BF16, DT_FP8>(a, head_dim, block_size, split, st);
    }
  }
  switch (dtype) {
    case DT_F32: return launch_vec_dt<DT_F32, DT_F32>(a, head_dim, block_size, split, st);
    case DT_F16: return launch_vec_dt<DT_F16, DT_F16>(a, head_dim, block_size, split, st);
    default: return launch_vec_dt<DT_BF16, DT_BF16>(a, head_dim, block_size, split, st);
  }
}

}  // namespace pkv
