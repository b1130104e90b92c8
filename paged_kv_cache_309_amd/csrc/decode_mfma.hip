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
// One workgroup (4 wavefronts) per (sequence, KV head); each K/V tile is
// read from HBM once for all G heads.  Split launches give each wavefront a
// partition of its own instead (wave w of workgroup z: partition 4z + w),
// walked as one stream of tiles.  The wave's state is already the whole
// partial of its G heads, so it goes to the workspace through the wave's
// own slice of LDS, with no barrier and no merge across wavefronts.  Per 16-token tile a
// wavefront issues D/32 v_mfma_f32_16x16x32 for the logits (keys as the A
// operand: 16 tokens x 32 dims, one token per lane-column; queries as B, one
// head per column) and 2 x D/16 v_mfma_f32_16x16x16 for the values (values
// as A: each lane holds four consecutive tokens of one dim, which the
// token-grouped V layout stores contiguously; probabilities as B).
//
// Lane layouts:
//  * the logits come out as lane l holding tokens 4*(l/16)+i of head l%16,
//    exactly the B operand layout of the value product, so probabilities
//    never move between lanes;
//  * the value product's row index m (= lane l%16 of the A operand) is
//    mapped to dim 32*u + 2*m + j for n-tile 2*u + j, so that every lane's
//    A operands of two consecutive n-tiles are one 16-byte chunk of the V
//    tile, and one load instruction covers four 256-byte runs;
//  * heads >= G are padding columns, masked to -inf;
//  * an 8-bit K tile with 128-byte rows is loaded as whole rows: load c,
//    lane (col, grp) reads token 8c + col%8, 16-byte chunk 2*grp + col/8;
//    one DPP move per dword then gives lane (col, grp) token col's chunks
//    2*grp and 2*grp+1 (dims 32*grp .. 32*grp+31).  Loads that each cover
//    half of sixteen rows read the 8-bit cache about 5% slower on MI355X.
//
// The probabilities enter the value product as a high and a low
// half-precision part (p = hi + lo to about 16 significant bits), so the
// weights keep near-fp32 precision.  Over 8-bit caches, whose values carry
// 4 significant bits, one operand rounded to the 16-bit type is used.
#include "mfma_ops.h"

namespace pkv {

// Half-row exchange: in each row of 16 lanes, the lanes that BANKS enables
// (bit i: lanes 4i..4i+3 of the row) take `src` from lane l ^ 8 (DPP
// row_ror:8), the others keep `old`.  One DPP move.
template <int BANKS>
__device__ __forceinline__ uint32_t from_other_half(uint32_t old, uint32_t src) {
  constexpr int kRowRor8 = 0x128;
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
      static_cast<int>(old), static_cast<int>(src), kRowRor8, 0xF, BANKS, false));
}

// QT: element type of q and out (16-bit); CT: of the caches (QT or E4M3)
// PFX: the shared-prefix partials of multi-head attention instead (below):
// the columns are up to 16 * kPrefixColTiles members of a sharer set, all
// with query head g = KV head g, walking a chunk of the set's prefix; each
// loaded tile meets every 16-column tile of them.
template <int QT, int CT, int D, int BS, bool SPLIT, bool PFX = false>
__global__ void __launch_bounds__(kDecodeThreads)
decode_mfma_kernel(DecodeArgs a) {
  using Ops = MfmaOps<QT>;
  using Tl = MfmaTile<CT, D>;
  constexpr bool F8 = CT == DT_FP8;
  constexpr int E = Elem<CT>::bytes;  // cache element bytes
  constexpr int KC = D / 32;          // logit MFMAs per tile
  constexpr int NT = D / 16;          // value n-tiles
  constexpr bool KW = F8 && D == 128; // K loaded as whole rows, then exchanged
  // 16-column tiles of the products (members, for prefix partials)
  constexpr int MCT = PFX ? kPrefixColTiles : 1;

  static_assert(!(PFX && SPLIT), "prefix partials run single-pass");
  const int g = blockIdx.x;
  const int Hq = a.num_heads, Hkv = a.num_kv_heads;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;

  // LDS: the merge of the 4 wavefronts; before the loop it holds the length
  // histogram of the longest-first order
  __shared__ float sm_o[kDecodeWaves][16 * MCT][D + 4];
  __shared__ float sm_m[kDecodeWaves][16 * MCT], sm_l[kDecodeWaves][16 * MCT];
  static_assert(sizeof(sm_o) >= kOrderScratchInts * sizeof(int), "order scratch");
  // prefix partials: set gi, its members mcol0 .. mcol0 + ncol - 1 as the
  // columns; the set's first member's table is walked over its prefix
  const int32_t *members = nullptr;
  int mcol0 = 0, ncol = G, ptok_set = 0;
  int s;
  int pchunk = 0;  // prefix partials: the chunk of the prefix walked
  if constexpr (PFX) {
    pchunk = blockIdx.y % a.n_pchunks;
    const int gm = blockIdx.y / a.n_pchunks;
    const int gi = gm / a.member_blocks, mb = gm % a.member_blocks;
    if (gi >= a.num_groups) return;  // the whole workgroup
    const int32_t *starts = a.plan + a.num_seqs;
    const int32_t *gtok = starts + a.num_groups + 1;
    members = gtok + a.num_groups;
    const int m0 = min(max(starts[gi], 0), a.num_members);
    const int m1 = min(max(starts[gi + 1], m0), a.num_members);
    mcol0 = m0 + mb * 16 * MCT;
    if (mcol0 >= m1) return;  // the whole workgroup
    ncol = min(16 * MCT, m1 - mcol0);
    s = min(max(members[m0], 0), a.num_seqs - 1);
    ptok_set = max(0, min(gtok[gi], a.max_blocks * BS));
  } else {
    s = SPLIT ? (int)blockIdx.y
              : longest_first_seq<kDecodeThreads>(a.context_lens, a.num_seqs,
                                                  a.max_blocks * BS, blockIdx.y,
                                                  reinterpret_cast<int *>(&sm_o[0][0][0]));
  }
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63, col = lane & 15, grp = lane >> 4;
  // split: this wave's partition (the split path has no workgroup barrier,
  // so a wave with nothing to do leaves at once)
  const int part = SPLIT ? (int)blockIdx.z * kDecodeWaves + w : 0;
  if (SPLIT && part >= a.num_parts) return;

  int L = PFX ? ptok_set : a.context_lens[s];
  L = max(0, min(L, a.max_blocks * BS));
  // shared-prefix decode: the prefix kernel computed tokens [0, ptok) in
  // n_pre chunks; the walk starts after them (ptok is a multiple of the
  // block size, so of the 16-token tile)
  int ptok = 0, n_pre = 0;
  if (!SPLIT && !PFX && a.seq_prefix) {
    ptok = max(0, min(a.seq_prefix[s], L)) & ~15;
    n_pre = min(a.n_pchunks, (ptok + a.pchunk_tokens - 1) / a.pchunk_tokens);
  }
  const int tok_begin = SPLIT ? part * a.part_tokens : PFX ? pchunk * a.pchunk_tokens : ptok;
  const int tok_end = SPLIT || PFX ? min(L, tok_begin + (SPLIT ? a.part_tokens : a.pchunk_tokens))
                                   : L;

  // the (sequence, query head) of column c: head g*G + c of sequence s, or
  // (prefix partials) head g of member mcol0 + c
  auto col_row = [&](int c) -> size_t {
    if constexpr (PFX)
      return (size_t)min(max(members[mcol0 + c], 0), a.num_seqs - 1) * Hq + g;
    else
      return (size_t)s * Hq + g * G + c;
  };
  // prefix partials: the partial of column c's (member, head) for this chunk
  auto pidx = [&](int c) -> size_t { return col_row(c) * a.n_pchunks + pchunk; };

  if (tok_begin >= tok_end && n_pre == 0) {
    if constexpr (PFX) {
      // an empty prefix: partials of weight 0
      for (int i = tid; i < ncol * D; i += kDecodeThreads) {
        const size_t pi = pidx(i / D);
        a.ws_o[pi * D + i % D] = 0.f;
        if (i % D == 0) {
          a.ws_m[pi] = -INFINITY;
          a.ws_l[pi] = 0.f;
        }
      }
    } else if (!SPLIT) {
      for (int i = tid; i < G * D; i += kDecodeThreads)
        store_elem<QT>(a.out, ((size_t)s * Hq + g * G) * D + i, 0.f);
    }
    return;
  }

  // Q^T operand: lane holds head `col` and the eight dims the K operand of
  // logit MFMA kk holds in this lane: (kk*4+grp)*8 for 16-bit caches,
  // 32*grp + 8*kk (D = 128) or 16*grp + 8*kk (D = 64) for 8-bit caches
  // (column tile ct: column col + 16 ct)
  u32x4 qop[MCT][KC];
#pragma unroll
  for (int ct = 0; ct < MCT; ++ct) {
    const int c = col + 16 * ct;
    const char *qp = static_cast<const char *>(a.q) + col_row(c < ncol ? c : 0) * D * 2;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      const int d0 = F8 ? (KW ? 32 : 16) * grp + 8 * kk : (kk * 4 + grp) * 8;
      qop[ct][kk] = c < ncol ? *reinterpret_cast<const u32x4 *>(qp + d0 * 2)
                             : u32x4{0u, 0u, 0u, 0u};
    }
  }

  const char *kc = static_cast<const char *>(a.k_cache);
  const char *vc = static_cast<const char *>(a.v_cache);
  const int32_t *trow = a.block_tables + (size_t)s * a.max_blocks;

  const int st_begin = tok_begin >> 4;
  const int st_end = (tok_end + 15) >> 4;
  const int n_tiles = st_end - st_begin;
  // the wave's tiles: tile0 + kStride * n for n < n_mine -- every tile of
  // its partition (split), or every fourth tile of the context
  constexpr int kStride = SPLIT ? 1 : kDecodeWaves;
  const int tile0 = SPLIT ? st_begin : st_begin + w;
  const int n_mine =
      SPLIT ? n_tiles : (n_tiles > w ? (n_tiles - w + kDecodeWaves - 1) / kDecodeWaves : 0);

  // lane offsets inside a tile, in bytes (chunk c adds KSTEP*c for K, 256*c
  // for V): K row `col` (8-bit, D = 128: row 8c + col%8), V token group `grp`
  const uint32_t koff = KW ? (uint32_t)((col % 8) * D + (2 * grp + col / 8) * 16)
                           : (uint32_t)(col * D * E + grp * 16);
  constexpr int KSTEP = KW ? 8 * D : 64;
  const uint32_t voff = (uint32_t)(grp * 4 * D * E + col * 16);

  // column col + 16 ct; l is this lane's share
  float m[MCT], l[MCT];
  f32x4 acc[MCT][NT];
#pragma unroll
  for (int ct = 0; ct < MCT; ++ct) {
    m[ct] = -INFINITY;
    l[ct] = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[ct][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // The wave's state to its LDS slice: head col's row sum (the four lanes'
  // shares added), maximum and weighted values; n-tile row m = 4*grp + i of
  // head col is dim 32u + 2m + j (n-tile 2u+j, 16-bit caches) or 64u + 4m + j
  // (n-tile 4u+j, 8-bit caches)
  auto stage_state = [&](int ct) {
    float lt = l[ct] + __shfl_xor(l[ct], 16);
    lt += __shfl_xor(lt, 32);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int mm = 4 * grp + i;
        const int d = F8 ? 64 * (nt / 4) + 4 * mm + nt % 4 : 32 * (nt / 2) + 2 * mm + nt % 2;
        sm_o[w][col + 16 * ct][d] = acc[ct][nt][i];
      }
    if (grp == 0) {
      sm_m[w][col + 16 * ct] = m[ct];
      sm_l[w][col + 16 * ct] = lt;
    }
  };



  // tiles are streamed (non-temporal loads); prefix partials read each tile
  // once per block of members, all on one XCD, so there the loads keep the
  // lines in its L2
  auto load = [&](Tl &t, size_t tile_bytes) {
    const char *kp = kc + tile_bytes + koff;
    const char *vp = vc + tile_bytes + voff;
#pragma unroll
    for (int c = 0; c < Tl::NC; ++c)
      t.k[c] = PFX ? load_keep16(kp + c * KSTEP) : load_stream16(kp + c * KSTEP);
#pragma unroll
    for (int c = 0; c < Tl::NC; ++c)
      t.v[c] = PFX ? load_keep16(vp + c * 256) : load_stream16(vp + c * 256);
  };

  auto compute = [&](Tl &t, int n) {
    // S^T[token 4*grp+i][column col + 16 ct]
    f32x4 sacc[MCT];
#pragma unroll
    for (int ct = 0; ct < MCT; ++ct) sacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (F8) {
      if constexpr (KW) {
        // lanes col >= 8 take chunk 2*grp of token col from load 1 (lane
        // col - 8); lanes col < 8 take chunk 2*grp+1 from load 0 (col + 8)
        const u32x4 a0 = t.k[0], a1 = t.k[1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          t.k[0][j] = from_other_half<0xC>(a0[j], a1[j]);
          t.k[1][j] = from_other_half<0x3>(a1[j], a0[j]);
        }
      }
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) {
        const uint32_t w0 = t.k[kk / 2][2 * (kk % 2)], w1 = t.k[kk / 2][2 * (kk % 2) + 1];
        const u32x4 kop = {fp8x2_to_16<QT>(w0, false), fp8x2_to_16<QT>(w0, true),
                           fp8x2_to_16<QT>(w1, false), fp8x2_to_16<QT>(w1, true)};
#pragma unroll
        for (int ct = 0; ct < MCT; ++ct) sacc[ct] = Ops::qk(kop, qop[ct][kk], sacc[ct]);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KC; ++kk)
#pragma unroll
        for (int ct = 0; ct < MCT; ++ct) sacc[ct] = Ops::qk(t.k[kk], qop[ct][kk], sacc[ct]);
    }

    const int t0 = (tile0 + kStride * n) * 16 + 4 * grp;
    const bool tail = (tile0 + kStride * n) * 16 + 16 > tok_end;
    const int nvalid = tail ? max(0, min(4, tok_end - t0)) : 4;
    float sc[MCT][4];
#pragma unroll
    for (int ct = 0; ct < MCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sc[ct][i] = (i < nvalid && col + 16 * ct < ncol) ? sacc[ct][i] * a.scale_log2 : -INFINITY;
    if (tail) {
      // masked tokens' values may hold anything (NaN included): zero them
      if constexpr (F8) {
        const uint32_t mk = nvalid >= 4 ? 0xffffffffu : ((1u << (8 * nvalid)) - 1u);
#pragma unroll
        for (int c = 0; c < Tl::NC; ++c) {
          t.v[c][0] &= mk;
          t.v[c][1] &= mk;
          t.v[c][2] &= mk;
          t.v[c][3] &= mk;
        }
      } else {
        const uint32_t m01 = nvalid >= 2 ? 0xffffffffu : (nvalid == 1 ? 0x0000ffffu : 0u);
        const uint32_t m23 = nvalid >= 4 ? 0xffffffffu : (nvalid == 3 ? 0x0000ffffu : 0u);
#pragma unroll
        for (int c = 0; c < Tl::NC; ++c) {
          t.v[c][0] &= m01;
          t.v[c][1] &= m23;
          t.v[c][2] &= m01;
          t.v[c][3] &= m23;
        }
      }
    }

#pragma unroll
    for (int ct = 0; ct < MCT; ++ct) {
      // running maximum of head `col`, shared by the 4 lanes holding it; only
      // moved (exactly, with the cross-lane max) when a logit exceeds it by
      // more than the slack somewhere in the wave
      const float mb = fmaxf(fmaxf(sc[ct][0], sc[ct][1]), fmaxf(sc[ct][2], sc[ct][3]));
      if (wave_any(mb > m[ct] + kRescaleSlack)) {
        float mh = fmaxf(mb, __shfl_xor(mb, 16));
        mh = fmaxf(mh, __shfl_xor(mh, 32));
        const float m_new = fmaxf(m[ct], mh);
        const float alpha = fast_exp2(m[ct] - (m_new == -INFINITY ? 0.f : m_new));
        l[ct] *= alpha;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[ct][nt] *= alpha;
        m[ct] = m_new;
      }
      const float m_use = m[ct] == -INFINITY ? 0.f : m[ct];
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sc[ct][i] - m_use);
      if constexpr (F8) {
        // values with 4 significant bits: one probability operand rounded to
        // the 16-bit type (8 or 11 bits) is ample, and the sum adds exactly
        // the rounded weights
        float r0, r1, r2, r3;
        const u32x2 pr = {Ops::round2(p[0], p[1], r0, r1), Ops::round2(p[2], p[3], r2, r3)};
        l[ct] += (r0 + r1) + (r2 + r3);
        // chunk u, word j: the four tokens of dim 64u + 4*col + j -> n-tile 4u+j
#pragma unroll
        for (int u = 0; u < Tl::NC; ++u) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const u32x2 va = {fp8x2_to_16<QT>(t.v[u][j], false), fp8x2_to_16<QT>(t.v[u][j], true)};
            acc[ct][4 * u + j] = Ops::pv(va, pr, acc[ct][4 * u + j]);
          }
        }
      } else if constexpr (PFX) {
        // prefix partials: one probability operand rounded to the 16-bit
        // type, the sum over exactly the rounded weights (the precision of
        // the chunked-prefill products); half the value products
        float r0, r1, r2, r3;
        const u32x2 pr = {Ops::round2(p[0], p[1], r0, r1), Ops::round2(p[2], p[3], r2, r3)};
        l[ct] += (r0 + r1) + (r2 + r3);
#pragma unroll
        for (int u = 0; u < Tl::NC; ++u) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const u32x2 va = {t.v[u][2 * j], t.v[u][2 * j + 1]};
            acc[ct][2 * u + j] = Ops::pv(va, pr, acc[ct][2 * u + j]);
          }
        }
      } else {
        l[ct] += (p[0] + p[1]) + (p[2] + p[3]);
        uint32_t h01, l01, h23, l23;
        Ops::split2(p[0], p[1], h01, l01);
        Ops::split2(p[2], p[3], h23, l23);
        const u32x2 phi = {h01, h23};
        const u32x2 plo = {l01, l23};
        // chunk u, words 2j..2j+1: the four tokens of dim 32u + 2*col + j
#pragma unroll
        for (int u = 0; u < Tl::NC; ++u) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const u32x2 va = {t.v[u][2 * j], t.v[u][2 * j + 1]};
            acc[ct][2 * u + j] = Ops::pv(va, phi, acc[ct][2 * u + j]);
            acc[ct][2 * u + j] = Ops::pv(va, plo, acc[ct][2 * u + j]);
          }
        }
      }
    }
  };

  // tiles in flight per wave while one is computed: three of the 2 KiB
  // tiles of 8-bit caches, two of the 4 KiB 16-bit tiles (measured: 8-bit
  // gqa70b 165 -> 154 us from one to three, 16-bit 278 -> 271 us from one
  // to two)
  if (n_mine > 0 && F8) {
    walk_tiles_n<Tl, 4, kStride>(trow, tile0, n_mine, BS / 16, (unsigned)a.num_blocks,
                        (size_t)g * BS * D * E, (size_t)Hkv * BS * D * E, (size_t)16 * D * E,
                        load, compute);
  } else if (n_mine > 0) {
    walk_tiles_n<Tl, 3, kStride>(trow, tile0, n_mine, BS / 16, (unsigned)a.num_blocks,
                        (size_t)g * BS * D * E, (size_t)Hkv * BS * D * E, (size_t)16 * D * E,
                        load, compute);
  }

  if constexpr (!PFX) stage_state(0);
  if constexpr (SPLIT) {
    // the wave's partial, row by row from its own LDS slice (written and
    // read by this wave only: ordering inside the wave is all it needs),
    // written through L2 (nothing in this kernel reads it); the partition
    // is not empty, so each real head's maximum is finite
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int idx = lane; idx < G * D; idx += 64) {
      const int hh = idx / D, d = idx % D;
      const size_t pi = ((size_t)s * Hq + g * G + hh) * a.num_parts + part;
      store_through(&a.ws_o[pi * D + d], sm_o[w][hh][d] * a.v_scale);
      if (d == 0) {
        store_through(&a.ws_m[pi], sm_m[w][hh]);
        store_through(&a.ws_l[pi], sm_l[w][hh]);
      }
    }
    return;
  }

  if constexpr (PFX) {
    // ---- merge the 4 wavefronts into each member's partial: maximum,
    //      sum of weights and un-normalised weighted values ----
#pragma unroll
    for (int ct = 0; ct < MCT; ++ct) stage_state(ct);
    __syncthreads();
    for (int idx = tid; idx < ncol * D; idx += kDecodeThreads) {
      const int hh = idx / D, d = idx % D;
      float M = -INFINITY;
#pragma unroll
      for (int i = 0; i < kDecodeWaves; ++i) M = fmaxf(M, sm_m[i][hh]);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int i = 0; i < kDecodeWaves; ++i) {
        const float f = fast_exp2(sm_m[i][hh] - M);  // a wave that saw no token: 0
        num = fmaf(f, sm_o[i][hh][d], num);
        den = fmaf(f, sm_l[i][hh], den);
      }
      const size_t pi = pidx(hh);
      a.ws_o[pi * D + d] = num;
      if (d == 0) {
        a.ws_m[pi] = M;
        a.ws_l[pi] = den;
      }
    }
    return;
  }

  // ---- merge the 4 wavefronts through LDS (and the prefix chunks'
  //      partial states, if any) ----
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kDecodeThreads) {
    const int hh = idx / D, d = idx % D;
    const size_t pbase = ((size_t)s * Hq + g * G + hh) * (size_t)a.n_pchunks;
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < kDecodeWaves; ++i) M = fmaxf(M, sm_m[i][hh]);
    for (int c = 0; c < n_pre; ++c) M = fmaxf(M, a.pws_m[pbase + c]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int i = 0; i < kDecodeWaves; ++i) {
      const float f = fast_exp2(sm_m[i][hh] - M);  // a wave that saw no token: m = -inf
      num = fmaf(f, sm_o[i][hh][d], num);
      den = fmaf(f, sm_l[i][hh], den);
    }
    for (int c = 0; c < n_pre; ++c) {
      const float f = fast_exp2(a.pws_m[pbase + c] - M);
      num = fmaf(f, a.pws_o[(pbase + c) * D + d], num);
      den = fmaf(f, a.pws_l[pbase + c], den);
    }
    const int h = g * G + hh;
    num *= a.v_scale;  // value dequantisation (1 for 16-bit caches)
    store_elem<QT>(a.out, ((size_t)s * Hq + h) * D + d, num / den);
  }
}

template <int QT, int CT, int D, int BS>
static hipError_t launch_mfma(const DecodeArgs &a, bool split, hipStream_t st) {
  if (split) {
    // one wavefront per partition, four partitions per workgroup
    const dim3 grid(a.num_kv_heads, a.num_seqs,
                    (a.num_parts + kDecodeWaves - 1) / kDecodeWaves);
    hipLaunchKernelGGL((decode_mfma_kernel<QT, CT, D, BS, true>), grid,
                       dim3(kDecodeThreads), 0, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((decode_mfma_kernel<QT, CT, D, BS, false>),
                     dim3(a.num_kv_heads, a.num_seqs, 1), dim3(kDecodeThreads), 0, st, a);
  return hipGetLastError();
}

template <int QT, int D, int BS>
static hipError_t launch_pfx(const DecodeArgs &a, hipStream_t st) {
  // x = head: all workgroups of one head have ids of one residue mod 8, so
  // they run on one XCD and re-read the head's prefix from its L2
  const dim3 grid(a.num_kv_heads, a.num_groups * a.member_blocks * a.n_pchunks, 1);
  hipLaunchKernelGGL((decode_mfma_kernel<QT, QT, D, BS, false, true>), grid,
                     dim3(kDecodeThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_prefix_mha(const DecodeArgs &a, int dtype, int head_dim, int block_size,
                             hipStream_t st) {
  if (a.num_groups == 0 || a.member_blocks == 0) return hipSuccess;
  if (dtype == DT_F16) {
    if (head_dim == 128)
      return block_size == 16 ? launch_pfx<DT_F16, 128, 16>(a, st)
                              : launch_pfx<DT_F16, 128, 32>(a, st);
    return block_size == 16 ? launch_pfx<DT_F16, 64, 16>(a, st)
                            : launch_pfx<DT_F16, 64, 32>(a, st);
  }
  if (head_dim == 128)
    return block_size == 16 ? launch_pfx<DT_BF16, 128, 16>(a, st)
                            : launch_pfx<DT_BF16, 128, 32>(a, st);
  return block_size == 16 ? launch_pfx<DT_BF16, 64, 16>(a, st)
                          : launch_pfx<DT_BF16, 64, 32>(a, st);
}

template <int QT, int CT>
static hipError_t launch_mfma_dt(const DecodeArgs &a, int head_dim,
                                 int block_size, bool split, hipStream_t st) {
  if (head_dim == 128)
    return block_size == 16 ? launch_mfma<QT, CT, 128, 16>(a, split, st)
                            : launch_mfma<QT, CT, 128, 32>(a, split, st);
  return block_size == 16 ? launch_mfma<QT, CT, 64, 16>(a, split, st)
                          : launch_mfma<QT, CT, 64, 32>(a, split, st);
}

hipError_t launch_decode_mfma(const DecodeArgs &a, int dtype, int cache_dtype,
                              int head_dim, int block_size, bool split,
                              hipStream_t st) {
  if (cache_dtype == DT_FP8) {
    if (dtype == DT_F16) return launch_mfma_dt<DT_F16, DT_FP8>(a, head_dim, block_size, split, st);
    return launch_mfma_dt<DT_BF16, DT_FP8>(a, head_dim, block_size, split, st);
  }
  if (dtype == DT_F16) return launch_mfma_dt<DT_F16, DT_F16>(a, head_dim, block_size, split, st);
  return launch_mfma_dt<DT_BF16, DT_BF16>(a, head_dim, block_size, split, st);
}

}  // namespace pkv
