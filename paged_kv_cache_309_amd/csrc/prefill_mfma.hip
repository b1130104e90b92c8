// prefill_mfma.hip - multi-query paged attention for chunked prefill on the
// matrix cores (fp16 / bf16).
//
// A long prompt is processed in chunks that share iterations with ongoing
// decodes ("Inside vLLM: How PagedAttention Eliminates KV-Cache Memory
// Waste", section "Continuous Batching and Chunked Prefill").  A chunk's
// keys and values are written into the sequence's blocks first, like a
// decode token's; then every chunk token attends, through the block table,
// to the context before it and to the chunk up to and including itself.
// Per query token this is the decode computation over a shorter prefix
// ("PagedAttention: how vLLM manages the KV cache", section "PagedAttention
// changes addressing inside attention"); the chunk turns it into dense
// products, so it runs on the matrix cores.
//
// The query rows of one (sequence, KV head) are the chunk's tokens times the
// G query heads of the group, row r = token (r / G), head (r % G).  A
// wavefront owns NQ tiles of 16 rows and walks every 16-token K/V tile its
// rows can see, in order; per tile and row tile it issues D/32
// v_mfma_f32_16x16x32 for S^T = K . Q^T and D/16 v_mfma_f32_16x16x16 for
// O^T += V^T . P^T, with the lane layouts of the decode kernel (the logits
// come out where the value product wants its B operand).  The K/V operands
// of a tile are loaded once per wavefront and used by all its row tiles.
// Tiles entirely before the wave's first query token need no mask; the
// others mask every logit whose token lies after the row's own position.
//
// Probabilities enter the value product rounded once to the 16-bit type of
// q (nearest even), and the running sum adds the same rounded values, so
// the normalisation matches the weights actually applied.
#include "mfma_ops.h"

namespace pkv {

constexpr int kPrefillThreads = 256;
constexpr int kPrefillWaves = 4;
constexpr int kPrefillNQ = 2;  // 16-row query tiles per wavefront
constexpr int kPrefillRows = kPrefillWaves * kPrefillNQ * 16;

int prefill_rows_per_workgroup() { return kPrefillRows; }

template <int QT, int D, int BS>
__global__ void __launch_bounds__(kPrefillThreads)
prefill_mfma_kernel(PrefillArgs a) {
  using Ops = MfmaOps<QT>;
  using Tl = MfmaTile<QT, D>;
  constexpr int E = 2;        // cache element bytes
  constexpr int KC = D / 32;  // logit MFMAs per tile and row tile
  constexpr int NT = D / 16;  // value n-tiles
  constexpr int NQ = kPrefillNQ;

  const int g = blockIdx.x, s = blockIdx.y;
  const int blk = a.q_blocks - 1 - (int)blockIdx.z;  // latest rows (longest prefixes) first
  const int Hq = a.num_heads, Hkv = a.num_kv_heads;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, col = lane & 15, grp = lane >> 4;

  const int T = a.num_query_tokens;
  const int q0 = min(max(a.query_start_loc[s], 0), T);
  const int q1 = min(max(a.query_start_loc[s + 1], q0), T);
  const int C = q1 - q0;
  const int L = max(0, min(a.context_lens[s], a.max_blocks * BS));
  const int R = C * G;
  const int row0 = blk * kPrefillRows + w * NQ * 16;
  if (row0 >= R) return;
  const int row_last = min(row0 + NQ * 16, R) - 1;
  const int pos_first = L - C + row0 / G;  // rows ascend with positions
  const int pos_last = L - C + row_last / G;
  const int kv_end = min(L, pos_last + 1);
  const int n_tiles = kv_end > 0 ? (kv_end + 15) >> 4 : 0;
  const int k_full = pos_first >= 0 ? (pos_first + 1) >> 4 : 0;  // tiles visible to every row

  // this lane's row of each row tile: its position (-1: no row) and its
  // Q^T operand (dims (kk*4 + grp)*8 .. +7 for logit MFMA kk)
  int pos[NQ];
  size_t orow[NQ];
  u32x4 qop[NQ][KC];
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    const int r = row0 + qt * 16 + col;
    const bool valid = r <= row_last;
    const int j = valid ? r / G : 0, hh = valid ? r % G : 0;
    pos[qt] = valid ? L - C + j : -1;
    orow[qt] = ((size_t)(q0 + j) * Hq + g * G + hh) * D;
    const char *qp = static_cast<const char *>(a.q) + orow[qt] * 2;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk)
      qop[qt][kk] = valid ? *reinterpret_cast<const u32x4 *>(qp + (kk * 4 + grp) * 16)
                          : u32x4{0u, 0u, 0u, 0u};
  }

  const char *kc = static_cast<const char *>(a.k_cache);
  const char *vc = static_cast<const char *>(a.v_cache);
  const int32_t *trow = a.block_tables + (size_t)s * a.max_blocks;
  const uint32_t koff = (uint32_t)(col * D * E + grp * 16);
  const uint32_t voff = (uint32_t)(grp * 4 * D * E + col * 16);

  float m[NQ], l[NQ];
  f32x4 acc[NQ][NT];
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    m[qt] = -INFINITY;
    l[qt] = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[qt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // K/V tiles are read by every row block of the sequence: ordinary
  // (cached) loads
  auto load = [&](Tl &t, size_t tile_bytes) {
    const char *kp = kc + tile_bytes + koff;
    const char *vp = vc + tile_bytes + voff;
#pragma unroll
    for (int c = 0; c < Tl::NC; ++c) t.k[c] = *reinterpret_cast<const u32x4 *>(kp + c * 64);
#pragma unroll
    for (int c = 0; c < Tl::NC; ++c) t.v[c] = *reinterpret_cast<const u32x4 *>(vp + c * 256);
  };

  auto compute = [&](Tl &t, int k) {
    const int t0 = k * 16 + 4 * grp;  // this lane's first token of the tile
    if (k * 16 + 16 > L) {
      // tokens at or past L may hold anything (NaN included): zero their values
      const int nvalid = max(0, min(4, L - t0));
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
    const bool masked = k >= k_full;
#pragma unroll
    for (int qt = 0; qt < NQ; ++qt) {
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) sacc = Ops::qk(t.k[kk], qop[qt][kk], sacc);
      float sc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[i] = sacc[i] * a.scale_log2;
        if (masked && t0 + i > pos[qt]) sc[i] = -INFINITY;
      }
      const float mb = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      if (wave_any(mb > m[qt] + kRescaleSlack)) {
        float mh = fmaxf(mb, __shfl_xor(mb, 16));
        mh = fmaxf(mh, __shfl_xor(mh, 32));
        const float m_new = fmaxf(m[qt], mh);
        const float alpha = fast_exp2(m[qt] - (m_new == -INFINITY ? 0.f : m_new));
        l[qt] *= alpha;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[qt][nt] *= alpha;
        m[qt] = m_new;
      }
      const float m_use = m[qt] == -INFINITY ? 0.f : m[qt];
      float r0, r1, r2, r3;
      const uint32_t p01 = Ops::round2(fast_exp2(sc[0] - m_use), fast_exp2(sc[1] - m_use), r0, r1);
      const uint32_t p23 = Ops::round2(fast_exp2(sc[2] - m_use), fast_exp2(sc[3] - m_use), r2, r3);
      l[qt] += (r0 + r1) + (r2 + r3);
      const u32x2 pb = {p01, p23};
      // chunk u, words 2j..2j+1: the four tokens of dim 32u + 2*col + j
#pragma unroll
      for (int u = 0; u < Tl::NC; ++u) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const u32x2 va = {t.v[u][2 * j], t.v[u][2 * j + 1]};
          acc[qt][2 * u + j] = Ops::pv(va, pb, acc[qt][2 * u + j]);
        }
      }
    }
  };

  if (n_tiles > 0)
    walk_tiles<Tl, 1>(trow, 0, n_tiles, BS / 16, (unsigned)a.num_blocks, (size_t)g * BS * D * E,
                      (size_t)Hkv * BS * D * E, (size_t)16 * D * E, load, compute);

  // normalise and store: n-tile 2u+j, row m = 4*grp + i is dim 32u + 2m + j
  // of the lane's query row, so the two n-tiles of a chunk give two
  // adjacent dims, stored as one 32-bit word
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    float lt = l[qt] + __shfl_xor(l[qt], 16);
    lt += __shfl_xor(lt, 32);
    if (row0 + qt * 16 + col > row_last) continue;  // no row in this column
    const float inv = lt > 0.f ? a.v_scale / lt : 0.f;
    uint32_t *op = reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(a.out) + orow[qt]);
#pragma unroll
    for (int u = 0; u < Tl::NC; ++u) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * u + 2 * (4 * grp + i);
        op[d >> 1] = from_f32<QT>(acc[qt][2 * u][i] * inv) |
                     (from_f32<QT>(acc[qt][2 * u + 1][i] * inv) << 16);
      }
    }
  }
}

template <int QT, int D, int BS>
static hipError_t launch_prefill(const PrefillArgs &a, hipStream_t st) {
  const dim3 grid(a.num_kv_heads, a.num_seqs, a.q_blocks);
  hipLaunchKernelGGL((prefill_mfma_kernel<QT, D, BS>), grid, dim3(kPrefillThreads), 0, st, a);
  return hipGetLastError();
}

template <int QT>
static hipError_t launch_prefill_dt(const PrefillArgs &a, int head_dim, int block_size,
                                    hipStream_t st) {
  if (head_dim == 128)
    return block_size == 16 ? launch_prefill<QT, 128, 16>(a, st)
                            : launch_prefill<QT, 128, 32>(a, st);
  return block_size == 16 ? launch_prefill<QT, 64, 16>(a, st) : launch_prefill<QT, 64, 32>(a, st);
}

hipError_t launch_prefill_mfma(const PrefillArgs &a, int dtype, int cache_dtype, int head_dim,
                               int block_size, int max_query_len, hipStream_t st) {
  (void)cache_dtype;
  (void)max_query_len;
  if (a.num_seqs == 0 || a.q_blocks == 0) return hipSuccess;
  if (dtype == DT_F16) return launch_prefill_dt<DT_F16>(a, head_dim, block_size, st);
  return launch_prefill_dt<DT_BF16>(a, head_dim, block_size, st);
}

}  // namespace pkv
