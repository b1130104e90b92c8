// prefill_mfma.hip - multi-query paged attention for chunked prefill on the
// matrix cores (fp16 / bf16 queries; caches of the query's type or E4M3).
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
// Work: the query rows of one (sequence, KV head) are the chunk's tokens
// times the G query heads of the group, row r = token (r / G), head (r % G).
// A workgroup (4 wavefronts) takes 128 consecutive rows, each wavefront 32
// of them (two row tiles of 16; with 64 rows per wavefront the registers
// allow one wavefront per SIMD only, which measured slower).  The workgroup walks the K/V of the
// sequence in 32-token super-tiles through the block table: the four
// wavefronts copy a super-tile (two 16-token tiles of K and of V) from HBM
// into a ring of LDS stages with direct global-to-LDS loads, three
// super-tiles ahead of the one being computed, and every wavefront takes
// its matrix-core operands from there.  Per super-tile and row tile a wavefront issues 2 x D/32
// v_mfma_f32_16x16x32 for S^T = K . Q^T (one per 16-token tile and 32 dims)
// and D/16 v_mfma_f32_16x16x32 for O^T += V^T . P^T contracting over all 32
// tokens.  Only tiles that reach past a wavefront's first query token are
// masked (logits of tokens after the row's own position set to -inf).
//
// Lane layouts: S^T of one 16-token tile comes out as lane l holding tokens
// 4*(l/16)+i of row l%16.  The value product's contraction index k (32
// tokens) is ordered so that lane l's eight B-operand slots k = 8*(l/16)+e
// are those tokens of the first tile (e < 4) and of the second (e >= 4):
// the probabilities stay in the lanes that computed them.  Its A operand
// (V^T: dim rows, token columns) then needs, per lane, four consecutive
// tokens of one dim from each tile, which the token-grouped V layout stores
// as 8 contiguous bytes.  N-tile 2u + j takes dims 32u + 16j + m (m = 0 ..
// 15), so the 16 lanes of one token group read 16 consecutive 8-byte words
// (every LDS bank once; dims 32u + 2m + j, two n-tiles per 16 bytes, left
// every other bank idle and doubled the value reads' time), and each lane's
// four output rows are four adjacent dims.  K rows are stored with their
// 16-byte chunks permuted (see PrefillRing) so that lanes reading different
// token rows use different banks.
//
// Scheduling: workgroup i runs on XCD i % 8, and on each XCD consecutive
// workgroups go to its four shader engines in turn, in grid order; a
// workgroup waits for a slot on its own shader engine, and the ones after
// it wait too.  All row blocks of one (sequence, KV head) belong to one XCD
// and are numbered consecutively, latest rows (longest prefixes) first, so
// the sequence's K/V stay in that XCD's L2 while its row blocks run; each
// window of four is rotated so that no shader engine gets the longest row
// blocks throughout.  A grid of at most 256 row blocks per XCD runs them
// longest walk first instead (ties in that order): with two or three row
// blocks per workgroup slot, a long one that starts late sets the end of
// the launch.
//
// 8-bit caches: the ring holds the 1-byte codes (half the bytes per stage).
// A 16-byte K read gives 16 dims of one token, widened exactly to the
// 16-bit type of q with one packed conversion per pair of codes, and feeds
// two logit products; q is loaded in the matching dimension order.  For V,
// one 16-byte read per tile gives the four tokens of four consecutive dims,
// so n-tile 4u + j takes dim 64u + 4m + j.  The key scale is folded into the
// logit scale, the value scale into the final normalisation.
//
// Probabilities enter the value product rounded to the 16-bit type of q
// (nearest even, one packed conversion per pair).  The running sum of each
// row comes out of one more 16x16x32 product with an A operand of ones, so
// it adds exactly the rounded weights the value product applied, and the
// softmax stays off the vector ALUs as far as possible: per logit one fused
// multiply-add and one exp2, plus the running maximum.  Accumulation is fp32.
#include <limits.h>

#include <type_traits>

#include "mfma_ops.h"

namespace pkv {

constexpr int kPrefillThreads = 256;
constexpr int kPrefillWaves = 4;
constexpr int kPrefillNQ = 2;  // 16-row query tiles per wavefront
constexpr int kPrefillRows = kPrefillWaves * kPrefillNQ * 16;
constexpr int kXcds = 8;
// Above this many row blocks per XCD the grid keeps its plain (rotated)
// order: the longest-first order costs every workgroup a select over all of
// its XCD's row blocks (about 2 us), and with many row blocks per slot the
// tail it saves is a small part of the launch.  Below it, longest first
// also covers a long sequence that the plain order would start last.
// Measured, 160 per XCD (13B-class prefill, 8 chunks of 512 tokens x 40
// heads): plain order unrotated 99.9 us, rotated 89.1, longest first 90.5;
// over E4M3 caches 98.2 / 87.5 / 84.5 us.  512 per XCD (70B-class): 530 us
// unrotated, 550 with longest first (a select over two row blocks per
// thread), 525 with a longest-first order precomputed on the host.
constexpr int kPrefillOrderMaxUnits = 256;

int prefill_rows_per_workgroup() { return kPrefillRows; }

int64_t prefill_grid(int num_seqs, int num_kv_heads, int q_blocks) {
  const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
  return (int64_t)kXcds * ((pairs + kXcds - 1) / kXcds) * q_blocks;
}

// LDS ring of super-tiles.  One super-tile is four 16-token pieces: K of
// tile 0, K of tile 1, V of tile 0, V of tile 1, each 16 * D * E bytes (E:
// cache element bytes) and each filled by one wavefront with direct
// global-to-LDS loads (64 lanes x 16 bytes per instruction, lane i writing
// bytes 16i .. 16i+15 of its 1 KiB block).  V pieces keep the HBM layout.
// K pieces are stored with the 16-byte chunks of each token row permuted:
// physical chunk p of row r holds logical chunk p ^ key(r), so that the 16
// lanes reading the same logical chunk of 16 different rows (one pass of a
// 16-byte LDS read) hit 16 different 16-byte bank groups of the 256-byte
// bank line.  key(r) = (r / RPL) % CR, with CR chunks per row and RPL rows
// per bank line.  The permutation is applied through the global address
// each lane loads from.
template <int CT, int D>
struct PrefillRing {
  static constexpr int ROWB = D * Elem<CT>::bytes;  // bytes per K row
  static constexpr int PIECE = 16 * ROWB;
  static constexpr int TILE = 4 * PIECE;
  static constexpr int STAGES = 4;
  static constexpr int CR = ROWB / 16;  // 16-byte chunks per K row
  static constexpr int RPL = ROWB >= 256 ? 1 : 256 / ROWB;
  static constexpr int LOADS = PIECE / 1024;  // per wavefront and super-tile
  __device__ static __forceinline__ int key(int r) { return (r / RPL) % CR; }
  // V pieces of 16-bit caches: the 16-byte chunks (two dims of one token
  // group) of odd token groups trade places with the chunk 128 bytes away,
  // so the two token groups of one 32-lane pass of 8-byte reads (lanes
  // reading 16 consecutive dims each) fill all 64 banks.  Byte offset of
  // dim d of token group g inside the piece.
  __device__ static __forceinline__ int voff(int g, int d) {
    return g * D * 8 + (((d >> 1) ^ ((g & 1) << 3)) << 4) + (d & 1) * 8;
  }
};

__device__ __forceinline__ u32x4 lds16(const char *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

// One direct global-to-LDS load: 16 bytes per lane from `src`, written to
// lds_base + 16 * lane.  The builtin only exists for the device; the host
// pass of this single-source file sees an empty body.
__device__ __forceinline__ void load_lds16(const char *src, char *lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
#else
  (void)src;
  (void)lds_base;
#endif
}

// Wait until at most n of this wavefront's vector-memory operations are
// outstanding (n < 16; expcnt and lgkmcnt not waited for).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(N | (7 << 4) | (15 << 8));
}

// QT: element type of q and out (16-bit); CT: of the caches (QT or E4M3).
// PREFIX: the shared-prefix partials instead of chunked prefill (below).
// ORDER (prefill): the row blocks of each XCD in longest-first order (below).
template <int QT, int CT, int D, int BS, bool PREFIX = false, bool ORDER = false>
__global__ void __launch_bounds__(kPrefillThreads)
prefill_mfma_kernel(PrefillArgs a) {
  using Ops = MfmaOps<QT>;
  using RG = PrefillRing<CT, D>;
  constexpr bool F8 = CT == DT_FP8;
  constexpr int E = Elem<CT>::bytes;
  constexpr int KC = D / 32;   // logit MFMAs per 16-token tile and row tile
  constexpr int NC = D / 32;   // 16-byte V reads per lane and tile (16-bit)
  constexpr int NT = D / 16;   // value n-tiles
  constexpr int V8 = D / 64;   // 16-byte V reads per lane and tile (8-bit)
  constexpr int NQ = kPrefillNQ;
  constexpr int S = RG::STAGES;
  __shared__ __attribute__((aligned(1024))) char ring[S * RG::TILE];

  const int Hkv = a.num_kv_heads, Hq = a.num_heads;
  const int G = Hq / Hkv;
  const int xcd = blockIdx.x % kXcds;
  int nth = blockIdx.x / kXcds;
  if constexpr (ORDER) {
    // Longest-first order of this XCD's row blocks.  The dispatcher starts
    // workgroups in grid order, and a row block's walk ranges from a few
    // super-tiles to the whole context; a long one that starts late
    // stretches the end of the launch.  Rank nth of the XCD therefore takes
    // the XCD-local row block of rank nth in an order of decreasing walk
    // (ties in grid order): a counting select over the walks in super-tiles,
    // 256 buckets of width 2^sh, one row block per thread, each walk
    // computed as below.  Neighbouring ranks have similar walks, so the
    // order also spreads the work evenly over the shader engines (below).
    static_assert(!PREFIX, "prefill only");
    static_assert(kPrefillOrderMaxUnits <= kPrefillThreads, "one row block per thread");
    static_assert(sizeof(ring) >= kOrderScratchInts * sizeof(int), "order scratch");
    const int units = gridDim.x / kXcds;  // <= kPrefillOrderMaxUnits (the host checks)
    const int max_tok = a.max_blocks * BS;
    const int max_work = (max_tok + 31) >> 5;
    int sh = 0;
    while ((max_work >> sh) >= kOrderBuckets) ++sh;
    // row block j = threadIdx.x (its three loads issued at once)
    const int j = threadIdx.x;
    const int pr = (j / a.q_blocks) * kXcds + xcd;
    const int sq = min(pr / Hkv, a.num_seqs - 1);
    const int T = a.num_query_tokens;
    const int c0 = min(max(a.query_start_loc[sq], 0), T);
    const int c1 = min(max(a.query_start_loc[sq + 1], c0), T);
    const int Cs = c1 - c0, Ls = max(0, min(a.context_lens[sq], max_tok));
    const int r0 = (a.q_blocks - 1 - j % a.q_blocks) * kPrefillRows;
    int work = 0;
    if (j < units && pr < a.num_seqs * Hkv && r0 < Cs * G) {
      const int kv_end = min(Ls, Ls - Cs + (min(r0 + kPrefillRows, Cs * G) - 1) / G + 1);
      work = kv_end > 0 ? (kv_end + 31) >> 5 : 0;
    }
    const int my_bucket = (max_work - work) >> sh;
    // with units <= threads, item i of both passes is thread i's
    nth = counting_select<kPrefillThreads>(
        units, nth, [&](int) { return my_bucket; }, reinterpret_cast<int *>(ring));
  }
  if constexpr (!ORDER && !PREFIX) {
    // The dispatcher also fixes each workgroup's shader engine: on every
    // XCD, consecutive workgroups go to its four shader engines in turn.
    // With a pair's row blocks consecutive and longest first, position
    // nth % 4 would always take the same one of four neighbouring row
    // blocks (for four row blocks per pair, always the same row block), so
    // one shader engine would get the longest walks throughout.  Rotating
    // each window of four positions by the window's index gives every shader
    // engine each of the four in turn; a pair's row blocks stay together.
    const int wi = nth >> 2;
    if ((wi << 2) + 4 <= (int)(gridDim.x / kXcds)) nth = (wi << 2) | ((nth + wi) & 3);
  }
  const int pair = (nth / a.q_blocks) * kXcds + xcd;
  const int blk = a.q_blocks - 1 - nth % a.q_blocks;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, col = lane & 15, grp = lane >> 4;

  // The walk covers tokens kv0 .. kv0 + L - 1 of sequence s's block table
  // (token offsets inside the walk are relative to kv0); n_super super-tiles
  // for the workgroup, n_super_w of them computed by this wavefront, whose
  // rows are row0 .. row_last.
  int s, g, L, kv0 = 0, n_super, n_super_w, row0, row_last, pos_first;
  int pos[NQ];
  size_t orow[NQ];   // q row (and, prefill, out row) of each row tile
  size_t pidx[NQ];   // prefix mode: the partial of each row tile
  // prefix mode: rows of one (set, KV head, chunk) are the set's members
  // times the G query heads of the group, row r = member r / G, head r % G;
  // they all attend to every token of the chunk, which the set's first
  // member's table maps (all members map the same blocks there)
  const int32_t *members = nullptr;
  int m0 = 0, chunk = 0;
  if constexpr (PREFIX) {
    if (pair >= a.num_groups * Hkv * a.n_chunks) return;  // the whole workgroup
    chunk = pair % a.n_chunks;
    g = (pair / a.n_chunks) % Hkv;
    const int gi = pair / a.n_chunks / Hkv;
    const int32_t *starts = a.plan + a.num_seqs;
    const int32_t *gtok = starts + a.num_groups + 1;
    members = gtok + a.num_groups;
    m0 = min(max(starts[gi], 0), a.num_members);
    const int m1 = min(max(starts[gi + 1], m0), a.num_members);
    const int R = (m1 - m0) * G;
    const int wg_row0 = blk * kPrefillRows;
    if (wg_row0 >= R) return;  // the whole workgroup
    s = min(max(members[m0], 0), a.num_seqs - 1);
    // the set's prefix lies inside every member's context (the planner
    // guarantees it), and inside the table whatever the plan holds
    const int ptok = max(0, min(gtok[gi], a.max_blocks * BS));
    kv0 = chunk * a.chunk_tokens;
    if (kv0 >= ptok) return;  // the whole workgroup
    L = min(a.chunk_tokens, ptok - kv0);
    n_super = (L + 31) >> 5;
    const int wg_row_last = min(wg_row0 + kPrefillRows, R) - 1;
    row0 = wg_row0 + w * NQ * 16;
    row_last = min(row0 + NQ * 16 - 1, wg_row_last);
    n_super_w = row0 <= wg_row_last ? n_super : 0;
    pos_first = INT_MAX;  // no causal mask
  } else {
    if (pair >= a.num_seqs * Hkv) return;  // the whole workgroup
    s = pair / Hkv;
    g = pair % Hkv;
  }
  const int T = a.num_query_tokens;
  const int q0 = PREFIX ? 0 : min(max(a.query_start_loc[s], 0), T);
  const int q1 = PREFIX ? 0 : min(max(a.query_start_loc[s + 1], q0), T);
  const int C = q1 - q0;
  if constexpr (!PREFIX) {
    L = max(0, min(a.context_lens[s], a.max_blocks * BS));
    const int R = C * G;
    const int wg_row0 = blk * kPrefillRows;
    if (wg_row0 >= R) return;  // the whole workgroup
    const int wg_row_last = min(wg_row0 + kPrefillRows, R) - 1;
    const int wg_kv_end = min(L, L - C + wg_row_last / G + 1);
    n_super = wg_kv_end > 0 ? (wg_kv_end + 31) >> 5 : 0;

    // this wavefront's rows
    row0 = wg_row0 + w * NQ * 16;
    const bool has_rows = row0 <= wg_row_last;
    row_last = min(row0 + NQ * 16 - 1, wg_row_last);
    pos_first = L - C + row0 / G;  // rows ascend with positions
    const int kv_end_w = has_rows ? min(L, L - C + row_last / G + 1) : 0;
    n_super_w = kv_end_w > 0 ? (kv_end_w + 31) >> 5 : 0;
  }

  u32x4 qop[NQ][KC];
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    const int r = row0 + qt * 16 + col;
    const bool valid = r <= row_last;
    const int j = valid ? r / G : 0, hh = valid ? r % G : 0;
    if constexpr (PREFIX) {
      const int sq = valid ? min(max(members[m0 + j], 0), a.num_seqs - 1) : 0;
      pos[qt] = valid ? INT_MAX : -1;
      orow[qt] = ((size_t)sq * Hq + g * G + hh) * D;
      pidx[qt] = ((size_t)sq * Hq + g * G + hh) * a.n_chunks + chunk;
    } else {
      pos[qt] = valid ? L - C + j : -1;
      orow[qt] = ((size_t)(q0 + j) * Hq + g * G + hh) * D;
      pidx[qt] = 0;
    }
  }
  // the eight dims logit product kk takes from this lane: chunk kk*4+grp of
  // the row (16-bit caches); half kk%2 of the 16 dims of 8-bit chunk
  // (kk/2)*4+grp
  auto load_q = [&]() {
#pragma unroll
    for (int qt = 0; qt < NQ; ++qt) {
      const bool valid = row0 + qt * 16 + col <= row_last;
      const char *qp = static_cast<const char *>(a.q) + orow[qt] * 2;
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) {
        const int off = F8 ? 32 * ((kk / 2) * 4 + grp) + 16 * (kk % 2) : (kk * 4 + grp) * 16;
        qop[qt][kk] =
            valid ? *reinterpret_cast<const u32x4 *>(qp + off) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  if constexpr (!PREFIX) {
    load_q();
    // the queries are in registers before the ring's loads are counted
    wait_vm<0>();
  }

  // block-table entries are wave-uniform: read through the scalar cache
  const __attribute__((address_space(4))) int32_t *trow =
      (const __attribute__((address_space(4))) int32_t *)(a.block_tables +
                                                          (size_t)s * a.max_blocks);
  const size_t block_bytes = (size_t)Hkv * BS * D * E;
  const char *src_base = static_cast<const char *>(w < 2 ? a.k_cache : a.v_cache) +
                         (size_t)g * BS * D * E;
  // this lane's source offset inside the piece, per 1 KiB block b
  uint32_t lane_off[RG::LOADS];
#pragma unroll
  for (int b = 0; b < RG::LOADS; ++b) {
    if (w < 2) {
      const int rows_per_kib = 1024 / RG::ROWB;
      const int r = b * rows_per_kib + lane / RG::CR, p = lane % RG::CR;
      lane_off[b] = (uint32_t)(r * RG::ROWB + ((p ^ RG::key(r)) * 16));
    } else if constexpr (F8) {
      lane_off[b] = (uint32_t)(b * 1024 + lane * 16);
    } else {
      // LDS chunk c = 64b + lane is chunk cg = c % (D/2) of token group
      // g = c / (D/2); by voff it holds that group's dims 2(cg ^ x) and
      // 2(cg ^ x) + 1, x = 8 (g odd) or 0, which sit 16 (cg ^ x) bytes into
      // the group in the cache's layout
      const int c = b * 64 + lane, g = c / (D / 2), cg = c % (D / 2);
      lane_off[b] = (uint32_t)(g * D * 8 + ((cg ^ ((g & 1) << 3)) << 4));
    }
  }
  // physical block of this wavefront's piece of super-tile n (a tile past
  // the context: any block, its contents are masked)
  auto lookup = [&](int n) -> int {
    const unsigned tb = 32u * n + 16u * (w & 1);
    const int phys = tb < (unsigned)L ? trow[(kv0 + tb) / BS] : 0;
    return (unsigned)phys < (unsigned)a.num_blocks ? phys : 0;
  };
  // wavefront w fills piece w of super-tile n into stage n % S
  auto issue = [&](int n, int phys, int stage) {
    const unsigned tb = 32u * n + 16u * (w & 1);
    // phys is in [0, num_blocks) and a block is far below 4 GiB: an unsigned
    // 32 x 32 -> 64-bit product
    const char *src = src_base + (uint64_t)(unsigned)phys * (unsigned)block_bytes +
                      ((kv0 + tb) % BS) * D * E;
    char *dst = ring + stage * RG::TILE + w * RG::PIECE;
#pragma unroll
    for (int b = 0; b < RG::LOADS; ++b)
      load_lds16(src + lane_off[b], dst + b * 1024);
  };

  float m[NQ];
  f32x4 acc[NQ][NT], lsum[NQ];
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    m[qt] = -INFINITY;
    lsum[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[qt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float c2 = a.scale_log2;  // > 0
  const uint32_t one2 = Ops::pack2(1.f, 1.f);
  const u32x4 ones = {one2, one2, one2, one2};

  // Key rows of tokens at or past L may hold anything, NaN included (stale
  // blocks, or the stand-in block 0 of a tile past the context).  This
  // lane's key operands are token row `col` of each tile: they are zeroed
  // bitwise before any float operation sees them, so every value that
  // reaches the logit products and the maxima is finite or -inf (the file
  // is compiled without NaN semantics, which holds by this construction for
  // finite q, K and V of the attended tokens).
  auto zero_tail_keys = [&](auto &kw, int n) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if (32 * n + 16 * st + col >= L) {
#pragma unroll
        for (int i = 0; i < (int)(sizeof(kw[st]) / sizeof(kw[st][0])); ++i)
          kw[st][i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  // stage = n % S; MAY_TAIL: the super-tile may reach past L
  auto compute = [&](int n, int stage, auto may_tail) {
    constexpr bool MAY_TAIL = decltype(may_tail)::value;
    const char *base = ring + stage * RG::TILE;
    const bool diag = !PREFIX && 32 * n + 31 > pos_first;
    // K operands of both tiles first: the logit products wait only for them,
    // and the value reads complete while those products run
    u32x4 kop[2][KC];
    u32x4 va[NT];
    u32x4 vraw[F8 ? V8 : 1][2];
    if constexpr (F8) {
      u32x4 kraw[2][KC / 2];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int k2 = 0; k2 < KC / 2; ++k2) {
          const int c = k2 * 4 + grp;
          kraw[st][k2] = lds16(base + st * RG::PIECE + col * RG::ROWB + ((c ^ RG::key(col)) * 16));
        }
      // four tokens of dims 64u + 4*col .. +3, tile 0 and tile 1
#pragma unroll
      for (int u = 0; u < V8; ++u) {
        const char *v0 = base + 2 * RG::PIECE + (grp * D + 64 * u + 4 * col) * 4;
        vraw[u][0] = lds16(v0);
        vraw[u][1] = lds16(v0 + RG::PIECE);
      }
      if (MAY_TAIL && 32 * n + 32 > L) zero_tail_keys(kraw, n);
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int k2 = 0; k2 < KC / 2; ++k2)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t w0 = kraw[st][k2][2 * h], w1 = kraw[st][k2][2 * h + 1];
            kop[st][2 * k2 + h] = u32x4{fp8x2_to_16<QT>(w0, false), fp8x2_to_16<QT>(w0, true),
                                        fp8x2_to_16<QT>(w1, false), fp8x2_to_16<QT>(w1, true)};
          }
    } else {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
          const int c = kk * 4 + grp;
          kop[st][kk] = lds16(base + st * RG::PIECE + col * RG::ROWB + ((c ^ RG::key(col)) * 16));
        }
      if (MAY_TAIL && 32 * n + 32 > L) zero_tail_keys(kop, n);
      // value operand of n-tile 2u+j: dim 32u + 16j + col, four tokens of
      // tile 0 then the same four of tile 1 (8 bytes each, one piece apart,
      // so one two-address LDS read fills the operand's registers in place;
      // the 16 lanes of a token group read 128 consecutive bytes, and the
      // two groups of a 32-lane pass different halves of the banks)
#pragma unroll
      for (int u = 0; u < NC; ++u)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const char *v0 = base + 2 * RG::PIECE + RG::voff(grp, 32 * u + 16 * j + col);
          const u32x2 lo = *(const volatile __attribute__((address_space(3))) u32x2 *)v0;
          const u32x2 hi = *(const volatile __attribute__((address_space(3))) u32x2 *)(v0 + RG::PIECE);
          va[2 * u + j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
    }
    // Row tile by row tile: each tile's logits, then its running-maximum
    // test (and the rare rescale) as a branch of its own; the weights and
    // value products of both tiles follow.  (Taking both tiles' logits
    // before one test for both, or interleaving the first tile's weights
    // with the second tile's logit products, measured 2-3% slower on the
    // 70B-class prefill.)
    float x[NQ][2][4];
    auto logits = [&](int qt) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) sacc = Ops::qk(kop[st][kk], qop[qt][kk], sacc);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[qt][st][i] = sacc[i];
      }
      if (diag) {  // wave-uniform: only tiles that reach past the first row
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int t0 = 32 * n + 16 * st + 4 * grp;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (t0 + i > pos[qt]) x[qt][st][i] = -INFINITY;
        }
      }
      if constexpr (PREFIX) {
        // no causal mask in prefix mode: the logits of tokens at or past L
        // are masked instead
        if (MAY_TAIL && 32 * n + 32 > L) {
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const int nvalid = max(0, min(4, L - (32 * n + 16 * st + 4 * grp)));
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (i >= nvalid) x[qt][st][i] = -INFINITY;
          }
        }
      }
    };
    if (MAY_TAIL && 32 * n + 32 > L) {
      // tokens at or past L may hold anything (NaN included): zero their
      // values (their logits are masked: by the causal mask in prefill,
      // every row's position being below L, and above in prefix mode)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int nvalid = max(0, min(4, L - (32 * n + 16 * st + 4 * grp)));
        if constexpr (F8) {
          const uint32_t mk = nvalid >= 4 ? 0xffffffffu : ((1u << (8 * nvalid)) - 1u);
#pragma unroll
          for (int u = 0; u < V8; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) vraw[u][st][j] &= mk;
        } else {
          const uint32_t m01 = nvalid >= 2 ? 0xffffffffu : (nvalid == 1 ? 0x0000ffffu : 0u);
          const uint32_t m23 = nvalid >= 4 ? 0xffffffffu : (nvalid == 3 ? 0x0000ffffu : 0u);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            va[t][2 * st] &= m01;
            va[t][2 * st + 1] &= m23;
          }
        }
      }
    }
    // running maximum (base-2 units) of row tile qt, moved only when a
    // logit exceeds it by more than the slack somewhere in the wave
    auto update_max = [&](int qt) {
      const float xm = fmaxf(fmaxf(fmaxf(x[qt][0][0], x[qt][0][1]), fmaxf(x[qt][0][2], x[qt][0][3])),
                             fmaxf(fmaxf(x[qt][1][0], x[qt][1][1]), fmaxf(x[qt][1][2], x[qt][1][3])));
      const float mb = xm * c2;
      if (wave_any(mb > m[qt] + kRescaleSlack)) {
        float mh = fmaxf(mb, __shfl_xor(mb, 16));
        mh = fmaxf(mh, __shfl_xor(mh, 32));
        const float m_new = fmaxf(m[qt], mh);
        const float alpha = fast_exp2(m[qt] - (m_new == -INFINITY ? 0.f : m_new));
        lsum[qt] *= alpha;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[qt][nt] *= alpha;
        m[qt] = m_new;
      }
    };
    auto weights = [&](int qt) -> u32x4 {
      const float nm = m[qt] == -INFINITY ? 0.f : -m[qt];
      float p[2][4];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[st][i] = fast_exp2(__builtin_fmaf(x[qt][st][i], c2, nm));
      return u32x4{Ops::pack2(p[0][0], p[0][1]), Ops::pack2(p[0][2], p[0][3]),
                   Ops::pack2(p[1][0], p[1][1]), Ops::pack2(p[1][2], p[1][3])};
    };
    auto values = [&](int qt, const u32x4 &pb) {
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[qt][t] = Ops::pv32(va[t], pb, acc[qt][t]);
      lsum[qt] = Ops::pv32(ones, pb, lsum[qt]);  // every row: the sum of the weights
    };
    if constexpr (F8) {
      // n-tile 4u + j: dim 64u + 4*col + j, its four tokens of tile 0 then
      // of tile 1
#pragma unroll
      for (int u = 0; u < V8; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w0 = vraw[u][0][j], w1 = vraw[u][1][j];
          va[4 * u + j] = u32x4{fp8x2_to_16<QT>(w0, false), fp8x2_to_16<QT>(w0, true),
                                fp8x2_to_16<QT>(w1, false), fp8x2_to_16<QT>(w1, true)};
        }
    }
    static_assert(NQ == 2, "two row tiles per wavefront");
    logits(0);
    update_max(0);
    logits(1);
    const u32x4 pb0 = weights(0);
    update_max(1);
    values(0, pb0);
    const u32x4 pb1 = weights(1);
    values(1, pb1);
  };

  // Pipeline: S - 1 super-tiles in flight.  Iteration n waits for its own
  // loads of super-tile n (the loads of later super-tiles may stay
  // outstanding), meets the other wavefronts at the barrier (then super-tile
  // n is complete in LDS and everyone is done with super-tile n - 1), refills
  // the stage super-tile n - 1 used, and computes on super-tile n.  Every
  // super-tile costs each wavefront exactly RG::LOADS loads, so the counts
  // below are exact.
  static_assert((S - 2) * RG::LOADS < 16, "vmcnt range");
  const int n_pre = min(S - 1, n_super);
  for (int n = 0; n < n_pre; ++n) issue(n, lookup(n), n);
  if constexpr (PREFIX) {
    // a chunk is a few super-tiles: the queries load together with the
    // first ones (one latency instead of two), and all of them are waited
    // for before the first step, after which only the ring's loads are
    // outstanding and the counts below are exact again
    load_q();
    wait_vm<0>();
  }
  // the table entry of the next super-tile to issue is read one iteration
  // ahead, so its latency hides behind a compute and a barrier
  int phys_next = n_pre < n_super ? lookup(n_pre) : 0;
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  int n = 0;
  // steady state, S iterations per trip while at least 2 S super-tiles
  // remain: every iteration leaves S - 2 later super-tiles in flight,
  // refills a stage, reads one entry ahead, and ends at least 32 tokens
  // before L (no tail mask); the stages are constants
  for (; n + 2 * S <= n_super; n += S) {
#pragma unroll
    for (int b = 0; b < S; ++b) {
      wait_vm<(S - 2) * RG::LOADS>();
      barrier();
      issue(n + b + S - 1, phys_next, (b + S - 1) % S);
      if (n + b < n_super_w) compute(n + b, b, std::false_type{});  // wave-uniform
      phys_next = lookup(n + b + S);
    }
  }
  for (; n < n_super; ++n) {
    const int later = min(S - 2, n_super - 1 - n);  // super-tiles issued after n
    if (later >= 2)
      wait_vm<2 * RG::LOADS>();
    else if (later == 1)
      wait_vm<RG::LOADS>();
    else
      wait_vm<0>();
    barrier();
    if (n + S - 1 < n_super) issue(n + S - 1, phys_next, (n + S - 1) % S);
    if (n < n_super_w) compute(n, n % S, std::true_type{});  // wave-uniform
    if (n + S < n_super) phys_next = lookup(n + S);
  }
  static_assert(S == 4, "the general loop's waits cover S - 2 = 2 later super-tiles");

  if constexpr (PREFIX) {
    // the partial state of each row: maximum (log2 units), sum of the
    // weights and weighted sum of values, un-normalised; every row of a
    // chunk saw at least one token, so its maximum is finite.  Row m =
    // 4*grp + i of n-tile 2u+j is dim 32u + 16j + m (16-bit caches; the
    // lane's four rows are four adjacent dims), of n-tile 4u+j dim
    // 64u + 4m + j (8-bit caches; four adjacent dims stored together).
#pragma unroll
    for (int qt = 0; qt < NQ; ++qt) {
      if (row0 + qt * 16 + col > row_last) continue;  // no row in this column
      float *po = a.ws_o + pidx[qt] * D;
      if (grp == 0) {
        a.ws_m[pidx[qt]] = m[qt];
        a.ws_l[pidx[qt]] = lsum[qt][0];
      }
      if constexpr (F8) {
#pragma unroll
        for (int u = 0; u < V8; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            *reinterpret_cast<f32x4 *>(po + 64 * u + 4 * (4 * grp + i)) =
                f32x4{acc[qt][4 * u][i], acc[qt][4 * u + 1][i], acc[qt][4 * u + 2][i],
                      acc[qt][4 * u + 3][i]};
      } else {
        // n-tile t: dims 32(t/2) + 16(t%2) + 4*grp .. +3, one 16-byte store
#pragma unroll
        for (int t = 0; t < NT; ++t)
          *reinterpret_cast<f32x4 *>(po + 32 * (t / 2) + 16 * (t % 2) + 4 * grp) = acc[qt][t];
      }
    }
    return;
  }

  // normalise and store: row m = 4*grp + i of n-tile 2u+j is dim
  // 32u + 16j + m of the lane's query row (16-bit caches), of n-tile 4u+j
  // dim 64u + 4m + j (8-bit caches); either way the lane holds four
  // adjacent dims, stored as one 64-bit word.  Each pair is rounded to the
  // 16-bit type (nearest even) by one packed conversion: the outputs are
  // finite, and the bit-level rounding with its NaN branch took more than
  // twice the instructions of the whole bfloat16 epilogue.
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    const float lt = lsum[qt][0];
    if (row0 + qt * 16 + col > row_last) continue;  // no row in this column
    const float inv = lt > 0.f ? a.v_scale / lt : 0.f;
    uint32_t *op = reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(a.out) + orow[qt]);
    if constexpr (F8) {
#pragma unroll
      for (int u = 0; u < V8; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = 64 * u + 4 * (4 * grp + i);
          const u32x2 wv = {Ops::pack2(acc[qt][4 * u][i] * inv, acc[qt][4 * u + 1][i] * inv),
                            Ops::pack2(acc[qt][4 * u + 2][i] * inv, acc[qt][4 * u + 3][i] * inv)};
          *reinterpret_cast<u32x2 *>(op + (d >> 1)) = wv;
        }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int d = 32 * (t / 2) + 16 * (t % 2) + 4 * grp;
        const u32x2 wv = {Ops::pack2(acc[qt][t][0] * inv, acc[qt][t][1] * inv),
                          Ops::pack2(acc[qt][t][2] * inv, acc[qt][t][3] * inv)};
        *reinterpret_cast<u32x2 *>(op + (d >> 1)) = wv;
      }
    }
  }
}

int64_t prefix_grid(int num_groups, int num_kv_heads, int n_chunks, int q_blocks) {
  const int64_t units = (int64_t)num_groups * num_kv_heads * n_chunks;
  return (int64_t)kXcds * ((units + kXcds - 1) / kXcds) * q_blocks;
}

template <int QT, int CT, int D, int BS>
static hipError_t launch_prefix(const PrefillArgs &a, hipStream_t st) {
  const int64_t n = prefix_grid(a.num_groups, a.num_kv_heads, a.n_chunks, a.q_blocks);
  hipLaunchKernelGGL((prefill_mfma_kernel<QT, CT, D, BS, true>), dim3((unsigned)n),
                     dim3(kPrefillThreads), 0, st, a);
  return hipGetLastError();
}

template <int QT, int CT>
static hipError_t launch_prefix_dt(const PrefillArgs &a, int head_dim, int block_size,
                                   hipStream_t st) {
  if (head_dim == 128)
    return block_size == 16 ? launch_prefix<QT, CT, 128, 16>(a, st)
                            : launch_prefix<QT, CT, 128, 32>(a, st);
  return block_size == 16 ? launch_prefix<QT, CT, 64, 16>(a, st)
                          : launch_prefix<QT, CT, 64, 32>(a, st);
}

hipError_t launch_prefix_mfma(const PrefillArgs &a, int dtype, int cache_dtype, int head_dim,
                              int block_size, hipStream_t st) {
  if (a.num_groups == 0 || a.q_blocks == 0 || a.n_chunks == 0) return hipSuccess;
  (void)cache_dtype;  // 16-bit caches of the query's type
  if (dtype == DT_F16) return launch_prefix_dt<DT_F16, DT_F16>(a, head_dim, block_size, st);
  return launch_prefix_dt<DT_BF16, DT_BF16>(a, head_dim, block_size, st);
}

template <int QT, int CT, int D, int BS>
static hipError_t launch_prefill(const PrefillArgs &a, hipStream_t st) {
  const int64_t n = prefill_grid(a.num_seqs, a.num_kv_heads, a.q_blocks);
  // a kernel of its own for the ordered grid: the select, inlined into the
  // other, changed the register allocation of its main loop (2% slower)
  if (n / kXcds <= kPrefillOrderMaxUnits)
    hipLaunchKernelGGL((prefill_mfma_kernel<QT, CT, D, BS, false, true>), dim3((unsigned)n),
                       dim3(kPrefillThreads), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_mfma_kernel<QT, CT, D, BS>), dim3((unsigned)n),
                       dim3(kPrefillThreads), 0, st, a);
  return hipGetLastError();
}

template <int QT, int CT>
static hipError_t launch_prefill_dt(const PrefillArgs &a, int head_dim, int block_size,
                                    hipStream_t st) {
  if (head_dim == 128)
    return block_size == 16 ? launch_prefill<QT, CT, 128, 16>(a, st)
                            : launch_prefill<QT, CT, 128, 32>(a, st);
  return block_size == 16 ? launch_prefill<QT, CT, 64, 16>(a, st)
                          : launch_prefill<QT, CT, 64, 32>(a, st);
}

hipError_t launch_prefill_mfma(const PrefillArgs &a, int dtype, int cache_dtype, int head_dim,
                               int block_size, int max_query_len, hipStream_t st) {
  (void)max_query_len;
  if (a.num_seqs == 0 || a.q_blocks == 0) return hipSuccess;
  if (cache_dtype == DT_FP8) {
    if (dtype == DT_F16) return launch_prefill_dt<DT_F16, DT_FP8>(a, head_dim, block_size, st);
    return launch_prefill_dt<DT_BF16, DT_FP8>(a, head_dim, block_size, st);
  }
  if (dtype == DT_F16) return launch_prefill_dt<DT_F16, DT_F16>(a, head_dim, block_size, st);
  return launch_prefill_dt<DT_BF16, DT_BF16>(a, head_dim, block_size, st);
}

}  // namespace pkv
