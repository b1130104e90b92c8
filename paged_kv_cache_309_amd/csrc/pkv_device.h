// pkv_device.h - device-side helpers shared by the gfx950 kernels.
//
// Storage types are handled as raw 32-bit words: a 16-byte global load
// brings four words, i.e. eight fp16/bf16 elements or four fp32 elements,
// and elements are widened to fp32 in registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_internal.h"

namespace pkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <int DT> struct Elem;
template <> struct Elem<DT_F32> { static constexpr int bytes = 4; };
template <> struct Elem<DT_F16> { static constexpr int bytes = 2; };
template <> struct Elem<DT_BF16> { static constexpr int bytes = 2; };
template <> struct Elem<DT_FP8> { static constexpr int bytes = 1; };

// Element j of a run of words (j counts elements, not words).
template <int DT>
__device__ __forceinline__ float elem(const uint32_t *w, int j) {
  if constexpr (DT == DT_F32) {
    return __uint_as_float(w[j]);
  } else if constexpr (DT == DT_FP8) {
    // E4M3 byte (j & 3) of word j / 4, widened exactly by the hardware (the
    // byte select is an immediate: j is a constant after unrolling)
    const int x = static_cast<int>(w[j >> 2]);
    switch (j & 3) {
      case 0: return __builtin_amdgcn_cvt_f32_fp8(x, 0);
      case 1: return __builtin_amdgcn_cvt_f32_fp8(x, 1);
      case 2: return __builtin_amdgcn_cvt_f32_fp8(x, 2);
      default: return __builtin_amdgcn_cvt_f32_fp8(x, 3);
    }
  } else if constexpr (DT == DT_BF16) {
    const uint32_t x = w[j >> 1];
    return (j & 1) ? __uint_as_float(x & 0xffff0000u) : __uint_as_float(x << 16);
  } else {
    const f16x2 h = __builtin_bit_cast(f16x2, w[j >> 1]);
    return (j & 1) ? static_cast<float>(h.y) : static_cast<float>(h.x);
  }
}

// fp32 -> storage bits, rounding to nearest-even.
template <int DT> __device__ __forceinline__ uint32_t from_f32(float x);
template <> __device__ __forceinline__ uint32_t from_f32<DT_F32>(float x) {
  return __float_as_uint(x);
}
template <> __device__ __forceinline__ uint32_t from_f32<DT_F16>(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}
template <> __device__ __forceinline__ uint32_t from_f32<DT_BF16>(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// float -> E4M3 byte (the OCP 8-bit float with 4 exponent bits, bias 7,
// 3 fraction bits, no infinity, largest finite 448), nearest value with
// ties to the even fraction; magnitudes of 448 and beyond saturate to +-448,
// NaN gives 0x7f.  Normal results round the float's 23-bit fraction to 3
// bits on its bit pattern; results below 2^-6 are multiples of 2^-9, found
// by rounding y * 512 to the nearest even integer.
__device__ __forceinline__ uint32_t e4m3_from_f32(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;                    // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;            // >= 448 (and inf)
  if (a < 0x3c800000u)                                  // below 2^-6
    return sign | static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.0f));
  const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;  // exponent | 3 bits
  const uint32_t code = r - (120u << 3);                       // bias 127 -> 7
  return sign | (code < 0x7eu ? code : 0x7eu);
}

template <int DT>
__device__ __forceinline__ void store_elem(void *base, size_t idx, float x) {
  if constexpr (DT == DT_F32) {
    static_cast<float *>(base)[idx] = x;
  } else {
    static_cast<uint16_t *>(base)[idx] = static_cast<uint16_t>(from_f32<DT>(x));
  }
}

// A store that writes through L2 to memory (a relaxed store at system
// scope).  Lines a kernel leaves dirty in L2 are written back when it ends,
// and that write-back runs far below the HBM write rate; results that no
// later read in the same kernel wants go through instead.  Used where a
// wave's store instruction covers whole 128-byte lines.
__device__ __forceinline__ void store_through(float *p, float x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// DPP lane permutations inside a row of 16 lanes.
enum : int {
  DPP_QUAD_XOR1 = 0xB1,    // quad_perm [1,0,3,2]
  DPP_QUAD_XOR2 = 0x4E,    // quad_perm [2,3,0,1]
  DPP_ROW_MIRROR = 0x140,  // lane i <- lane 15-i
  DPP_ROW_HMIRROR = 0x141  // lane i <- lane 7-i within each half row
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a row; every lane of the row receives the same
// bits (each step adds the same two partial sums, in either order).
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<DPP_QUAD_XOR1>(x);
  x += dpp<DPP_QUAD_XOR2>(x);
  x += dpp<DPP_ROW_HMIRROR>(x);
  x += dpp<DPP_ROW_MIRROR>(x);
  return x;
}

// K/V tiles are streamed: each is read once per decode step, so the loads
// carry the non-temporal hint (measured on MI355X: random 4 KiB tile reads
// reach about 6.8 TB/s with it and about 6.0 TB/s without).
__device__ __forceinline__ u32x4 load_stream16(const void *p) {
  return __builtin_nontemporal_load(static_cast<const u32x4 *>(p));
}
// Plain loads: the lines stay in cache for other readers.
__device__ __forceinline__ u32x4 load_keep16(const void *p) {
  return *static_cast<const u32x4 *>(p);
}
__device__ __forceinline__ u32x2 load_keep8(const void *p) {
  return *static_cast<const u32x2 *>(p);
}
__device__ __forceinline__ u32x2 load_stream8(const void *p) {
  return __builtin_nontemporal_load(static_cast<const u32x2 *>(p));
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// Rescaling threshold of the online softmax, in log2 units.  The running
// maximum m of a softmax state is only moved when a new logit exceeds it by
// more than this; until then the weights 2^(x - m) may reach 2^kRescaleSlack.
// The final division by the running sum cancels the common factor, so the
// result is the same softmax; the wave skips the rescale of its accumulators
// on almost every tile.
constexpr float kRescaleSlack = 8.0f;

// True in every lane when any lane of the wavefront has `pred` set.
__device__ __forceinline__ bool wave_any(bool pred) {
  return __builtin_amdgcn_ballot_w64(pred) != 0;
}

// Counting select: the item of rank r (0 <= r < n) when items 0 .. n-1 are
// ordered by bucket(i) in [0, kOrderBuckets), ascending, and by index within
// a bucket.  Computed in every workgroup that needs it:
//   * a histogram of the buckets in LDS and its prefix sum give the bucket
//     that holds rank r and r's place k inside it;
//   * the k-th item of that bucket in index order is the result.
// Each thread does O(n / NT + 1) work and calls bucket() at most twice per
// item (item i in pass p by thread i % NT).  `scratch` is LDS of at least
// kOrderScratchInts ints, free for reuse once this returns; the select takes
// no other LDS (in a kernel whose LDS sits at the limit for two workgroups
// per CU, a few more bytes halve the occupancy).  Called by every thread of
// the workgroup.
constexpr int kOrderBuckets = 256;
constexpr int kOrderScratchInts = kOrderBuckets + 8;

template <int NT, class Bucket>
__device__ __forceinline__ int counting_select(int n, int r, const Bucket &bucket,
                                               int *scratch) {
  static_assert(NT == kOrderBuckets, "one thread per bucket");
  int *hist = scratch;                  // kOrderBuckets counters
  int *wsum = scratch + kOrderBuckets;  // one total per wavefront
  int &sel_bucket = scratch[kOrderBuckets + 4], &sel_k = scratch[kOrderBuckets + 5];
  int &chosen = scratch[kOrderBuckets + 6];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  hist[tid] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += NT) atomicAdd(&hist[bucket(i)], 1);
  __syncthreads();
  // inclusive prefix sum of the histogram: within each wavefront, then the
  // totals of the wavefronts before it
  const int h = hist[tid];
  int x = h;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  for (int q = 0; q < w; ++q) x += wsum[q];
  if (x - h <= r && r < x) {  // exactly one bucket holds rank r (r < n)
    sel_bucket = tid;
    sel_k = r - (x - h);
  }
  __syncthreads();
  const int bsel = sel_bucket, k = sel_k;
  // the k-th member of bucket bsel in index order, NT items a pass
  int base = 0;
  for (int c = 0; c < n; c += NT) {
    const int i = c + tid;
    const bool f = i < n && bucket(i) == bsel;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(f);
    const int before_lane = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[w] = __builtin_popcountll(bal);
    __syncthreads();
    int before = base, total = 0;
    for (int q = 0; q < NT / 64; ++q) {
      if (q < w) before += wsum[q];
      total += wsum[q];
    }
    if (f && before + before_lane == k) chosen = i;
    base += total;
    __syncthreads();  // wsum is rewritten by the next pass
    if (base > k) break;  // uniform: every thread holds the same base
  }
  const int result = chosen;
  __syncthreads();  // the scratch is the caller's again
  return result;
}

// Longest-first order of the single-pass grid.  Work items of one launch
// differ in length by up to two orders of magnitude; the dispatcher starts
// workgroups in grid order, so a long sequence that starts late stretches
// the end of the kernel.  Workgroup row r therefore processes the sequence
// of rank r in an order of decreasing context length, a counting select
// over context_lens: lengths (clamped to [0, max_tokens]) fall into 256
// buckets of equal width 2^sh, bucket (max_tokens - L) >> sh, so bucket 0
// holds the longest.  The order is longest-first up to the bucket width
// (max_tokens / 256 tokens or less); it only chooses which workgroup does
// which sequence, never the arithmetic.
// Every workgroup reads all S lengths to find its rank, so the order costs
// O(S) per workgroup.  Above this many sequences the grid keeps sequence
// order: its cost outgrows the tail it saves (short contexts, bf16, 2 or 8
// heads: 2048 sequences 26.6 -> 15.5 us, 4096 62 -> 22 us, 16384 544 -> 74
// us; 1024 sequences alike either way).
constexpr int kOrderMaxSeqs = 1024;

template <int NT>
__device__ __forceinline__ int longest_first_seq(const int32_t *context_lens, int S,
                                                 int max_tokens, int r, int *scratch) {
  if (S > kOrderMaxSeqs) return r;  // uniform over the workgroup
  max_tokens = max(max_tokens, 0);
  int sh = 0;
  while ((max_tokens >> sh) >= kOrderBuckets) ++sh;
  const auto bucket = [&](int i) {
    const int L = max(0, min(context_lens[i], max_tokens));
    return (max_tokens - L) >> sh;
  };
  return counting_select<NT>(S, r, bucket, scratch);
}

// Leading blocks of a context of tok_end tokens that the neighbouring
// sequence's table (the next sequence's; the previous one's for the last)
// maps to the same physical blocks: a shared prefix, which every sharer
// reads, so its tiles are read with loads that keep them in cache.
// Sequences that share a prefix sit side by side in a batch.  64 entries
// per step (one vector load of each table and a ballot), stopping at the
// first entry that differs - at once for a sequence that shares nothing.
// Wave-uniform.
template <int BS>
__device__ __forceinline__ int shared_prefix_blocks(const int32_t *block_tables,
                                                    int max_blocks, int num_seqs, int s,
                                                    int tok_end, int lane) {
  if (num_seqs <= 1) return 0;
  const int32_t *trow = block_tables + (size_t)s * max_blocks;
  const int32_t *tnb = block_tables + (size_t)(s + 1 < num_seqs ? s + 1 : s - 1) * max_blocks;
  const int nblk = (tok_end + BS - 1) / BS;
  int j0 = 0;
  for (; j0 < nblk; j0 += 64) {
    const int j = j0 + lane;
    const uint64_t differ = __builtin_amdgcn_ballot_w64(j < nblk && trow[j] != tnb[j]);
    if (differ) return j0 + (int)__builtin_ctzll(differ);
  }
  return nblk;
}

// Walks the 16-token tiles a wavefront owns, with one tile of prefetch.
//
// The wave owns tiles k = k0 + STRIDE*n, n = 0 .. n_mine-1 (decode: k0 =
// first tile of the range + wave index, STRIDE = 4 waves); tile k lives in
// block table entry k / subs, at token offset 16 * (k % subs) of that
// block.  Entries are wave-uniform and read with scalar loads, one tile
// ahead of their use; they count on their own counter, apart from the
// tiles' vector loads.
//
//   load(tile, byte_offset)  issues the loads of one tile
//   compute(tile, n)         consumes the n-th tile
//
// Two tile buffers alternate (no register copies between iterations).  In
// the steady state no load is conditional, so the wait before each compute
// leaves the next tile's loads outstanding: a load that may or may not have
// been issued makes the compiler count conservatively and drain it.
// n_mine >= 1.
template <class Tile, int STRIDE = 4, class Load, class Compute>
__device__ __forceinline__ void walk_tiles(const int32_t *trow, int k0, int n_mine,
                                           int subs, unsigned num_blocks,
                                           size_t head_off_bytes,
                                           size_t block_bytes, size_t sub_bytes,
                                           Load load, Compute compute) {
  const __attribute__((address_space(4))) int32_t *tr =
      (const __attribute__((address_space(4))) int32_t *)trow;
  auto entry = [&](int n) -> int { return tr[(k0 + STRIDE * n) / subs]; };
  auto offset_of = [&](int n, int phys) -> size_t {
    phys = (unsigned)phys < num_blocks ? phys : 0;
    const int k = k0 + STRIDE * n;
    return (size_t)phys * block_bytes + head_off_bytes + (size_t)(k % subs) * sub_bytes;
  };
  Tile ta, tb;
  load(ta, offset_of(0, entry(0)));
  int phys_next = 1 < n_mine ? entry(1) : 0;  // entry of the next tile to load
  int n = 0;
  for (; n + 2 < n_mine; n += 2) {
    load(tb, offset_of(n + 1, phys_next));
    phys_next = entry(n + 2);
    compute(ta, n);
    load(ta, offset_of(n + 2, phys_next));
    if (n + 3 < n_mine) phys_next = entry(n + 3);
    compute(tb, n + 1);
  }
  // one or two tiles left; ta holds tile n
  if (n + 1 < n_mine) {
    load(tb, offset_of(n + 1, phys_next));
    compute(ta, n);
    compute(tb, n + 1);
  } else {
    compute(ta, n);
  }
}

// The same walk with NBUF - 1 tiles in flight while one is computed
// (NBUF buffers in rotation), for the matrix-core kernel: two tiles of
// lookahead for 16-bit caches, three for the 2 KiB tiles of 8-bit caches.
// Block-table entries are read with scalar loads one tile ahead, as in
// walk_tiles.
template <class Tile, int NBUF, int STRIDE = 4, class Load, class Compute>
__device__ __forceinline__ void walk_tiles_n(const int32_t *trow, int k0, int n_mine,
                                             int subs, unsigned num_blocks,
                                             size_t head_off_bytes,
                                             size_t block_bytes, size_t sub_bytes,
                                             Load load, Compute compute) {
  static_assert(NBUF >= 2, "at least two buffers");
  const __attribute__((address_space(4))) int32_t *tr =
      (const __attribute__((address_space(4))) int32_t *)trow;
  auto entry = [&](int n) -> int { return tr[(k0 + STRIDE * n) / subs]; };
  auto offset_of = [&](int n, int phys) -> size_t {
    phys = (unsigned)phys < num_blocks ? phys : 0;
    const int k = k0 + STRIDE * n;
    return (size_t)phys * block_bytes + head_off_bytes + (size_t)(k % subs) * sub_bytes;
  };
  // invariant at the top of each loop: t[b] holds tile n + b, b < NBUF - 1,
  // and phys_next is the entry of tile n + NBUF - 1
  Tile t[NBUF];
  int n = 0, phys_next = 0;
  if (n_mine > 2 * NBUF - 2) {
    // a walk long enough for the steady state: nothing before it is
    // conditional either, so the waits there leave exactly the later
    // tiles' loads outstanding (a load that may or may not have been
    // issued makes the compiler count conservatively, draining them)
    // in tile order (a scheduling barrier after each tile keeps the
    // compiler from reordering the loads, which would make the first
    // compute wait for all of them)
#pragma unroll
    for (int b = 0; b < NBUF - 1; ++b) {
      load(t[b], offset_of(b, entry(b)));
      __builtin_amdgcn_sched_barrier(0);
    }
    phys_next = entry(NBUF - 1);
    for (; n + 2 * NBUF - 2 < n_mine; n += NBUF) {
#pragma unroll
      for (int b = 0; b < NBUF; ++b) {
        const int nl = n + b + NBUF - 1;  // the tile loaded in this step
        load(t[(b + NBUF - 1) % NBUF], offset_of(nl, phys_next));
        if (nl + 1 < n_mine) phys_next = entry(nl + 1);
        compute(t[b], n + b);
      }
    }
  } else {
#pragma unroll
    for (int b = 0; b < NBUF - 1; ++b)
      if (b < n_mine) load(t[b], offset_of(b, entry(b)));
    phys_next = NBUF - 1 < n_mine ? entry(NBUF - 1) : 0;
  }
  // the last round (at most one), with the loads guarded
  for (; n + NBUF - 1 < n_mine; n += NBUF) {
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      const int nl = n + b + NBUF - 1;
      if (nl < n_mine) {
        load(t[(b + NBUF - 1) % NBUF], offset_of(nl, phys_next));
        if (nl + 1 < n_mine) phys_next = entry(nl + 1);
      }
      compute(t[b], n + b);
    }
  }
#pragma unroll
  for (int b = 0; b < NBUF - 1; ++b)
    if (n + b < n_mine) compute(t[b], n + b);
}

}  // namespace pkv
