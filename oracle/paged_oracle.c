/*
 * paged_oracle.c - the oracle for paged decode attention and for the
 * cache write that fills the paged KV pool.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  The product path (the HIP library
 * and its Python binding) never calls it, and it shares no code, header or
 * constant with that path.
 *
 * What it computes, in IEEE double precision and in the plainest order:
 *
 *  1. The cache write.  A KV cache is cut into fixed-size blocks, and a
 *     token's key and value live in one slot of one physical block
 *     ("Why vLLM Uses PagedAttention", section "The insight": a page maps to
 *     a KV block, a byte to one token's KV; section "The mechanism": 16-token
 *     blocks by default).  A slot number is physical_block * block_size +
 *     offset_in_block.  Each new token's K and V bits are copied into the
 *     slot it is given; every other byte of the pool stays as it was.
 *
 *  2. Decode attention.  For every sequence s and query head h the result is
 *     ordinary single-query attention softmax(q . K^T * scale) . V over the
 *     sequence's first context_lens[s] tokens ("PagedAttention: how vLLM
 *     manages the KV cache", section "PagedAttention changes addressing
 *     inside attention": the computation is that of ordinary attention, only
 *     the way K and V are located changes).  K and V of token t are reached
 *     through the block table: logical block t / block_size, offset
 *     t % block_size, physical block block_tables[s][t / block_size]
 *     ("Paged Attention" placement notes, section "Paged Attention's
 *     Approach": the worked request whose token 48 lands in logical block 3;
 *     "Why vLLM Uses PagedAttention", section "The mechanism": the block table
 *     maps logical to physical blocks like a page table).
 *
 *     The softmax is done in two passes (all logits, then their maximum,
 *     then the weights), not with a running maximum, so that it shares no
 *     algorithm with the device kernels.
 *
 * Readings of the pages (they are silent or garbled on these points):
 *   - the context length counts the token being decoded, which was written
 *     to the cache just before attention, so tokens 0 .. L-1 are attended
 *     (the worked example attends to tokens 0-48 while token 48 is placed);
 *   - the number of blocks walked is ceil(L / block_size): a partly filled
 *     last block is still read, only up to token L-1;
 *   - K and V are two pools of the same block structure (the sketch keeps
 *     them in one tensor);
 *   - grouped-query attention maps query head h to KV head
 *     h / (num_heads / num_kv_heads) (consecutive groups);
 *   - L = 0 yields an all-zero output;
 *   - a negative slot means "no write" (a padding token); a slot beyond the
 *     pool, or two writes to one slot, is rejected with an error code.
 *
 * Pool layouts (the product library documents the same two formulas; they
 * are restated here independently):
 *   K element (block p, kv head g, offset o, dim d):
 *       ((p * Hkv + g) * bs + o) * D + d
 *   V element (block p, kv head g, offset o, dim d):
 *       (p * Hkv + g) * bs * D + (o / 4) * 4 * D + d * 4 + (o % 4)
 *   i.e. V keeps each run of four consecutive tokens of one dimension next to
 *   each other.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_FP8 = 3 };

enum {
  OR_OK = 0,
  OR_ERR_ARG = 1,        /* bad sizes or dtype */
  OR_ERR_TABLE = 2,      /* a block-table entry outside [0, num_blocks) */
  OR_ERR_CONTEXT = 3,    /* context length above max_blocks * block_size */
  OR_ERR_SLOT_RANGE = 4, /* slot >= num_blocks * block_size */
  OR_ERR_SLOT_DUP = 5,   /* two tokens share one slot */
  OR_ERR_NOMEM = 6
};

/* ---- element decoding ------------------------------------------------ */

/* IEEE binary16 -> double, written out from the format's definition:
 * sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double half_bits_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int ex = (h >> 10) & 0x1f;
  int fr = h & 0x3ff;
  double v;
  if (ex == 0) {
    v = ldexp((double)fr, -24); /* subnormal: fr * 2^-14 * 2^-10 */
  } else if (ex == 31) {
    v = fr ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + fr), ex - 25); /* (1 + fr/1024) * 2^(ex-15) */
  }
  return sign ? -v : v;
}

/* bfloat16 -> double: a bfloat16 is the upper half of a binary32. */
static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* 8-bit float E4M3 ("FN" variant of the OCP 8-bit formats), written out
 * from the format's definition: sign bit, 4 exponent bits (bias 7), 3
 * fraction bits; exponent 0 encodes subnormals fr * 2^-9; there is no
 * infinity, and exponent 15 with fraction 7 is NaN, so the largest finite
 * value is 1.75 * 2^8 = 448. */
static double e4m3_bits_to_double(uint8_t b) {
  int sign = (b >> 7) & 1;
  int ex = (b >> 3) & 0xf;
  int fr = b & 7;
  double v;
  if (ex == 0xf && fr == 7)
    return NAN;
  if (ex == 0)
    v = ldexp((double)fr, -9);
  else
    v = ldexp((double)(8 + fr), ex - 10); /* (1 + fr/8) * 2^(ex-7) */
  return sign ? -v : v;
}

/* Nearest E4M3 value of a float, ties to the even fraction; magnitudes
 * beyond the largest finite value saturate to +-448; NaN -> NaN (0x7f).
 * The candidates come from the definition: the representable non-negative
 * values are e4m3_bits_to_double(0 .. 126), increasing with the code, and
 * the code just below a value is found by bisection over them. */
static uint8_t e4m3_encode(float y) {
  if (isnan(y))
    return 0x7f;
  uint8_t sign = signbit(y) ? 0x80 : 0x00;
  double a = fabs((double)y);
  if (a >= 448.0)
    return sign | 0x7e;
  /* largest code whose value is <= a: value(lo) <= a < value(hi) */
  int lo = 0, hi = 126;
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (e4m3_bits_to_double((uint8_t)mid) <= a)
      lo = mid;
    else
      hi = mid;
  }
  if (e4m3_bits_to_double((uint8_t)hi) <= a)
    lo = hi;
  int code = lo;
  if (lo < 126) {
    double vlo = e4m3_bits_to_double((uint8_t)lo);
    double vhi = e4m3_bits_to_double((uint8_t)(lo + 1));
    if (a - vlo > vhi - a || (a - vlo == vhi - a && (lo & 1)))
      code = lo + 1;
  }
  return sign | (uint8_t)code;
}

static double load_elem(const void *base, size_t idx, int dtype) {
  switch (dtype) {
  case OR_F32:
    return (double)((const float *)base)[idx];
  case OR_F16:
    return half_bits_to_double(((const uint16_t *)base)[idx]);
  case OR_FP8:
    return e4m3_bits_to_double(((const uint8_t *)base)[idx]);
  default:
    return bf16_bits_to_double(((const uint16_t *)base)[idx]);
  }
}

static int elem_bytes(int dtype) {
  return dtype == OR_F32 ? 4 : (dtype == OR_FP8 ? 1 : 2);
}

/* ---- pool addressing ---------------------------------------------------- */

static size_t k_index(size_t p, size_t g, size_t o, size_t d, size_t hkv,
                      size_t bs, size_t hd) {
  return ((p * hkv + g) * bs + o) * hd + d;
}

static size_t v_index(size_t p, size_t g, size_t o, size_t d, size_t hkv,
                      size_t bs, size_t hd) {
  return (p * hkv + g) * bs * hd + (o / 4) * 4 * hd + d * 4 + (o % 4);
}

/* ---- the cache write ----------------------------------------------------- */

/* k, v: [num_tokens, num_kv_heads, head_dim] in the pool's element type.
 * k_cache, v_cache: flat pools of num_blocks * num_kv_heads * block_size *
 * head_dim elements.  Returns an OR_* code; on error the pools are left
 * untouched. */
int oracle_reshape_and_cache(const void *k, const void *v, void *k_cache,
                             void *v_cache, const int64_t *slot_mapping,
                             int64_t num_tokens, int num_kv_heads,
                             int head_dim, int block_size, int64_t num_blocks,
                             int dtype) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      block_size % 4 != 0 || num_blocks < 0 || dtype < OR_F32 ||
      dtype > OR_BF16)
    return OR_ERR_ARG;
  const int64_t nslots = num_blocks * (int64_t)block_size;
  /* precheck: every slot in range, no slot written twice */
  unsigned char *seen = calloc((size_t)(nslots / 8 + 1), 1);
  if (!seen)
    return OR_ERR_NOMEM;
  for (int64_t i = 0; i < num_tokens; ++i) {
    int64_t s = slot_mapping[i];
    if (s < 0)
      continue;
    if (s >= nslots) {
      free(seen);
      return OR_ERR_SLOT_RANGE;
    }
    if (seen[s / 8] & (1u << (s % 8))) {
      free(seen);
      return OR_ERR_SLOT_DUP;
    }
    seen[s / 8] |= (unsigned char)(1u << (s % 8));
  }
  free(seen);

  const size_t eb = (size_t)elem_bytes(dtype);
  const size_t hkv = (size_t)num_kv_heads, hd = (size_t)head_dim,
               bs = (size_t)block_size;
  for (int64_t i = 0; i < num_tokens; ++i) {
    int64_t s = slot_mapping[i];
    if (s < 0)
      continue;
    size_t p = (size_t)(s / block_size), o = (size_t)(s % block_size);
    for (size_t g = 0; g < hkv; ++g) {
      for (size_t d = 0; d < hd; ++d) {
        size_t src = ((size_t)i * hkv + g) * hd + d;
        memcpy((char *)k_cache + k_index(p, g, o, d, hkv, bs, hd) * eb,
               (const char *)k + src * eb, eb);
        memcpy((char *)v_cache + v_index(p, g, o, d, hkv, bs, hd) * eb,
               (const char *)v + src * eb, eb);
      }
    }
  }
  return OR_OK;
}

/* ---- decode attention ------------------------------------------------------ */

struct decode_job {
  double *out;
  const void *q, *k_cache, *v_cache;
  const int32_t *block_tables, *context_lens;
  double scale;
  int block_size, num_seqs, num_heads, num_kv_heads, head_dim;
  int64_t num_blocks;
  int max_blocks_per_seq, dtype; /* dtype: of the caches */
  int q_dtype;                     /* of q */
  double k_scale, v_scale;         /* dequantisation scales of the caches */
  const int32_t *sel; /* optional (seq, head) or (query row, head) pairs */
  /* multi-query (chunked prefill): query rows of sequence s are
   * query_start_loc[s] .. query_start_loc[s+1]-1; NULL for decode */
  const int32_t *query_start_loc;
  int64_t num_items;
  int num_threads;
  int status; /* first error seen (written under the lock) */
  pthread_mutex_t lock;
};

/* One query row `qrow` of sequence s and query head h, attending to the
 * first L tokens of the sequence: fills out[0 .. head_dim-1]. */
static int attend_one(const struct decode_job *jb, int s, int64_t qrow, int h,
                      int L, double *out) {
  const int hd = jb->head_dim, bs = jb->block_size;
  const int group = jb->num_heads / jb->num_kv_heads;
  const int g = h / group;
  for (int d = 0; d < hd; ++d)
    out[d] = 0.0;
  if (L <= 0)
    return OR_OK;
  if ((int64_t)L > (int64_t)jb->max_blocks_per_seq * bs)
    return OR_ERR_CONTEXT;

  const size_t hkv = (size_t)jb->num_kv_heads;
  const size_t qbase = ((size_t)qrow * jb->num_heads + h) * hd;
  const int32_t *table = jb->block_tables + (size_t)s * jb->max_blocks_per_seq;

  double *x = malloc(sizeof(double) * (size_t)L);
  if (!x)
    return OR_ERR_NOMEM;

  /* pass 1: logits x_t = scale * sum_d q[d] * K_t[d] */
  for (int t = 0; t < L; ++t) {
    int p = table[t / bs];
    int o = t % bs;
    if (p < 0 || p >= jb->num_blocks) {
      free(x);
      return OR_ERR_TABLE;
    }
    double dot = 0.0;
    for (int d = 0; d < hd; ++d)
      dot += load_elem(jb->q, qbase + d, jb->q_dtype) *
             (load_elem(jb->k_cache,
                        k_index((size_t)p, (size_t)g, (size_t)o, (size_t)d, hkv,
                                (size_t)bs, (size_t)hd),
                        jb->dtype) *
              jb->k_scale);
    x[t] = jb->scale * dot;
  }

  /* the maximum logit */
  double m = x[0];
  for (int t = 1; t < L; ++t)
    if (x[t] > m)
      m = x[t];

  /* pass 2: weights w_t = exp(x_t - m), their sum, and sum_t w_t * V_t */
  double z = 0.0;
  for (int t = 0; t < L; ++t) {
    int p = table[t / bs];
    int o = t % bs;
    double w = exp(x[t] - m);
    z += w;
    for (int d = 0; d < hd; ++d)
      out[d] += w * (load_elem(jb->v_cache,
                               v_index((size_t)p, (size_t)g, (size_t)o,
                                       (size_t)d, hkv, (size_t)bs, (size_t)hd),
                               jb->dtype) *
                     jb->v_scale);
  }
  for (int d = 0; d < hd; ++d)
    out[d] /= z;
  free(x);
  return OR_OK;
}

struct worker_arg {
  struct decode_job *jb;
  int tid;
};

/* Decode: the one query of sequence s sits at the end of its context and
 * attends to all context_lens[s] tokens.  Multi-query: the C = (number of
 * query rows of s) queries are the last C tokens of the context, in order,
 * and query j attends to the tokens up to and including itself, i.e. the
 * first context_lens[s] - C + j + 1 tokens (causal within the chunk). */
static void *decode_worker(void *argp) {
  struct worker_arg *wa = argp;
  struct decode_job *jb = wa->jb;
  for (int64_t it = wa->tid; it < jb->num_items; it += jb->num_threads) {
    int64_t r; /* query row: the sequence (decode) or a row of q */
    int h;
    if (jb->sel) {
      r = jb->sel[2 * it];
      h = jb->sel[2 * it + 1];
    } else {
      r = it / jb->num_heads;
      h = (int)(it % jb->num_heads);
    }
    int s = (int)r, L;
    if (jb->query_start_loc) {
      const int32_t *qsl = jb->query_start_loc;
      s = 0;
      while (s + 1 < jb->num_seqs && qsl[s + 1] <= r)
        ++s;
      const int64_t C = qsl[s + 1] - qsl[s];
      L = (int)(jb->context_lens[s] - C + (r - qsl[s]) + 1);
    } else {
      L = jb->context_lens[s];
    }
    int rc = attend_one(jb, s, r, h, L, jb->out + (size_t)it * jb->head_dim);
    if (rc != OR_OK) {
      pthread_mutex_lock(&jb->lock);
      if (jb->status == OR_OK)
        jb->status = rc;
      pthread_mutex_unlock(&jb->lock);
      return NULL;
    }
  }
  return NULL;
}

/* Runs the job's items on jb->num_threads POSIX threads; returns the first
 * error any item reported.  Every item is computed on its own, so the
 * result does not depend on the thread count. */
static int run_job(struct decode_job *jb) {
  const int num_threads = jb->num_threads;
  jb->status = OR_OK;
  pthread_mutex_init(&jb->lock, NULL);
  pthread_t *th = malloc(sizeof(pthread_t) * (size_t)num_threads);
  struct worker_arg *wa = malloc(sizeof(struct worker_arg) * (size_t)num_threads);
  if (!th || !wa) {
    free(th);
    free(wa);
    pthread_mutex_destroy(&jb->lock);
    return OR_ERR_NOMEM;
  }
  int started = 0;
  for (int t = 0; t < num_threads; ++t) {
    wa[t].jb = jb;
    wa[t].tid = t;
    if (pthread_create(&th[t], NULL, decode_worker, &wa[t]) != 0)
      break;
    ++started;
  }
  if (started == 0) { /* no thread could start: run the items here */
    wa[0].jb = jb;
    wa[0].tid = 0;
    jb->num_threads = 1;
    decode_worker(&wa[0]);
  } else if (started < num_threads) {
    /* items owned by threads that never started: run them here */
    for (int t = started; t < num_threads; ++t)
      decode_worker(&wa[t]);
  }
  for (int t = 0; t < started; ++t)
    pthread_join(th[t], NULL);
  free(th);
  free(wa);
  pthread_mutex_destroy(&jb->lock);
  return jb->status;
}

/* out: double [num_items, head_dim].  Without `sel`, the items are every
 * (s, h) in row-major order (num_items = num_seqs * num_heads) and `out` is
 * [num_seqs, num_heads, head_dim]; with `sel` (num_sel pairs of int32
 * (seq, head)), item i is pair i.  q: [num_seqs, num_heads, head_dim];
 * block_tables: [num_seqs, max_blocks_per_seq]; context_lens: [num_seqs].
 * The items are spread over `num_threads` POSIX threads; every item is
 * computed on its own, so the result does not depend on the thread count. */
/* The general form: q in q_dtype, caches in cache_dtype holding values
 * that dequantise as element * k_scale (keys) and element * v_scale
 * (values).  Attention is that of the dequantised K and V. */
int oracle_paged_decode_q(double *out, const void *q, const void *k_cache,
                          const void *v_cache, const int32_t *block_tables,
                          const int32_t *context_lens, float scale,
                          int block_size, int num_seqs, int num_heads,
                          int num_kv_heads, int head_dim, int64_t num_blocks,
                          int max_blocks_per_seq, int q_dtype, int cache_dtype,
                          float k_scale, float v_scale, const int32_t *sel,
                          int64_t num_sel, int num_threads) {
  const int dtype = cache_dtype;
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
      num_heads % num_kv_heads != 0 || head_dim <= 0 || block_size <= 0 ||
      block_size % 4 != 0 || num_blocks < 0 || max_blocks_per_seq < 0 ||
      dtype < OR_F32 || dtype > OR_FP8 || q_dtype < OR_F32 ||
      q_dtype > OR_BF16 || num_threads <= 0)
    return OR_ERR_ARG;
  struct decode_job jb;
  memset(&jb, 0, sizeof jb);
  jb.out = out;
  jb.q = q;
  jb.k_cache = k_cache;
  jb.v_cache = v_cache;
  jb.block_tables = block_tables;
  jb.context_lens = context_lens;
  jb.scale = (double)scale; /* the float argument, exactly */
  jb.block_size = block_size;
  jb.num_seqs = num_seqs;
  jb.num_heads = num_heads;
  jb.num_kv_heads = num_kv_heads;
  jb.head_dim = head_dim;
  jb.num_blocks = num_blocks;
  jb.max_blocks_per_seq = max_blocks_per_seq;
  jb.dtype = dtype;
  jb.q_dtype = q_dtype;
  jb.k_scale = (double)k_scale;
  jb.v_scale = (double)v_scale;
  jb.sel = sel;
  jb.num_items = sel ? num_sel : (int64_t)num_seqs * num_heads;
  if (sel) {
    for (int64_t i = 0; i < num_sel; ++i)
      if (sel[2 * i] < 0 || sel[2 * i] >= num_seqs || sel[2 * i + 1] < 0 ||
          sel[2 * i + 1] >= num_heads)
        return OR_ERR_ARG;
  }
  jb.num_threads = num_threads;
  return run_job(&jb);
}

/* Multi-query attention for chunked prefill: a long prompt is processed
 * in chunks ("Inside vLLM: How PagedAttention Eliminates KV-Cache Memory
 * Waste", section "Continuous Batching and Chunked Prefill"), so each
 * sequence brings a chunk of C_s new query tokens whose keys and values are
 * already in its blocks.  Query rows of sequence s are
 * query_start_loc[s] .. query_start_loc[s+1]-1 of q ([num_query_tokens,
 * num_heads, head_dim]); they are the last C_s tokens of its
 * context_lens[s] tokens, and each attends causally (see decode_worker).
 * out: double [num_query_tokens, num_heads, head_dim], or one row per
 * (query row, head) pair of `sel`.  Rejected: query_start_loc not starting
 * at 0, decreasing, not ending at num_query_tokens, or a chunk longer than
 * its context. */
int oracle_paged_prefill(double *out, const void *q, const void *k_cache,
                         const void *v_cache, const int32_t *block_tables,
                         const int32_t *context_lens,
                         const int32_t *query_start_loc, float scale,
                         int block_size, int num_seqs, int64_t num_query_tokens,
                         int num_heads, int num_kv_heads, int head_dim,
                         int64_t num_blocks, int max_blocks_per_seq,
                         int q_dtype, int cache_dtype, float k_scale,
                         float v_scale, const int32_t *sel, int64_t num_sel,
                         int num_threads) {
  const int dtype = cache_dtype;
  if (num_seqs < 0 || num_query_tokens < 0 || num_heads <= 0 ||
      num_kv_heads <= 0 || num_heads % num_kv_heads != 0 || head_dim <= 0 ||
      block_size <= 0 || block_size % 4 != 0 || num_blocks < 0 ||
      max_blocks_per_seq < 0 || dtype < OR_F32 || dtype > OR_FP8 ||
      q_dtype < OR_F32 || q_dtype > OR_BF16 || num_threads <= 0 ||
      !query_start_loc)
    return OR_ERR_ARG;
  if (query_start_loc[0] != 0 || query_start_loc[num_seqs] != num_query_tokens)
    return OR_ERR_ARG;
  for (int s = 0; s < num_seqs; ++s) {
    const int64_t C = (int64_t)query_start_loc[s + 1] - query_start_loc[s];
    if (C < 0 || C > context_lens[s])
      return OR_ERR_ARG;
  }
  if (sel) {
    for (int64_t i = 0; i < num_sel; ++i)
      if (sel[2 * i] < 0 || sel[2 * i] >= num_query_tokens ||
          sel[2 * i + 1] < 0 || sel[2 * i + 1] >= num_heads)
        return OR_ERR_ARG;
  }
  struct decode_job jb;
  memset(&jb, 0, sizeof jb);
  jb.out = out;
  jb.q = q;
  jb.k_cache = k_cache;
  jb.v_cache = v_cache;
  jb.block_tables = block_tables;
  jb.context_lens = context_lens;
  jb.query_start_loc = query_start_loc;
  jb.scale = (double)scale;
  jb.block_size = block_size;
  jb.num_seqs = num_seqs;
  jb.num_heads = num_heads;
  jb.num_kv_heads = num_kv_heads;
  jb.head_dim = head_dim;
  jb.num_blocks = num_blocks;
  jb.max_blocks_per_seq = max_blocks_per_seq;
  jb.dtype = dtype;
  jb.q_dtype = q_dtype;
  jb.k_scale = (double)k_scale;
  jb.v_scale = (double)v_scale;
  jb.sel = sel;
  jb.num_items = sel ? num_sel : num_query_tokens * num_heads;
  jb.num_threads = num_threads;
  return run_job(&jb);
}

/* q and caches of one type, no scaling. */
int oracle_paged_decode(double *out, const void *q, const void *k_cache,
                        const void *v_cache, const int32_t *block_tables,
                        const int32_t *context_lens, float scale,
                        int block_size, int num_seqs, int num_heads,
                        int num_kv_heads, int head_dim, int64_t num_blocks,
                        int max_blocks_per_seq, int dtype, const int32_t *sel,
                        int64_t num_sel, int num_threads) {
  if (dtype == OR_FP8)
    return OR_ERR_ARG;
  return oracle_paged_decode_q(out, q, k_cache, v_cache, block_tables,
                               context_lens, scale, block_size, num_seqs,
                               num_heads, num_kv_heads, head_dim, num_blocks,
                               max_blocks_per_seq, dtype, dtype, 1.0f, 1.0f,
                               sel, num_sel, num_threads);
}

/* Widen n stored elements to double with the decoders above; exported so
 * the decoders themselves can be checked against a library conversion. */
int oracle_widen(const void *src, double *dst, int64_t n, int dtype) {
  if (n < 0 || dtype < OR_F32 || dtype > OR_FP8)
    return OR_ERR_ARG;
  for (int64_t i = 0; i < n; ++i)
    dst[i] = load_elem(src, (size_t)i, dtype);
  return OR_OK;
}

/* ---- block copy (copy-on-write) ------------------------------------------ */

/* Copy-on-write at block granularity: when a block held by several
 * sequences must be written, the writer gets a fresh block holding a copy of
 * it ("Why vLLM Uses PagedAttention", section "The bonus"; "PagedAttention:
 * how vLLM manages the KV cache", section "Copy-on-write makes shared
 * prefixes practical": only the block being written is copied).
 *
 * For each pair i, block mapping[2i+1] of both pools becomes a byte copy of
 * block mapping[2i].  A block spans num_kv_heads * block_size * head_dim
 * elements in either pool, whatever the layout inside it.  Rejected (no
 * write): an index outside the pool, a destination that appears twice, or
 * a destination that is also a source. */
int oracle_copy_blocks(void *k_cache, void *v_cache, const int64_t *mapping,
                       int64_t num_pairs, int64_t num_blocks,
                       int64_t block_elems, int dtype) {
  if (num_pairs < 0 || num_blocks < 0 || block_elems <= 0 || dtype < OR_F32 ||
      dtype > OR_FP8)
    return OR_ERR_ARG;
  unsigned char *dst_seen = calloc((size_t)num_blocks + 1, 1);
  unsigned char *src_seen = calloc((size_t)num_blocks + 1, 1);
  if (!dst_seen || !src_seen) {
    free(dst_seen);
    free(src_seen);
    return OR_ERR_NOMEM;
  }
  int rc = OR_OK;
  for (int64_t i = 0; i < num_pairs && rc == OR_OK; ++i) {
    int64_t s = mapping[2 * i], d = mapping[2 * i + 1];
    if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks)
      rc = OR_ERR_TABLE;
    else if (dst_seen[d])
      rc = OR_ERR_SLOT_DUP;
    else {
      dst_seen[d] = 1;
      src_seen[s] = 1;
    }
  }
  for (int64_t i = 0; i < num_pairs && rc == OR_OK; ++i)
    if (src_seen[mapping[2 * i + 1]])
      rc = OR_ERR_SLOT_DUP;
  free(dst_seen);
  free(src_seen);
  if (rc != OR_OK)
    return rc;
  const size_t bytes = (size_t)block_elems * (size_t)elem_bytes(dtype);
  for (int64_t i = 0; i < num_pairs; ++i) {
    size_t s = (size_t)mapping[2 * i], d = (size_t)mapping[2 * i + 1];
    memcpy((char *)k_cache + d * bytes, (const char *)k_cache + s * bytes, bytes);
    memcpy((char *)v_cache + d * bytes, (const char *)v_cache + s * bytes, bytes);
  }
  return OR_OK;
}

/* Swapping: under memory pressure a request's blocks can be moved out of
 * device memory and later back, as an operating system evicts pages ("PagedAttention
 * - Virtual Memory for the KV Cache" explainer, chapter 05, card "Preemption &
 * swapping"; deep dive, card "What Indirection Buys").  For each pair i,
 * block mapping[2i+1] of the destination pools becomes a byte copy of block
 * mapping[2i] of the source pools (distinct pools).  Rejected (no write):
 * an index outside its pool, or a destination that appears twice. */
int oracle_swap_blocks(const void *src_k, const void *src_v, void *dst_k,
                       void *dst_v, const int64_t *mapping, int64_t num_pairs,
                       int64_t src_num_blocks, int64_t dst_num_blocks,
                       int64_t block_elems, int dtype) {
  if (num_pairs < 0 || src_num_blocks < 0 || dst_num_blocks < 0 ||
      block_elems <= 0 || dtype < OR_F32 || dtype > OR_FP8)
    return OR_ERR_ARG;
  unsigned char *dst_seen = calloc((size_t)dst_num_blocks + 1, 1);
  if (!dst_seen)
    return OR_ERR_NOMEM;
  int rc = OR_OK;
  for (int64_t i = 0; i < num_pairs && rc == OR_OK; ++i) {
    int64_t s = mapping[2 * i], d = mapping[2 * i + 1];
    if (s < 0 || s >= src_num_blocks || d < 0 || d >= dst_num_blocks)
      rc = OR_ERR_TABLE;
    else if (dst_seen[d])
      rc = OR_ERR_SLOT_DUP;
    else
      dst_seen[d] = 1;
  }
  free(dst_seen);
  if (rc != OR_OK)
    return rc;
  const size_t bytes = (size_t)block_elems * (size_t)elem_bytes(dtype);
  for (int64_t i = 0; i < num_pairs; ++i) {
    size_t s = (size_t)mapping[2 * i], d = (size_t)mapping[2 * i + 1];
    memcpy((char *)dst_k + d * bytes, (const char *)src_k + s * bytes, bytes);
    memcpy((char *)dst_v + d * bytes, (const char *)src_v + s * bytes, bytes);
  }
  return OR_OK;
}

/* ---- 8-bit cache ----------------------------------------------------------
 * Lower-precision cache formats reduce the bytes per element ("PagedAttention:
 * how vLLM manages the KV cache", section "Keep the tensor formula beside the
 * allocator model").  The cache write of an E4M3 cache stores, for every
 * element, e4m3_encode(x / scale) with x / scale the float quotient (IEEE
 * single precision, as the device computes it); slots and layouts are those
 * of the plain cache write. */
struct fp8_write_job {
  const void *k, *v;
  void *k_cache, *v_cache;
  const int64_t *slot_mapping;
  int64_t num_tokens;
  int num_kv_heads, head_dim, block_size, in_dtype;
  float k_scale, v_scale;
  int num_threads;
};

struct fp8_write_arg {
  struct fp8_write_job *jb;
  int tid;
};

static void *fp8_write_worker(void *argp) {
  struct fp8_write_arg *wa = argp;
  const struct fp8_write_job *jb = wa->jb;
  const size_t hkv = (size_t)jb->num_kv_heads, hd = (size_t)jb->head_dim,
               bs = (size_t)jb->block_size;
  for (int64_t i = wa->tid; i < jb->num_tokens; i += jb->num_threads) {
    int64_t s = jb->slot_mapping[i];
    if (s < 0)
      continue;
    size_t p = (size_t)(s / jb->block_size), o = (size_t)(s % jb->block_size);
    for (size_t g = 0; g < hkv; ++g) {
      for (size_t d = 0; d < hd; ++d) {
        size_t src = ((size_t)i * hkv + g) * hd + d;
        float xk = (float)load_elem(jb->k, src, jb->in_dtype);
        float xv = (float)load_elem(jb->v, src, jb->in_dtype);
        ((uint8_t *)jb->k_cache)[k_index(p, g, o, d, hkv, bs, hd)] =
            e4m3_encode(xk / jb->k_scale);
        ((uint8_t *)jb->v_cache)[v_index(p, g, o, d, hkv, bs, hd)] =
            e4m3_encode(xv / jb->v_scale);
      }
    }
  }
  return NULL;
}

int oracle_reshape_and_cache_fp8(const void *k, const void *v, void *k_cache,
                                 void *v_cache, const int64_t *slot_mapping,
                                 int64_t num_tokens, int num_kv_heads,
                                 int head_dim, int block_size,
                                 int64_t num_blocks, int in_dtype,
                                 float k_scale, float v_scale,
                                 int num_threads) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      block_size % 4 != 0 || num_blocks < 0 || in_dtype < OR_F32 ||
      in_dtype > OR_BF16)
    return OR_ERR_ARG;
  const int64_t nslots = num_blocks * (int64_t)block_size;
  unsigned char *seen = calloc((size_t)(nslots / 8 + 1), 1);
  if (!seen)
    return OR_ERR_NOMEM;
  for (int64_t i = 0; i < num_tokens; ++i) {
    int64_t s = slot_mapping[i];
    if (s < 0)
      continue;
    if (s >= nslots || (seen[s / 8] & (1u << (s % 8)))) {
      free(seen);
      return s >= nslots ? OR_ERR_SLOT_RANGE : OR_ERR_SLOT_DUP;
    }
    seen[s / 8] |= (unsigned char)(1u << (s % 8));
  }
  free(seen);
  struct fp8_write_job jb = {k, v, k_cache, v_cache, slot_mapping, num_tokens,
                             num_kv_heads, head_dim, block_size, in_dtype,
                             k_scale, v_scale, num_threads};
  /* the slots are distinct (checked above), so threads that take disjoint
   * tokens write disjoint bytes */
  pthread_t th[64];
  struct fp8_write_arg wa[64];
  int nt = num_threads < 1 ? 1 : (num_threads > 64 ? 64 : num_threads);
  jb.num_threads = nt;
  int started = 0;
  for (int t = 0; t < nt; ++t) {
    wa[t].jb = &jb;
    wa[t].tid = t;
    if (pthread_create(&th[t], NULL, fp8_write_worker, &wa[t]) != 0)
      break;
    ++started;
  }
  for (int t = started; t < nt; ++t) /* threads that never started */
    fp8_write_worker(&wa[t]);
  for (int t = 0; t < started; ++t)
    pthread_join(th[t], NULL);
  return OR_OK;
}

/* Element-wise encoding, exported so it can be checked on its own. */
int oracle_e4m3_encode(const float *src, uint8_t *dst, int64_t n) {
  if (n < 0)
    return OR_ERR_ARG;
  for (int64_t i = 0; i < n; ++i)
    dst[i] = e4m3_encode(src[i]);
  return OR_OK;
}
