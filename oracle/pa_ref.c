/*
 * pa_ref.c — CPU oracle (fp64) for paged-attention decode.  TEST INFRASTRUCTURE ONLY.
 * What each function follows is stated in pa_ref.h; this file is plain C99 + pthreads.
 *
 * Parity pins (tests/test_oracle_*.py): the pages' block-table example, dense attention
 * (a separate routine fed with unpaged keys), torch's scaled_dot_product_attention in
 * fp64, closed forms, physical-block permutation and prefix-sharing invariances, the
 * partition merge, and NaN poison in every slot the method must not read.
 */
#define _GNU_SOURCE
#include "pa_ref.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

static int elem_bytes(int32_t dtype) {
  return dtype == PA_REF_F32 ? 4 : dtype == PA_REF_FP8_E4M3 ? 1 : 2;
}

/* element type of q, key and value */
static int32_t q_type(const pa_ref_geom* g) { return g->q_dtype >= 0 ? g->q_dtype : g->dtype; }

/* ---------------------------------------------------------------- FP8 E4M3 */

double pa_ref_fp8_decode(uint8_t code) {
  const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9); /* subnormal: m/8 * 2^(1-7) */
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -v : v;
}

uint8_t pa_ref_fp8_encode(float x) {
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return sign | 0x7F;
  const double a = fabs((double)x);
  if (a >= 448.0) return sign | 0x7E; /* saturate at the largest finite value */
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: multiples of 2^-9; nearbyint rounds half to even (default mode).
     * m = 8 is the smallest normal number, whose code is 0x08 as well. */
    return sign | (uint8_t)nearbyint(a * 512.0);
  }
  int e;
  const double fr = frexp(a, &e); /* a = fr * 2^e, fr in [0.5, 1) */
  const int E = e - 1;            /* a = (2 fr) * 2^E, 2 fr in [1, 2), E in [-6, 8] */
  const int q = (int)nearbyint((2.0 * fr - 1.0) * 8.0); /* 3 fraction bits, 0..8 */
  return sign | (uint8_t)(((E + 7) << 3) + q);          /* q = 8 carries into the exponent */
}

/* ---------------------------------------------------------------- element conversion */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double f16_bits_to_double(uint16_t h) {
  int sign = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(m | 0x400), e - 25); /* (1.m) * 2^(e-15) = (1024+m) * 2^(e-25) */
  return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double bf16_bits_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double load_elem(const void* base, int32_t dtype, int64_t idx) {
  if (dtype == PA_REF_F32) {
    float f;
    memcpy(&f, (const char*)base + 4 * idx, 4);
    return (double)f;
  }
  if (dtype == PA_REF_FP8_E4M3) return pa_ref_fp8_decode(((const uint8_t*)base)[idx]);
  uint16_t h;
  memcpy(&h, (const char*)base + 2 * idx, 2);
  return dtype == PA_REF_F16 ? f16_bits_to_double(h) : bf16_bits_to_double(h);
}

void pa_ref_to_double(const void* src, int32_t dtype, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = load_elem(src, dtype, i);
}

/* ---------------------------------------------------------------- pool layout */

/* A block of block_size tokens is R sub-blocks of T tokens (T = block_size up to 16, else 16;
 * R = block_size / T), each holding every KV head: K [NB][R][Hkv][D/X][T][X],
 * V [NB][R][Hkv][D][T].  For block_size 16 (R = 1) this is [NB][Hkv][D/X][16][X] and
 * [NB][Hkv][D][16]. */
static int32_t sub_tokens(const pa_ref_geom* g) { return g->block_size < 16 ? g->block_size : 16; }

int64_t pa_ref_k_offset(const pa_ref_geom* g, int64_t block, int32_t kv_head, int32_t token,
                        int32_t dim) {
  const int64_t x = 16 / elem_bytes(g->dtype);
  const int64_t chunks = g->head_dim / x;
  const int32_t T = sub_tokens(g), R = g->block_size / T;
  const int64_t sub = block * R + token / T; /* sub-block index in the pool */
  return (((sub * g->num_kv_heads + kv_head) * chunks + dim / x) * T + token % T) * x + dim % x;
}

int64_t pa_ref_v_offset(const pa_ref_geom* g, int64_t block, int32_t kv_head, int32_t token,
                        int32_t dim) {
  const int32_t T = sub_tokens(g), R = g->block_size / T;
  const int64_t sub = block * R + token / T;
  return ((sub * g->num_kv_heads + kv_head) * (int64_t)g->head_dim + dim) * T + token % T;
}

static int geom_ok(const pa_ref_geom* g) {
  if (!g || g->num_seqs < 0 || g->num_q_heads <= 0 || g->num_kv_heads <= 0 || g->head_dim <= 0 ||
      g->block_size <= 0 || g->num_blocks <= 0 || g->max_blocks_per_seq < 0)
    return 0;
  if (g->dtype < PA_REF_F32 || g->dtype > PA_REF_FP8_E4M3) return 0;
  if (g->q_dtype >= 0 && g->q_dtype != g->dtype && g->dtype != PA_REF_FP8_E4M3) return 0;
  if (g->dtype == PA_REF_FP8_E4M3 && (q_type(g) < PA_REF_F32 || q_type(g) > PA_REF_BF16)) return 0;
  if (g->dtype == PA_REF_FP8_E4M3 && !(g->k_scale > 0.0 && g->v_scale > 0.0)) return 0;
  if (g->num_q_heads % g->num_kv_heads) return 0;
  if (g->head_dim % (16 / elem_bytes(g->dtype))) return 0;
  if (g->block_size > 16 && g->block_size % 16) return 0;
  return 1;
}

/* ---------------------------------------------------------------- reshape_and_cache */

int32_t pa_ref_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                 const int64_t* slot_mapping, int64_t num_tokens,
                                 const pa_ref_geom* g) {
  if (!geom_ok(g) || num_tokens < 0) return -1;
  const int e = elem_bytes(g->dtype);
  const int64_t pool_slots = (int64_t)g->num_blocks * g->block_size;
  for (int64_t i = 0; i < num_tokens; ++i) {
    const int64_t slot = slot_mapping[i];
    if (slot < 0) continue; /* padding token */
    if (slot >= pool_slots) return -1;
    const int64_t block = slot / g->block_size;
    const int32_t offset = (int32_t)(slot % g->block_size);
    for (int32_t h = 0; h < g->num_kv_heads; ++h) {
      for (int32_t d = 0; d < g->head_dim; ++d) {
        const int64_t src = (i * g->num_kv_heads + h) * (int64_t)g->head_dim + d;
        const int64_t ko = pa_ref_k_offset(g, block, h, offset, d);
        const int64_t vo = pa_ref_v_offset(g, block, h, offset, d);
        if (g->dtype == PA_REF_FP8_E4M3) {
          /* quantise: the fp32 quotient by the pool's scale, rounded to E4M3 */
          const float kq = (float)load_elem(key, q_type(g), src) / (float)g->k_scale;
          const float vq = (float)load_elem(value, q_type(g), src) / (float)g->v_scale;
          ((uint8_t*)k_cache)[ko] = pa_ref_fp8_encode(kq);
          ((uint8_t*)v_cache)[vo] = pa_ref_fp8_encode(vq);
        } else {
          memcpy((char*)k_cache + e * ko, (const char*)key + e * src, e);
          memcpy((char*)v_cache + e * vo, (const char*)value + e * src, e);
        }
      }
    }
  }
  return 0;
}

/* ---------------------------------------------------------------- copy-on-write block copy */

int32_t pa_ref_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping,
                           int64_t num_pairs, const pa_ref_geom* g) {
  if (!geom_ok(g) || num_pairs < 0) return -1;
  const int e = elem_bytes(g->dtype);
  for (int64_t p = 0; p < num_pairs; ++p) {
    const int64_t src = block_mapping[2 * p], dst = block_mapping[2 * p + 1];
    if (src < 0 || src >= g->num_blocks || dst < 0 || dst >= g->num_blocks) continue;
    for (int32_t h = 0; h < g->num_kv_heads; ++h)
      for (int32_t t = 0; t < g->block_size; ++t)
        for (int32_t d = 0; d < g->head_dim; ++d) {
          memcpy((char*)k_cache + e * pa_ref_k_offset(g, dst, h, t, d),
                 (const char*)k_cache + e * pa_ref_k_offset(g, src, h, t, d), e);
          memcpy((char*)v_cache + e * pa_ref_v_offset(g, dst, h, t, d),
                 (const char*)v_cache + e * pa_ref_v_offset(g, src, h, t, d), e);
        }
  }
  return 0;
}

/* ---------------------------------------------------------------- swap to / from host */

int32_t pa_ref_swap_blocks(void* dst_k, void* dst_v, int64_t dst_num_blocks, const void* src_k,
                           const void* src_v, int64_t src_num_blocks,
                           const int64_t* block_mapping, int64_t num_pairs,
                           const pa_ref_geom* g) {
  if (!geom_ok(g) || num_pairs < 0 || dst_num_blocks < 0 || src_num_blocks < 0) return -1;
  for (int64_t p = 0; p < num_pairs; ++p) {
    const int64_t src = block_mapping[2 * p], dst = block_mapping[2 * p + 1];
    if (src < 0 || src >= src_num_blocks || dst < 0 || dst >= dst_num_blocks) return -1;
  }
  const int e = elem_bytes(g->dtype);
  for (int64_t p = 0; p < num_pairs; ++p) {
    const int64_t src = block_mapping[2 * p], dst = block_mapping[2 * p + 1];
    for (int32_t h = 0; h < g->num_kv_heads; ++h)
      for (int32_t t = 0; t < g->block_size; ++t)
        for (int32_t d = 0; d < g->head_dim; ++d) {
          memcpy((char*)dst_k + e * pa_ref_k_offset(g, dst, h, t, d),
                 (const char*)src_k + e * pa_ref_k_offset(g, src, h, t, d), e);
          memcpy((char*)dst_v + e * pa_ref_v_offset(g, dst, h, t, d),
                 (const char*)src_v + e * pa_ref_v_offset(g, src, h, t, d), e);
        }
  }
  return 0;
}

/* ---------------------------------------------------------------- row bookkeeping */

typedef struct {
  int32_t seq;      /* sequence the row belongs to */
  int32_t last_key; /* highest visible key position (-1: no keys) */
} row_info;

static int find_row(const int32_t* context_lens, const int32_t* qsl, int32_t num_seqs,
                    int32_t num_q_rows, int32_t r, row_info* out) {
  if (r < 0 || r >= num_q_rows) return -1;
  int32_t s, n, j;
  if (qsl == NULL) {
    if (r >= num_seqs) return -1;
    s = r;
    n = 1;
    j = 0;
  } else {
    s = -1;
    for (int32_t t = 0; t < num_seqs; ++t)
      if (qsl[t] <= r && r < qsl[t + 1]) {
        s = t;
        break;
      }
    if (s < 0) return -1;
    n = qsl[s + 1] - qsl[s];
    j = r - qsl[s];
  }
  const int32_t ctx = context_lens[s];
  if (ctx < 0) return -1;
  out->seq = s;
  /* The n rows of this step are the last n positions of the context: row j sits at
   * ctx - n + j and sees keys [0, ctx - n + j].  A negative position sees no key. */
  out->last_key = ctx - n + j;
  return 0;
}

/* Keys [t0, t1) of sequence s, KV head kvh: scores x[t - t0] = scale * q . k_t. */
static void scores(double* x, const double* qv, const void* k_cache, const int32_t* bt_row,
                   int32_t kvh, int32_t t0, int32_t t1, double scale, const pa_ref_geom* g) {
  const double kscale = g->dtype == PA_REF_FP8_E4M3 ? g->k_scale : 1.0;
  for (int32_t t = t0; t < t1; ++t) {
    const int64_t block = bt_row[t / g->block_size]; /* logical block -> physical block */
    const int32_t off = t % g->block_size;
    double dot = 0.0;
    for (int32_t d = 0; d < g->head_dim; ++d)
      dot += qv[d] * (load_elem(k_cache, g->dtype, pa_ref_k_offset(g, block, kvh, off, d)) *
                      kscale);
    x[t - t0] = scale * dot;
  }
}

/* Softmax over x[0..n) (max-subtracted, two passes) and the weighted sum of V rows. */
static void softmax_v(double* out, double* m_out, double* l_out, const double* x, double* w,
                      const void* v_cache, const int32_t* bt_row, int32_t kvh, int32_t t0,
                      int32_t n, const pa_ref_geom* g) {
  const int32_t D = g->head_dim;
  const double vscale = g->dtype == PA_REF_FP8_E4M3 ? g->v_scale : 1.0;
  for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
  if (n <= 0) {
    *m_out = -INFINITY;
    *l_out = 0.0;
    return;
  }
  double m = x[0];
  for (int32_t i = 1; i < n; ++i)
    if (x[i] > m) m = x[i];
  double l = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    w[i] = exp(x[i] - m);
    l += w[i];
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t t = t0 + i;
    const int64_t block = bt_row[t / g->block_size];
    const int32_t off = t % g->block_size;
    for (int32_t d = 0; d < D; ++d)
      out[d] += w[i] * (load_elem(v_cache, g->dtype, pa_ref_v_offset(g, block, kvh, off, d)) *
                        vscale);
  }
  for (int32_t d = 0; d < D; ++d) out[d] /= l;
  *m_out = m;
  *l_out = l;
}

/* ---------------------------------------------------------------- threaded driver */

typedef struct {
  /* inputs */
  const void *q, *k_cache, *v_cache;
  const int32_t *block_tables, *context_lens, *qsl, *rows;
  int32_t num_q_rows, num_sel;
  double scale;
  const pa_ref_geom* g;
  int32_t partition_size, max_partitions; /* partition_size <= 0: whole context */
  /* outputs */
  double *out, *lse, *o_part, *m_part, *l_part;
  /* work split */
  int32_t tid, nthreads;
  int32_t status;
} job;

static void* run_job(void* arg) {
  job* J = (job*)arg;
  const pa_ref_geom* g = J->g;
  const int32_t D = g->head_dim, Hq = g->num_q_heads, grp = g->num_q_heads / g->num_kv_heads;
  const int32_t max_keys = g->max_blocks_per_seq * g->block_size;
  double* qv = (double*)malloc(sizeof(double) * D);
  double* x = (double*)malloc(sizeof(double) * (max_keys > 0 ? max_keys : 1));
  double* w = (double*)malloc(sizeof(double) * (max_keys > 0 ? max_keys : 1));
  J->status = 0;
  /* work item = (selected row k, query head h), interleaved over threads */
  const int64_t items = (int64_t)J->num_sel * Hq;
  for (int64_t it = J->tid; it < items; it += J->nthreads) {
    const int32_t k = (int32_t)(it / Hq), h = (int32_t)(it % Hq);
    const int32_t r = J->rows ? J->rows[k] : k;
    row_info ri;
    if (find_row(J->context_lens, J->qsl, g->num_seqs, J->num_q_rows, r, &ri) ||
        ri.last_key >= max_keys) { /* a context longer than its block-table row */
      J->status = -1;
      break;
    }
    const int32_t* bt_row = J->block_tables + (int64_t)ri.seq * g->max_blocks_per_seq;
    const int32_t kvh = h / grp; /* GQA: contiguous groups of query heads share a KV head */
    for (int32_t d = 0; d < D; ++d)
      qv[d] = load_elem(J->q, q_type(g), ((int64_t)r * Hq + h) * D + d);
    const int32_t nkeys = ri.last_key >= 0 ? ri.last_key + 1 : 0;
    if (J->partition_size <= 0) {
      double m, l;
      double* o = J->out + ((int64_t)k * Hq + h) * D;
      scores(x, qv, J->k_cache, bt_row, kvh, 0, nkeys, J->scale, g);
      softmax_v(o, &m, &l, x, w, J->v_cache, bt_row, kvh, 0, nkeys, g);
      if (J->lse) J->lse[(int64_t)k * Hq + h] = nkeys > 0 ? m + log(l) : -INFINITY;
    } else {
      const int32_t P = J->max_partitions, ps = J->partition_size;
      if ((int64_t)(nkeys + ps - 1) / ps > P) {
        J->status = -1;
        break;
      }
      for (int32_t p = 0; p < P; ++p) {
        const int64_t pi = ((int64_t)k * Hq + h) * P + p;
        const int32_t t0 = p * ps;
        const int32_t t1 = t0 + ps < nkeys ? t0 + ps : nkeys;
        const int32_t n = t1 > t0 ? t1 - t0 : 0;
        if (n > 0) scores(x, qv, J->k_cache, bt_row, kvh, t0, t1, J->scale, g);
        softmax_v(J->o_part + pi * D, &J->m_part[pi], &J->l_part[pi], x, w, J->v_cache, bt_row,
                  kvh, t0, n, g);
      }
    }
  }
  free(qv);
  free(x);
  free(w);
  return NULL;
}

static int32_t run_all(job* proto, int32_t num_threads) {
  if (num_threads <= 0) num_threads = (int32_t)sysconf(_SC_NPROCESSORS_ONLN);
  if (num_threads < 1) num_threads = 1;
  if (num_threads > 256) num_threads = 256;
  job* jobs = (job*)malloc(sizeof(job) * num_threads);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * num_threads);
  for (int32_t t = 0; t < num_threads; ++t) {
    jobs[t] = *proto;
    jobs[t].tid = t;
    jobs[t].nthreads = num_threads;
  }
  for (int32_t t = 1; t < num_threads; ++t) pthread_create(&th[t], NULL, run_job, &jobs[t]);
  run_job(&jobs[0]);
  int32_t status = jobs[0].status;
  for (int32_t t = 1; t < num_threads; ++t) {
    pthread_join(th[t], NULL);
    if (jobs[t].status) status = jobs[t].status;
  }
  free(jobs);
  free(th);
  return status;
}

int32_t pa_ref_paged_attention(double* out, double* lse, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* context_lens, const int32_t* query_start_loc,
                               int32_t num_q_rows, double scale, const pa_ref_geom* g,
                               const int32_t* rows, int32_t num_rows, int32_t num_threads) {
  if (!geom_ok(g) || !out || num_q_rows < 0) return -1;
  job J;
  memset(&J, 0, sizeof(J));
  J.q = q;
  J.k_cache = k_cache;
  J.v_cache = v_cache;
  J.block_tables = block_tables;
  J.context_lens = context_lens;
  J.qsl = query_start_loc;
  J.rows = rows;
  J.num_q_rows = num_q_rows;
  J.num_sel = rows ? num_rows : num_q_rows;
  J.scale = scale;
  J.g = g;
  J.out = out;
  J.lse = lse;
  return run_all(&J, num_threads);
}

int32_t pa_ref_partition_attention(double* o_part, double* m_part, double* l_part, const void* q,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   const int32_t* query_start_loc, int32_t num_q_rows,
                                   double scale, int32_t partition_size, int32_t max_partitions,
                                   const pa_ref_geom* g, const int32_t* rows, int32_t num_rows,
                                   int32_t num_threads) {
  if (!geom_ok(g) || partition_size <= 0 || max_partitions <= 0 || num_q_rows < 0) return -1;
  job J;
  memset(&J, 0, sizeof(J));
  J.q = q;
  J.k_cache = k_cache;
  J.v_cache = v_cache;
  J.block_tables = block_tables;
  J.context_lens = context_lens;
  J.qsl = query_start_loc;
  J.rows = rows;
  J.num_q_rows = num_q_rows;
  J.num_sel = rows ? num_rows : num_q_rows;
  J.scale = scale;
  J.g = g;
  J.partition_size = partition_size;
  J.max_partitions = max_partitions;
  J.o_part = o_part;
  J.m_part = m_part;
  J.l_part = l_part;
  return run_all(&J, num_threads);
}

/* ---------------------------------------------------------------- partition merge */

void pa_ref_merge_partitions(double* out, double* lse, const double* o_part, const double* m_part,
                             const double* l_part, int64_t num_items, int32_t head_dim,
                             int32_t max_partitions) {
  const int32_t D = head_dim, P = max_partitions;
  for (int64_t i = 0; i < num_items; ++i) {
    const double* m = m_part + i * P;
    const double* l = l_part + i * P;
    double* o = out + i * D;
    double M = -INFINITY;
    for (int32_t p = 0; p < P; ++p)
      if (l[p] > 0.0 && m[p] > M) M = m[p];
    for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
    if (M == -INFINITY) { /* no keys at all */
      if (lse) lse[i] = -INFINITY;
      continue;
    }
    double L = 0.0;
    for (int32_t p = 0; p < P; ++p) {
      if (!(l[p] > 0.0)) continue;
      const double wp = l[p] * exp(m[p] - M); /* partition weight relative to the global max */
      L += wp;
      for (int32_t d = 0; d < D; ++d) o[d] += wp * o_part[(i * P + p) * D + d];
    }
    for (int32_t d = 0; d < D; ++d) o[d] /= L;
    if (lse) lse[i] = M + log(L);
  }
}

/* ---------------------------------------------------------------- dense attention */

void pa_ref_dense_attention(double* out, double* lse, const double* q, const double* k,
                            const double* v, int32_t n, int32_t d, double scale) {
  for (int32_t j = 0; j < d; ++j) out[j] = 0.0;
  if (n <= 0) {
    if (lse) *lse = -INFINITY;
    return;
  }
  double* x = (double*)malloc(sizeof(double) * n);
  for (int32_t i = 0; i < n; ++i) {
    double dot = 0.0;
    for (int32_t j = 0; j < d; ++j) dot += q[j] * k[(int64_t)i * d + j];
    x[i] = scale * dot;
  }
  double m = x[0];
  for (int32_t i = 1; i < n; ++i)
    if (x[i] > m) m = x[i];
  double l = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    x[i] = exp(x[i] - m);
    l += x[i];
  }
  for (int32_t i = 0; i < n; ++i)
    for (int32_t j = 0; j < d; ++j) out[j] += x[i] * v[(int64_t)i * d + j];
  for (int32_t j = 0; j < d; ++j) out[j] /= l;
  if (lse) *lse = m + log(l);
  free(x);
}
