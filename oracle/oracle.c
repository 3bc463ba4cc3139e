/*
 * fp64 CPU oracle for speculative-decoding verify attention.
 *
 * TEST INFRASTRUCTURE (see oracle.h): only tests/, __graft_entry__.smoke() and
 * bench.py's cpu_baseline leg use it.  Plain loops in the order the definition
 * states them; the only parallelism is a pthread split over independent
 * (row, head) outputs so it can be timed on many cores.  No blocking, no
 * fusion, no reordering of any sum.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define ORC_PAGE 16

/* ---- scalar decoders (IEEE binary16 / bfloat16 bit patterns -> double) ---- */

static double f16_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = ldexp((double)(m + 1024), e - 25); /* (1 + m/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double load_q(const orc_shape* p, const void* q, int64_t idx) {
  switch (p->q_dtype) {
    case ORC_F32: return (double)((const float*)q)[idx];
    case ORC_F16: return f16_to_double(((const uint16_t*)q)[idx]);
    default: return bf16_to_double(((const uint16_t*)q)[idx]);
  }
}

/* ---- validation ---- */

static int check_shape(const orc_shape* p) {
  if (p->num_seqs < 1 || p->B < 1 || p->H < 1 || p->KVH < 1 || p->D < 1) return ORC_EINVAL;
  if (p->H % p->KVH) return ORC_EINVAL;
  if (p->kv_dtype == ORC_Q8 && p->D % 32) return ORC_EINVAL;
  if (p->q_dtype != ORC_F32 && p->q_dtype != ORC_F16 && p->q_dtype != ORC_BF16) return ORC_EINVAL;
  if (p->kv_dtype != ORC_F32 && p->kv_dtype != ORC_F16 && p->kv_dtype != ORC_Q8) return ORC_EINVAL;
  return ORC_OK;
}

/* Sequence s has n query rows; par_s (NULL = chain) is its slice of parent. */
static int check_seq(const orc_shape* p, const int32_t* bt, const int32_t* ctx_lens,
                     const int32_t* par_s, int n, int s) {
  int ctx = ctx_lens[s];
  if (ctx < n || ctx > p->max_pages * ORC_PAGE) return ORC_EINVAL;
  for (int pg = 0; pg < (ctx + ORC_PAGE - 1) / ORC_PAGE; ++pg) {
    int id = bt[(int64_t)s * p->max_pages + pg];
    if (id < 0 || id >= p->num_pages) return ORC_EINVAL;
  }
  if (par_s) {
    for (int i = 0; i < n; ++i) {
      int par = par_s[i];
      if (par < -1 || par >= i) return ORC_EINVAL;
    }
  }
  return ORC_OK;
}

/* Rows of sequence s: count n and first packed row row0.  Without cu_rows
 * every sequence has B rows; with it, rows cu_rows[s] .. cu_rows[s+1]. */
static void seq_rows(const orc_shape* p, const int32_t* cu_rows, int s, int* n, int64_t* row0) {
  if (cu_rows) {
    *row0 = cu_rows[s];
    *n = cu_rows[s + 1] - cu_rows[s];
  } else {
    *row0 = (int64_t)s * p->B;
    *n = p->B;
  }
}

/* anc[i*n + a] = 1 iff in-window row a is row i or one of its ancestors. */
static void build_ancestry(const int32_t* par_s, int n, unsigned char* anc) {
  memset(anc, 0, (size_t)n * n);
  for (int i = 0; i < n; ++i) {
    int a = i;
    while (a >= 0) {
      anc[(int64_t)i * n + a] = 1;
      a = par_s ? par_s[a] : a - 1;
    }
  }
}

/* ---- K / V gather and decode for one (sequence, KV head) ---- */

static void decode_seq_kv(const orc_shape* p, const void* k_pool, const void* v_pool,
                          const uint16_t* k_scale, const uint16_t* v_scale, const int32_t* bt,
                          int s, int g, int ctx, double* K, double* V) {
  const int D = p->D, KVH = p->KVH;
  for (int j = 0; j < ctx; ++j) {
    int64_t page = bt[(int64_t)s * p->max_pages + j / ORC_PAGE];
    int slot = j % ORC_PAGE;
    int64_t krow = ((page * KVH + g) * ORC_PAGE + slot) * D;   /* k_pool[page][g][slot][:] */
    int64_t vbase = (page * KVH + g) * (int64_t)D * ORC_PAGE;  /* v_pool[page][g][:][:]    */
    for (int d = 0; d < D; ++d) {
      int64_t vidx = vbase + (int64_t)d * ORC_PAGE + slot;     /* v_pool[page][g][d][slot] */
      double kx, vx;
      if (p->kv_dtype == ORC_Q8) {
        int8_t kq = ((const int8_t*)k_pool)[krow + d];
        int8_t vq = ((const int8_t*)v_pool)[vidx];
        /* k_scale[page][g][slot][d/32], v_scale[page][g][d/32][slot] */
        double kd = f16_to_double(k_scale[((page * KVH + g) * ORC_PAGE + slot) * (D / 32) + d / 32]);
        double vd = f16_to_double(v_scale[((page * KVH + g) * (D / 32) + d / 32) * ORC_PAGE + slot]);
        kx = kd * (double)kq;
        vx = vd * (double)vq;
      } else if (p->kv_dtype == ORC_F16) {
        kx = f16_to_double(((const uint16_t*)k_pool)[krow + d]);
        vx = f16_to_double(((const uint16_t*)v_pool)[vidx]);
      } else {
        kx = (double)((const float*)k_pool)[krow + d];
        vx = (double)((const float*)v_pool)[vidx];
      }
      K[(int64_t)j * D + d] = kx;
      V[(int64_t)j * D + d] = vx;
    }
  }
}

/* ---- one (row, head): definition or one split of the split form ---- */

typedef struct {
  const orc_shape* p;
  const void* q;
  const double* K;
  const double* V;
  const unsigned char* anc;
  int s, ctx;
  int n;       /* query rows of this sequence; they sit at slots ctx - n + i */
  int64_t row0; /* packed index of its row 0 in q / out */
} seq_ctx;

static int visible(const seq_ctx* c, int i, int j) {
  int base = c->ctx - c->n;
  if (j < base) return 1;
  return c->anc[(int64_t)i * c->n + (j - base)];
}

static double score(const seq_ctx* c, int i, int h, int j) {
  const orc_shape* p = c->p;
  int64_t qrow = ((c->row0 + i) * p->H + h) * p->D;
  double acc = 0.0;
  for (int d = 0; d < p->D; ++d) acc += load_q(p, c->q, qrow + d) * c->K[(int64_t)j * p->D + d];
  return p->scale * acc;
}

/* Definition: O and lse over all of Vis(i). */
static void attend_direct(const seq_ctx* c, int i, int h, double* z, double* o, double* lse) {
  const int D = c->p->D;
  double M = -INFINITY;
  for (int j = 0; j < c->ctx; ++j) {
    if (!visible(c, i, j)) continue;
    z[j] = score(c, i, h, j);
    if (z[j] > M) M = z[j];
  }
  double L = 0.0;
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  for (int j = 0; j < c->ctx; ++j) {
    if (!visible(c, i, j)) continue;
    double w = exp(z[j] - M);
    L += w;
    for (int d = 0; d < D; ++d) o[d] += w * c->V[(int64_t)j * D + d];
  }
  for (int d = 0; d < D; ++d) o[d] /= L;
  *lse = M + log(L);
}

/* One split [lo, hi): unnormalised (m, l, O). */
static void attend_split(const seq_ctx* c, int i, int h, int lo, int hi, double* z, double* m,
                         double* l, double* o) {
  const int D = c->p->D;
  double mk = -INFINITY;
  for (int j = lo; j < hi; ++j) {
    if (!visible(c, i, j)) continue;
    z[j] = score(c, i, h, j);
    if (z[j] > mk) mk = z[j];
  }
  double lk = 0.0;
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  if (mk != -INFINITY) {
    for (int j = lo; j < hi; ++j) {
      if (!visible(c, i, j)) continue;
      double w = exp(z[j] - mk);
      lk += w;
      for (int d = 0; d < D; ++d) o[d] += w * c->V[(int64_t)j * D + d];
    }
  }
  *m = mk;
  *l = lk;
}

/* ---- threading over (row, head) work items of one sequence / KV head ---- */

typedef struct {
  const seq_ctx* c;
  int mode; /* 0 direct into full arrays, 1 split partials, 2 direct into item arrays */
  int g, G;
  int n_work;
  const int32_t* work; /* pairs (i, h) */
  const int32_t* item_index; /* mode 2: destination index per work item */
  int tid, nthreads;
  /* outputs */
  double* out;
  double* lse;
  int nsplit;
  const int32_t* bounds;
  double* m;
  double* l;
  double* o;
  int64_t nrows_total;
} job;

static void* run_job(void* arg) {
  job* jb = (job*)arg;
  const seq_ctx* c = jb->c;
  const orc_shape* p = c->p;
  double* z = (double*)malloc(sizeof(double) * (size_t)(c->ctx > 0 ? c->ctx : 1));
  for (int w = jb->tid; w < jb->n_work; w += jb->nthreads) {
    int i = jb->work[2 * w], h = jb->work[2 * w + 1];
    int64_t row = (c->row0 + i) * p->H + h; /* (packed row, head) */
    if (jb->mode == 0) {
      attend_direct(c, i, h, z, jb->out + row * p->D, jb->lse + row);
    } else if (jb->mode == 2) {
      int64_t dst = jb->item_index[w];
      attend_direct(c, i, h, z, jb->out + dst * p->D, jb->lse + dst);
    } else {
      const int32_t* b = jb->bounds + (int64_t)c->s * (jb->nsplit + 1);
      for (int k = 0; k < jb->nsplit; ++k) {
        int64_t r = (int64_t)k * jb->nrows_total + row;
        attend_split(c, i, h, b[k], b[k + 1], z, jb->m + r, jb->l + r, jb->o + r * p->D);
      }
    }
  }
  free(z);
  return NULL;
}

static void run_parallel(job* proto, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  job jobs[256];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = *proto;
    jobs[t].tid = t;
    jobs[t].nthreads = nthreads;
  }
  int started = 0;
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, run_job, &jobs[t]) != 0) break;
    started = t;
  }
  run_job(&jobs[0]);
  for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
  /* any thread that failed to start: run its share here */
  for (int t = started + 1; t < nthreads; ++t) run_job(&jobs[t]);
}

/* Shared driver: for every sequence and KV head, decode K/V, then evaluate the
 * requested (row, head) items. */
static int drive(const orc_shape* p, const void* q, const void* k_pool, const void* v_pool,
                 const uint16_t* k_scale, const uint16_t* v_scale, const int32_t* bt,
                 const int32_t* ctx_lens, const int32_t* parent, const int32_t* cu_rows, int mode,
                 int32_t n_items, const int32_t* items, double* out, double* lse, int32_t nsplit,
                 const int32_t* bounds, double* m, double* l, double* o, int nthreads) {
  if (check_shape(p) != ORC_OK) return ORC_EINVAL;
  if (p->kv_dtype == ORC_Q8 && (!k_scale || !v_scale)) return ORC_EINVAL;
  if (cu_rows) {
    if (cu_rows[0] != 0) return ORC_EINVAL;
    for (int s = 0; s < p->num_seqs; ++s)
      if (cu_rows[s + 1] < cu_rows[s]) return ORC_EINVAL;
  }
  int n_max = 0;
  int64_t total_rows = 0;
  for (int s = 0; s < p->num_seqs; ++s) {
    int n;
    int64_t row0;
    seq_rows(p, cu_rows, s, &n, &row0);
    if (check_seq(p, bt, ctx_lens, parent ? parent + row0 : NULL, n, s) != ORC_OK) return ORC_EINVAL;
    if (n > n_max) n_max = n;
    total_rows = row0 + n;
  }
  if (mode == 1) {
    if (nsplit < 1) return ORC_EINVAL;
    for (int s = 0; s < p->num_seqs; ++s) {
      const int32_t* b = bounds + (int64_t)s * (nsplit + 1);
      if (b[0] != 0 || b[nsplit] != ctx_lens[s]) return ORC_EINVAL;
      for (int k = 0; k < nsplit; ++k)
        if (b[k + 1] < b[k]) return ORC_EINVAL;
    }
  }
  if (mode == 2) {
    for (int t = 0; t < n_items; ++t) {
      int s = items[3 * t], i = items[3 * t + 1], h = items[3 * t + 2];
      if (s < 0 || s >= p->num_seqs || h < 0 || h >= p->H) return ORC_EINVAL;
      int n;
      int64_t row0;
      seq_rows(p, cu_rows, s, &n, &row0);
      if (i < 0 || i >= n) return ORC_EINVAL;
    }
  }

  const int G = p->H / p->KVH;
  const int64_t nrows_total = total_rows * p->H;
  const int64_t n_anc = n_max > 0 ? (int64_t)n_max * n_max : 1;
  unsigned char* anc = (unsigned char*)malloc((size_t)n_anc);
  int32_t* work = (int32_t*)malloc(sizeof(int32_t) * 2 * (size_t)(n_max * G > n_items ? n_max * G : n_items + 1));
  int32_t* widx = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_items + 1));
  if (!anc || !work || !widx) {
    free(anc); free(work); free(widx);
    return ORC_EINVAL;
  }
  int rc = ORC_OK;
  for (int s = 0; s < p->num_seqs && rc == ORC_OK; ++s) {
    int ctx = ctx_lens[s];
    int n;
    int64_t row0;
    seq_rows(p, cu_rows, s, &n, &row0);
    build_ancestry(parent ? parent + row0 : NULL, n, anc);
    for (int g = 0; g < p->KVH; ++g) {
      int n_work = 0;
      if (mode == 2) {
        for (int t = 0; t < n_items; ++t) {
          if (items[3 * t] != s || items[3 * t + 2] / G != g) continue;
          work[2 * n_work] = items[3 * t + 1];
          work[2 * n_work + 1] = items[3 * t + 2];
          widx[n_work] = t;
          ++n_work;
        }
      } else {
        for (int hh = 0; hh < G; ++hh)
          for (int i = 0; i < n; ++i) {
            work[2 * n_work] = i;
            work[2 * n_work + 1] = g * G + hh;
            ++n_work;
          }
      }
      if (n_work == 0) continue;
      double* K = (double*)malloc(sizeof(double) * (size_t)ctx * p->D);
      double* V = (double*)malloc(sizeof(double) * (size_t)ctx * p->D);
      if (!K || !V) {
        free(K); free(V);
        rc = ORC_EINVAL;
        break;
      }
      decode_seq_kv(p, k_pool, v_pool, k_scale, v_scale, bt, s, g, ctx, K, V);
      seq_ctx c = {p, q, K, V, anc, s, ctx, n, row0};
      job proto;
      memset(&proto, 0, sizeof proto);
      proto.c = &c;
      proto.mode = mode;
      proto.g = g;
      proto.G = G;
      proto.n_work = n_work;
      proto.work = work;
      proto.item_index = widx;
      proto.out = out;
      proto.lse = lse;
      proto.nsplit = nsplit;
      proto.bounds = bounds;
      proto.m = m;
      proto.l = l;
      proto.o = o;
      proto.nrows_total = nrows_total;
      run_parallel(&proto, nthreads);
      free(K);
      free(V);
    }
  }
  free(anc);
  free(work);
  free(widx);
  return rc;
}

int orc_attention(const orc_shape* p, const void* q, const void* k_pool, const void* v_pool,
                  const uint16_t* k_scale, const uint16_t* v_scale, const int32_t* block_table,
                  const int32_t* ctx_lens, const int32_t* parent, const int32_t* cu_rows,
                  double* out, double* lse, int nthreads) {
  return drive(p, q, k_pool, v_pool, k_scale, v_scale, block_table, ctx_lens, parent, cu_rows, 0, 0,
               NULL, out, lse, 0, NULL, NULL, NULL, NULL, nthreads);
}

int orc_attention_items(const orc_shape* p, const void* q, const void* k_pool, const void* v_pool,
                        const uint16_t* k_scale, const uint16_t* v_scale,
                        const int32_t* block_table, const int32_t* ctx_lens,
                        const int32_t* parent, const int32_t* cu_rows, int32_t n_items,
                        const int32_t* items, double* out, double* lse, int nthreads) {
  if (n_items < 0 || (n_items > 0 && !items)) return ORC_EINVAL;
  return drive(p, q, k_pool, v_pool, k_scale, v_scale, block_table, ctx_lens, parent, cu_rows, 2,
               n_items, items, out, lse, 0, NULL, NULL, NULL, NULL, nthreads);
}

int orc_split_partials(const orc_shape* p, const void* q, const void* k_pool,
                       const void* v_pool, const uint16_t* k_scale, const uint16_t* v_scale,
                       const int32_t* block_table, const int32_t* ctx_lens,
                       const int32_t* parent, const int32_t* cu_rows, int32_t nsplit,
                       const int32_t* bounds, double* m, double* l, double* o, int nthreads) {
  return drive(p, q, k_pool, v_pool, k_scale, v_scale, block_table, ctx_lens, parent, cu_rows, 1, 0,
               NULL, NULL, NULL, nsplit, bounds, m, l, o, nthreads);
}

int orc_merge(int32_t nsplit, int64_t nrows, int32_t D, const double* m, const double* l,
              const double* o, double* out, double* lse) {
  if (nsplit < 1 || nrows < 0 || D < 1) return ORC_EINVAL;
  for (int64_t r = 0; r < nrows; ++r) {
    double M = -INFINITY;
    for (int k = 0; k < nsplit; ++k) {
      int64_t e = (int64_t)k * nrows + r;
      if (l[e] > 0.0 && m[e] > M) M = m[e];
    }
    double L = 0.0;
    for (int d = 0; d < D; ++d) out[r * D + d] = 0.0;
    for (int k = 0; k < nsplit; ++k) {
      int64_t e = (int64_t)k * nrows + r;
      if (!(l[e] > 0.0)) continue; /* empty split */
      double w = exp(m[e] - M);
      L += w * l[e];
      for (int d = 0; d < D; ++d) out[r * D + d] += w * o[e * D + d];
    }
    for (int d = 0; d < D; ++d) out[r * D + d] /= L;
    lse[r] = M + log(L);
  }
  return ORC_OK;
}

/* ---- KV append with 8-bit block quantisation (the step before verify) ----
 *
 * The B drafted rows' K and V vectors are written into their slots
 * ctx_s - B + i of the paged pools (same layouts as above), before the verify
 * attention reads them (page "perf(qwen35): retain speculation during paged
 * prefill", State and commit invariants: the drafted rows' KV writes are shared
 * by all row kinds).  8-bit pools store one fp16 scale per 32 consecutive
 * head_dim entries with scale = max|x| / 127 of the block, computed in fp32
 * and stored as fp16 round-to-nearest-even; codes
 * q = clamp(round-half-away(x / d), -127, 127) with d the stored fp16 value,
 * in fp32; an all-zero block stores d = 0 and q = 0; a NaN input stores code
 * 0.  These decisions produce integers, so they are made in fp32, the
 * precision the device kernel uses, not in fp64.  fp16 pools store the input
 * rounded to nearest even.
 */

/* fp32 -> IEEE binary16 bits, round to nearest, ties to even. */
static uint16_t f32_to_f16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);  /* NaN */
  if (a >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u); /* >= 65520: rounds to inf */
  if (a >= 0x38800000u) {                                   /* |f| >= 2^-14: normal half */
    const uint32_t mant = a & 0x7fffffu;
    const uint32_t e = (a >> 23) - 127 + 15;
    uint32_t h = (e << 10) | (mant >> 13);
    const uint32_t rem = mant & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++; /* a carry moves to the exponent */
    return (uint16_t)(sign | h);
  }
  /* subnormal half: count units of 2^-24 */
  const uint32_t E = a >> 23;
  if (E == 0) return (uint16_t)sign; /* fp32 subnormal: far below 2^-25 */
  const uint32_t m = (a & 0x7fffffu) | 0x800000u; /* value = m * 2^(E - 150) */
  const uint32_t shift = 126 - E;                  /* value / 2^-24 = m >> shift */
  if (shift >= 32) return (uint16_t)sign;
  uint32_t q = m >> shift;
  const uint32_t rem = m & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) q++;
  return (uint16_t)(sign | q);
}

static float f16_to_f32(uint16_t h) { return (float)f16_to_double(h); }

static float new_to_f32(int dtype, const void* x, int64_t idx) {
  switch (dtype) {
    case ORC_F32: return ((const float*)x)[idx];
    case ORC_F16: return f16_to_f32(((const uint16_t*)x)[idx]);
    default: return (float)bf16_to_double(((const uint16_t*)x)[idx]);
  }
}

static void quantize_block(const float* x, int8_t* q, uint16_t* dbits) {
  float amax = 0.0f;
  for (int e = 0; e < 32; ++e) {
    const float a = fabsf(x[e]);
    if (a > amax) amax = a;
  }
  const float d = amax / 127.0f;
  const uint16_t h = f32_to_f16_rne(d);
  const float d16 = f16_to_f32(h);
  for (int e = 0; e < 32; ++e) {
    float r = 0.0f;
    if (d16 != 0.0f) r = x[e] / d16;
    if (r != r) r = 0.0f;
    r = roundf(r);
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    q[e] = (int8_t)r;
  }
  *dbits = h;
}

int orc_decode_f16(int64_t n, const uint16_t* h, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f16_to_double(h[i]);
  return ORC_OK;
}

int orc_decode_bf16(int64_t n, const uint16_t* b, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_to_double(b[i]);
  return ORC_OK;
}

int orc_f32_to_f16(int64_t n, const float* x, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_f16_rne(x[i]);
  return ORC_OK;
}

int orc_quantize_blocks(int64_t nblocks, const float* x, int8_t* q, uint16_t* d) {
  for (int64_t b = 0; b < nblocks; ++b) quantize_block(x + 32 * b, q + 32 * b, d + b);
  return ORC_OK;
}

int orc_append_kv(const orc_shape* p, int32_t new_dtype, const void* k_new, const void* v_new,
                  void* k_pool, void* v_pool, uint16_t* k_scale, uint16_t* v_scale,
                  const int32_t* block_table, const int32_t* ctx_lens) {
  if (check_shape(p) != ORC_OK) return ORC_EINVAL;
  if (p->kv_dtype != ORC_Q8 && p->kv_dtype != ORC_F16) return ORC_EINVAL;
  if (new_dtype != ORC_F32 && new_dtype != ORC_F16 && new_dtype != ORC_BF16) return ORC_EINVAL;
  for (int s = 0; s < p->num_seqs; ++s)
    if (check_seq(p, block_table, ctx_lens, NULL, p->B, s) != ORC_OK) return ORC_EINVAL;
  const int D = p->D, KVH = p->KVH, nb = D / 32;
  float x[32];
  int8_t q[32];
  for (int s = 0; s < p->num_seqs; ++s) {
    const int base = ctx_lens[s] - p->B;
    for (int i = 0; i < p->B; ++i) {
      const int t = base + i;
      const int64_t page = block_table[(int64_t)s * p->max_pages + t / ORC_PAGE];
      const int slot = t % ORC_PAGE;
      for (int g = 0; g < KVH; ++g) {
        const int64_t src = ((int64_t)(s * p->B + i) * KVH + g) * D;
        const int64_t pk = (page * KVH + g) * ORC_PAGE * D; /* element offset of this page / head */
        for (int which = 0; which < 2; ++which) {
          const void* xin = which ? v_new : k_new;
          if (p->kv_dtype == ORC_F16) {
            uint16_t* pool = (uint16_t*)(which ? v_pool : k_pool);
            for (int d = 0; d < D; ++d) {
              const uint16_t h = f32_to_f16_rne(new_to_f32(new_dtype, xin, src + d));
              if (which) pool[pk + (int64_t)d * ORC_PAGE + slot] = h;
              else pool[pk + (int64_t)slot * D + d] = h;
            }
            continue;
          }
          int8_t* pool = (int8_t*)(which ? v_pool : k_pool);
          uint16_t* sc = which ? v_scale : k_scale;
          const int64_t ps = (page * KVH + g) * ORC_PAGE * nb; /* scale offset of this page / head */
          for (int b = 0; b < nb; ++b) {
            uint16_t dbits;
            for (int e = 0; e < 32; ++e) x[e] = new_to_f32(new_dtype, xin, src + 32 * b + e);
            quantize_block(x, q, &dbits);
            for (int e = 0; e < 32; ++e) {
              const int d = 32 * b + e;
              if (which) pool[pk + (int64_t)d * ORC_PAGE + slot] = q[e];
              else pool[pk + (int64_t)slot * D + d] = q[e];
            }
            if (which) sc[ps + (int64_t)b * ORC_PAGE + slot] = dbits;
            else sc[ps + (int64_t)slot * nb + b] = dbits;
          }
        }
      }
    }
  }
  return ORC_OK;
}

/* ---- accepted-path KV promotion (the step after verify, tree mode) ----
 *
 * After the tree rows are verified, the caller picks for each sequence an
 * accepted path r_0, ..., r_{n-1} of drafted rows (root first, each node the
 * child of the previous one: parent[r_k] == r_{k-1}).  Promotion copies their
 * K / V vectors (and 8-bit scales) to the consecutive slots that directly
 * follow the first node's parent, dst = base + parent[r_0] + 1 (base when the
 * parent is -1), so the durable prefix then reads as the accepted tokens in
 * order; new_ctx = dst + n.  Every sequence is checked before any pool byte
 * changes, and on any failure nothing is written (the page "perf(qwen35):
 * retain speculation during paged prefill", State and commit invariants:
 * promotion moves only the accepted prefix and preflights before mutating).
 * Sources and destinations may overlap; the copy goes through a buffer.
 */
static int64_t slot_elem(int kv_dtype_is_v, int64_t page, int KVH, int g, int D, int slot, int d) {
  const int64_t head = (page * KVH + g) * ORC_PAGE * D;
  return kv_dtype_is_v ? head + (int64_t)d * ORC_PAGE + slot : head + (int64_t)slot * D + d;
}

int orc_promote_kv(const orc_shape* p, const int32_t* accepted, const int32_t* n_accepted,
                   const int32_t* parent, void* k_pool, void* v_pool, uint16_t* k_scale,
                   uint16_t* v_scale, const int32_t* block_table, const int32_t* ctx_lens,
                   int32_t* new_ctx) {
  if (check_shape(p) != ORC_OK) return ORC_EINVAL;
  if (p->kv_dtype != ORC_Q8 && p->kv_dtype != ORC_F16) return ORC_EINVAL;
  const int B = p->B, D = p->D, KVH = p->KVH, nb = D / 32;
  /* preflight: every sequence, before any write */
  for (int s = 0; s < p->num_seqs; ++s) {
    if (check_seq(p, block_table, ctx_lens, parent ? parent + (int64_t)s * B : NULL, B, s) != ORC_OK)
      return ORC_EINVAL;
    const int n = n_accepted[s];
    if (n < 0 || n > B) return ORC_EINVAL;
    for (int k = 0; k < n; ++k) {
      const int r = accepted[(int64_t)s * B + k];
      if (r < 0 || r >= B) return ORC_EINVAL;
      const int par = parent ? parent[(int64_t)s * B + r] : r - 1;
      if (k > 0 && par != accepted[(int64_t)s * B + k - 1]) return ORC_EINVAL;
    }
  }
  const int esz = p->kv_dtype == ORC_Q8 ? 1 : 2;
  unsigned char* kbuf = (unsigned char*)malloc((size_t)B * KVH * D * esz);
  unsigned char* vbuf = (unsigned char*)malloc((size_t)B * KVH * D * esz);
  uint16_t* ksbuf = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)B * KVH * nb + 2);
  uint16_t* vsbuf = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)B * KVH * nb + 2);
  if (!kbuf || !vbuf || !ksbuf || !vsbuf) {
    free(kbuf); free(vbuf); free(ksbuf); free(vsbuf);
    return ORC_EINVAL;
  }
  for (int s = 0; s < p->num_seqs; ++s) {
    const int n = n_accepted[s];
    const int base = ctx_lens[s] - B;
    const int32_t* bt = block_table + (int64_t)s * p->max_pages;
    int dst = base;
    if (n > 0) {
      const int r0 = accepted[(int64_t)s * B];
      const int par0 = parent ? parent[(int64_t)s * B + r0] : r0 - 1;
      dst = base + par0 + 1;
    }
    /* gather the accepted rows */
    for (int k = 0; k < n; ++k) {
      const int t = base + accepted[(int64_t)s * B + k];
      const int64_t page = bt[t / ORC_PAGE];
      const int slot = t % ORC_PAGE;
      for (int g = 0; g < KVH; ++g) {
        for (int d = 0; d < D; ++d) {
          const int64_t kb = ((int64_t)(k * KVH + g) * D + d) * esz;
          memcpy(kbuf + kb, (unsigned char*)k_pool + slot_elem(0, page, KVH, g, D, slot, d) * esz, esz);
          memcpy(vbuf + kb, (unsigned char*)v_pool + slot_elem(1, page, KVH, g, D, slot, d) * esz, esz);
        }
        if (p->kv_dtype == ORC_Q8)
          for (int b = 0; b < nb; ++b) {
            ksbuf[(k * KVH + g) * nb + b] = k_scale[((page * KVH + g) * ORC_PAGE + slot) * nb + b];
            vsbuf[(k * KVH + g) * nb + b] = v_scale[((page * KVH + g) * nb + b) * ORC_PAGE + slot];
          }
      }
    }
    /* write them to the consecutive slots after the anchor */
    for (int k = 0; k < n; ++k) {
      const int t = dst + k;
      const int64_t page = bt[t / ORC_PAGE];
      const int slot = t % ORC_PAGE;
      for (int g = 0; g < KVH; ++g) {
        for (int d = 0; d < D; ++d) {
          const int64_t kb = ((int64_t)(k * KVH + g) * D + d) * esz;
          memcpy((unsigned char*)k_pool + slot_elem(0, page, KVH, g, D, slot, d) * esz, kbuf + kb, esz);
          memcpy((unsigned char*)v_pool + slot_elem(1, page, KVH, g, D, slot, d) * esz, vbuf + kb, esz);
        }
        if (p->kv_dtype == ORC_Q8)
          for (int b = 0; b < nb; ++b) {
            k_scale[((page * KVH + g) * ORC_PAGE + slot) * nb + b] = ksbuf[(k * KVH + g) * nb + b];
            v_scale[((page * KVH + g) * nb + b) * ORC_PAGE + slot] = vsbuf[(k * KVH + g) * nb + b];
          }
      }
    }
    if (new_ctx) new_ctx[s] = dst + n;
  }
  free(kbuf); free(vbuf); free(ksbuf); free(vsbuf);
  return ORC_OK;
}
