/*
 * attn_oracle.c - plain FP64 CPU reference for grouped-query attention over a
 * paged K/V cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library calls this file; only the
 * tests, the smoke check and the benchmark's CPU-baseline timing load it.  It
 * shares no code, header or constant with the HIP path.
 *
 * What it computes is the textbook definition of scaled dot-product attention
 * (softmax of scaled query-key dot products weighting the values), evaluated
 * in double precision over the *stored* (already quantised) K/V values:
 *   - Geramy/LSE README, "K/V storage" paragraph: attention accumulation,
 *     softmax state and output are FP32 on the GPU; the oracle uses FP64.
 *   - Geramy/LSE releases, v0.4.21 "joint decode attention": the query heads
 *     of a group read the same K/V; here query head h reads KV head h / G.
 *   - Geramy/LSE releases, v0.4.19 and v0.4.20: verify rows and split-KV
 *     partitions merged by log-sum-exp give the same result as unsplit
 *     attention; the oracle evaluates the unsplit definition directly and
 *     offers the partition + merge form separately for invariant checks.
 *   - Geramy/LSE releases, v0.4.14: skipping fully masked key windows keeps
 *     the arithmetic of the rest, so masked keys simply do not contribute.
 *   - TokenSpeed-Kernel-AMD page, "Attention": full causal attention with
 *     attention sinks; a sink adds exp(sink) to the softmax denominator only.
 *   - Geramy/LSE README, FlashPrefill V2 paragraph: sparse prefill attends
 *     only to the selected blocks, so a block mask removes keys.
 *
 * Readings where the pages are silent (kept identical on the GPU side):
 *   query head h uses KV head floor(h / G), G = Hq / Hkv;
 *   row i of the n rows of a sequence (n = n_q, or the sequence's own row
 *   count when rows vary per sequence) sits at absolute position L - n + i (bottom-right
 *   causal alignment) and sees keys j <= that position;
 *   a sink is one logit per query head in the units of the scaled score,
 *   natural base, contributing exp(sink) to the denominator and no value;
 *   a block-mask entry [b][mh][qb][kb] != 0 keeps key block kb for query
 *   block qb (qb from the absolute position), entries outside the mask's
 *   extent count as 0; mh = 0 for one mask head, else the KV head;
 *   a row with no allowed key has o = 0 and lse = sink (or -inf);
 *   a sequence holds at most as many keys as its page-table row addresses
 *   (page_table_stride * page_size): a longer seq_lens entry counts as that
 *   capacity (the partition count of a split follows the K/V table's
 *   capacity, Geramy/LSE releases v0.4.20 "automatic split attention", so
 *   no key lies beyond it);
 *   FP8 is OCP e4m3fn (bias 7, no infinities, S.1111.111 is NaN) and BF8
 *   is OCP e5m2 (bias 15, with infinities), each times the per-tensor scale
 *   and, where the cache carries them, the FP32 scale of its (token, head)
 *   vector (Geramy/LSE README, "K/V storage": fp8 and bf8 kept with scales,
 *   33,280 bytes per token = codes plus one FP32 scale per K or V vector;
 *   the architecture paragraph: FP8/BF8 loads decoded with per-vector
 *   scales).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_E4M3 = 3, ORC_E5M2 = 4 };

typedef struct {
  int32_t kv_dtype;
  const void *k_pool, *v_pool;   /* K tile: [16 tokens][d]; V tile: [d][16 tokens] */
  int64_t k_stride_page, k_stride_head, v_stride_page, v_stride_head; /* elements */
  int32_t num_pages, num_kv_heads, head_dim, page_size;
  double k_scale, v_scale;
  const int32_t *page_table;
  int32_t page_table_stride;
  const int32_t *seq_lens;
  int32_t q_dtype;
  const void *q;                 /* [batch][n_q][Hq][d], contiguous */
  int32_t batch, n_q, num_q_heads;
  double softmax_scale;
  const float *sinks;            /* NULL or [Hq] */
  const uint8_t *mask;           /* NULL or [batch][mask_heads][mask_nqb][mask_nkb] */
  int32_t mask_heads, mask_block, mask_nqb, mask_nkb;
  const int32_t *rows_per_seq;   /* NULL or [batch]: sequence b has rows 0 .. r_b - 1 */
  const float *k_vs, *v_vs;      /* NULL, or per-vector scales [page][kv head][16 tokens] */
  int64_t vs_stride_page, vs_stride_head;   /* floats */
} orc_problem;

/* ---- storage decoding (bit formulas, one per format) ---------------------- */

static double dec_f16(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
  else if (e == 31) v = f ? NAN : INFINITY;
  else v = ldexp(1.0 + f / 1024.0, e - 15);
  return s ? -v : v;
}

static double dec_bf16(uint16_t h) {
  int s = h >> 15, e = (h >> 7) & 255, f = h & 127;
  double v;
  if (e == 0) v = ldexp((double)f, -133);                /* f/128 * 2^-126 */
  else if (e == 255) v = f ? NAN : INFINITY;
  else v = ldexp(1.0 + f / 128.0, e - 127);
  return s ? -v : v;
}

static double dec_e4m3(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, f = c & 7;
  double v;
  if (e == 15 && f == 7) return NAN;                     /* e4m3fn: no infinities */
  if (e == 0) v = ldexp((double)f, -9);                  /* f/8 * 2^-6 */
  else v = ldexp(1.0 + f / 8.0, e - 7);
  return s ? -v : v;
}

static double dec_e5m2(uint8_t c) {
  int s = c >> 7, e = (c >> 2) & 31, f = c & 3;
  double v;
  if (e == 31) v = f ? NAN : INFINITY;                   /* e5m2 keeps IEEE specials */
  else if (e == 0) v = ldexp((double)f, -16);            /* f/4 * 2^-14 */
  else v = ldexp(1.0 + f / 4.0, e - 15);
  return s ? -v : v;
}

static double dec_f32(const void *p) {
  float f;
  memcpy(&f, p, 4);
  return (double)f;
}

double orc_decode(int32_t dtype, const void *base, int64_t idx) {
  switch (dtype) {
    case ORC_F32: return dec_f32((const char *)base + 4 * idx);
    case ORC_F16: { uint16_t h; memcpy(&h, (const char *)base + 2 * idx, 2); return dec_f16(h); }
    case ORC_BF16: { uint16_t h; memcpy(&h, (const char *)base + 2 * idx, 2); return dec_bf16(h); }
    case ORC_E4M3: return dec_e4m3(((const uint8_t *)base)[idx]);
    case ORC_E5M2: return dec_e5m2(((const uint8_t *)base)[idx]);
  }
  return NAN;
}

/* decode n codes into out[] (used to check the formulas code by code) */
void orc_decode_array(int32_t dtype, const void *base, int64_t n, double *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_decode(dtype, base, i);
}

/* ---- paged gather ---------------------------------------------------------- */

/* the per-vector scale of token slot t of (page, g), 1 without per-vector scales */
static double vector_scale(const orc_problem *P, const float *vs, int32_t page, int g, int64_t t) {
  if (!vs) return 1.0;
  return (double)vs[page * P->vs_stride_page + g * P->vs_stride_head + t];
}

/* logical key j of sequence b, KV head g, component c (dequantised, scaled);
 * the products are exact in double precision (a code has at most 4
 * significant bits, each scale 24) */
static double key_at(const orc_problem *P, int b, int g, int64_t j, int c) {
  int32_t page = P->page_table[(int64_t)b * P->page_table_stride + j / P->page_size];
  int64_t t = j % P->page_size;
  int64_t idx = page * P->k_stride_page + g * P->k_stride_head + t * P->head_dim + c;
  return orc_decode(P->kv_dtype, P->k_pool, idx) * vector_scale(P, P->k_vs, page, g, t) *
         P->k_scale;
}

static double value_at(const orc_problem *P, int b, int g, int64_t j, int c) {
  int32_t page = P->page_table[(int64_t)b * P->page_table_stride + j / P->page_size];
  int64_t t = j % P->page_size;
  int64_t idx = page * P->v_stride_page + g * P->v_stride_head + (int64_t)c * P->page_size + t;
  return orc_decode(P->kv_dtype, P->v_pool, idx) * vector_scale(P, P->v_vs, page, g, t) *
         P->v_scale;
}

/* keys of sequence b: its seq_lens entry, at most the page table's capacity */
static int64_t len_of(const orc_problem *P, int b) {
  int64_t L = P->seq_lens[b];
  int64_t cap = (int64_t)P->page_table_stride * P->page_size;
  return L < cap ? L : cap;
}

/* K and V of sequence b, KV head g as logical [L][d] FP64 arrays */
void orc_gather(const orc_problem *P, int b, int g, double *k_out, double *v_out) {
  int64_t L = len_of(P, b);
  int d = P->head_dim;
  for (int64_t j = 0; j < L; ++j)
    for (int c = 0; c < d; ++c) {
      k_out[j * d + c] = key_at(P, b, g, j, c);
      v_out[j * d + c] = value_at(P, b, g, j, c);
    }
}

/* ---- attention, by definition ---------------------------------------------- */

static double query_at(const orc_problem *P, int b, int i, int h, int c) {
  int64_t idx = (((int64_t)b * P->n_q + i) * P->num_q_heads + h) * P->head_dim + c;
  return orc_decode(P->q_dtype, P->q, idx);
}

static int key_allowed(const orc_problem *P, int b, int g, int64_t pos, int64_t j) {
  if (j > pos) return 0;                                 /* causal */
  if (!P->mask) return 1;
  int64_t qb = pos / P->mask_block, kb = j / P->mask_block;
  if (qb >= P->mask_nqb || kb >= P->mask_nkb) return 0;
  int mh = P->mask_heads == 1 ? 0 : g;
  int64_t idx = (((int64_t)b * P->mask_heads + mh) * P->mask_nqb + qb) * P->mask_nkb + kb;
  return P->mask[idx] != 0;
}

/* rows of sequence b (all n_q unless they vary per sequence) */
static int64_t rows_of(const orc_problem *P, int b) {
  return P->rows_per_seq ? P->rows_per_seq[b] : P->n_q;
}

static double scale_of(const orc_problem *P) {
  return P->softmax_scale > 0 ? P->softmax_scale : 1.0 / sqrt((double)P->head_dim);
}

/* the query row (b, i, h), decoded once */
static void load_query(const orc_problem *P, int b, int i, int h, double *q) {
  for (int c = 0; c < P->head_dim; ++c) q[c] = query_at(P, b, i, h, c);
}

/* score of a decoded query row against key j of KV head g */
static double score(const orc_problem *P, const double *q, int b, int g, int64_t j) {
  double acc = 0.0;
  for (int c = 0; c < P->head_dim; ++c) acc += q[c] * key_at(P, b, g, j, c);
  return scale_of(P) * acc;
}

/*
 * Attention over the allowed keys of [j0, j1) for one row, *without* the sink:
 * returns the partition's max score m, its sum l = sum exp(s_j - m) and the
 * normalised output o = sum exp(s_j - m) v_j / l.  An empty set gives
 * m = -inf, l = 0, o = 0.  This is the per-partition state that a split-KV
 * evaluation combines (Geramy/LSE releases, v0.4.19 partial/merge families).
 */
void orc_attend_partial(const orc_problem *P, int b, int i, int h, int64_t j0, int64_t j1,
                        double *o, double *m_out, double *l_out) {
  int G = P->num_q_heads / P->num_kv_heads, g = h / G, d = P->head_dim;
  int64_t L = len_of(P, b), pos = L - rows_of(P, b) + i;
  if (j1 > L) j1 = L;
  double q[1024];
  load_query(P, b, i, h, q);
  double m = -INFINITY;
  for (int64_t j = j0; j < j1; ++j)
    if (key_allowed(P, b, g, pos, j)) {
      double s = score(P, q, b, g, j);
      if (s > m) m = s;
    }
  double l = 0.0;
  for (int c = 0; c < d; ++c) o[c] = 0.0;
  if (m != -INFINITY) {
    for (int64_t j = j0; j < j1; ++j)
      if (key_allowed(P, b, g, pos, j)) {
        double p = exp(score(P, q, b, g, j) - m);
        l += p;
        for (int c = 0; c < d; ++c) o[c] += p * value_at(P, b, g, j, c);
      }
    for (int c = 0; c < d; ++c) o[c] /= l;
  }
  *m_out = m;
  *l_out = l;
}

/*
 * Log-sum-exp merge of n partition states (o_k, m_k, l_k) plus an optional
 * sink logit: M = max(max_k m_k, sink), Z = sum_k l_k e^{m_k - M} + e^{sink - M},
 * o = sum_k l_k e^{m_k - M} o_k / Z, lse = M + ln Z.
 */
void orc_merge(int n, int d, const double *o_parts, const double *m, const double *l,
               double sink, double *o, double *lse) {
  double M = sink;
  for (int k = 0; k < n; ++k) if (m[k] > M) M = m[k];
  for (int c = 0; c < d; ++c) o[c] = 0.0;
  if (M == -INFINITY) { *lse = -INFINITY; return; }
  double Z = exp(sink - M);
  for (int k = 0; k < n; ++k) {
    if (m[k] == -INFINITY) continue;
    double w = l[k] * exp(m[k] - M);
    Z += w;
    for (int c = 0; c < d; ++c) o[c] += w * o_parts[(int64_t)k * d + c];
  }
  for (int c = 0; c < d; ++c) o[c] /= Z;
  *lse = M + log(Z);
}

/* one output row by the definition: softmax over the allowed keys and the sink */
static void attend_row(const orc_problem *P, int b, int i, int h, double *o, double *lse,
                       double *s_buf) {
  int G = P->num_q_heads / P->num_kv_heads, g = h / G, d = P->head_dim;
  int64_t L = len_of(P, b), pos = L - rows_of(P, b) + i;
  double sink = P->sinks ? (double)P->sinks[h] : -INFINITY;
  if (i >= rows_of(P, b)) {            /* no such row: marked NaN (not part of the output) */
    for (int c = 0; c < d; ++c) o[c] = NAN;
    *lse = NAN;
    return;
  }
  double q[1024];
  load_query(P, b, i, h, q);
  double m = sink;
  for (int64_t j = 0; j < L; ++j) {
    if (key_allowed(P, b, g, pos, j)) {
      s_buf[j] = score(P, q, b, g, j);
      if (s_buf[j] > m) m = s_buf[j];
    } else {
      s_buf[j] = -INFINITY;
    }
  }
  for (int c = 0; c < d; ++c) o[c] = 0.0;
  if (m == -INFINITY) { *lse = -INFINITY; return; }
  double Z = exp(sink - m);
  for (int64_t j = 0; j < L; ++j) {
    if (s_buf[j] == -INFINITY) continue;
    double p = exp(s_buf[j] - m);
    Z += p;
    for (int c = 0; c < d; ++c) o[c] += p * value_at(P, b, g, j, c);
  }
  for (int c = 0; c < d; ++c) o[c] /= Z;
  *lse = m + log(Z);
}

/* ---- driver: a list of rows, split over threads ------------------------------- */

typedef struct {
  const orc_problem *P;
  int64_t nrows;
  const int32_t *rows;   /* triples (b, i, h) */
  double *o, *lse;
  int64_t first, step;
} orc_job;

static void *run_job(void *arg) {
  orc_job *J = (orc_job *)arg;
  int64_t maxL = 0;
  for (int b = 0; b < J->P->batch; ++b)
    if (len_of(J->P, b) > maxL) maxL = len_of(J->P, b);
  double *s_buf = (double *)malloc(sizeof(double) * (size_t)(maxL > 0 ? maxL : 1));
  for (int64_t r = J->first; r < J->nrows; r += J->step) {
    const int32_t *t = J->rows + 3 * r;
    attend_row(J->P, t[0], t[1], t[2], J->o + r * J->P->head_dim, J->lse + r, s_buf);
  }
  free(s_buf);
  return NULL;
}

/* o[nrows][d], lse[nrows] for the listed rows; returns the threads used */
int orc_attend_rows(const orc_problem *P, int64_t nrows, const int32_t *rows, double *o,
                    double *lse, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > nrows) nthreads = (int)(nrows > 0 ? nrows : 1);
  pthread_t th[256];
  orc_job jobs[256];
  if (nthreads > 256) nthreads = 256;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = (orc_job){P, nrows, rows, o, lse, t, nthreads};
    if (nthreads == 1) run_job(&jobs[t]);
    else pthread_create(&th[t], NULL, run_job, &jobs[t]);
  }
  if (nthreads > 1)
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  return nthreads;
}

/* ------------------------------------------------------------------------
 * Encoding for the K/V append step.  The cache is kept in 16-bit or FP8
 * storage (Geramy/LSE README, "K/V storage") and the writes into it are
 * checked against CPU references (Geramy/LSE releases, v0.4.20,
 * "Correctness").
 *
 * A stored value is the source value divided by the per-tensor scale (one
 * IEEE single-precision division; the scale is 1 except for FP8), rounded to
 * the storage format with round-to-nearest, ties to even (IEEE 754
 * roundTiesToEven).  IEEE formats overflow to infinity; e4m3fn has no
 * infinity, and a value beyond its largest finite magnitude (448) is stored as
 * +-448 (saturation).  e5m2 saturates finite values beyond 57344 the same
 * way and keeps infinities.  NaN stays NaN.
 *
 * With per-vector scales (8-bit storage, Geramy/LSE README "K/V storage":
 * fp8 and bf8 with scales) each (token, head) vector x of K or V gets its own
 * scale u = amax / fmax, one single-precision division, where amax is the
 * largest |x_i| over its finite entries and fmax the format's largest finite
 * value (448, 57344); u = 1 when that quotient is 0.  Each x_i is then stored
 * as x_i / u (one single-precision division) rounded as above, and u is
 * stored beside the codes.  (Reading: the pages fix no rule for the scale;
 * mapping the vector's largest magnitude to the format's largest code is the
 * plainest.)
 *
 * The rounding is evaluated from the definition in double precision: the
 * value's quantum (the spacing of the format's grid at its magnitude) is a
 * power of two, so a / quantum is exact and rint() applies the tie rule.
 * ------------------------------------------------------------------------ */

/* code of a finite, non-negative grid value r of a format with eb exponent
 * bits, mb mantissa bits and bias (2^(eb-1) - 1) */
static uint32_t pack_grid_value(double r, int eb, int mb) {
  const int bias = (1 << (eb - 1)) - 1;
  const int emin = 1 - bias;
  if (r == 0.0) return 0u;
  int k;
  (void)frexp(r, &k);
  const int e = k - 1;                        /* r = 1.f * 2^e */
  if (e < emin)                               /* subnormal: field 0 */
    return (uint32_t)(r / ldexp(1.0, emin - mb));
  const uint32_t field = (uint32_t)(e + bias);
  const uint32_t mant = (uint32_t)(r / ldexp(1.0, e - mb)) - (1u << mb);
  return (field << mb) | mant;
}

/* round-to-nearest-even of |x| onto the grid of a format with eb / mb bits */
static double round_to_grid(double a, int eb, int mb) {
  const int bias = (1 << (eb - 1)) - 1;
  const int emin = 1 - bias;
  if (a == 0.0) return 0.0;
  int k;
  (void)frexp(a, &k);
  int e = k - 1;
  if (e < emin) e = emin;
  const double q = ldexp(1.0, e - mb);
  return rint(a / q) * q;
}

/* IEEE binary16 (eb 5, mb 10) and bfloat16 (eb 8, mb 7) */
static uint32_t enc_ieee(double x, int eb, int mb) {
  const uint32_t sign = signbit(x) ? 1u : 0u;
  const uint32_t sbit = sign << (eb + mb);
  const uint32_t inf = ((1u << eb) - 1u) << mb;
  if (isnan(x)) return sbit | inf | (1u << (mb - 1));          /* quiet NaN */
  const double a = fabs(x);
  const int bias = (1 << (eb - 1)) - 1;
  const double maxfin = ldexp(2.0 - ldexp(1.0, -mb), ((1 << eb) - 2) - bias);
  if (isinf(a)) return sbit | inf;
  const double r = round_to_grid(a, eb, mb);
  if (r > maxfin) return sbit | inf;
  return sbit | pack_grid_value(r, eb, mb);
}

/* OCP e4m3fn: bias 7, no infinities, S.1111.111 is NaN, largest finite 448 */
static uint32_t enc_e4m3fn(double x) {
  const uint32_t sbit = signbit(x) ? 0x80u : 0u;
  if (isnan(x)) return sbit | 0x7Fu;
  const double a = fabs(x);
  const double r = isinf(a) ? 448.0 : round_to_grid(a, 4, 3);
  if (r >= 448.0) return sbit | 0x7Eu;                          /* saturate */
  return sbit | pack_grid_value(r, 4, 3);
}

/* OCP e5m2: bias 15, IEEE specials (S.11111.00 infinity, S.11111.xx NaN),
 * largest finite 57344; finite values beyond it saturate */
static uint32_t enc_e5m2(double x) {
  const uint32_t sbit = signbit(x) ? 0x80u : 0u;
  if (isnan(x)) return sbit | 0x7Fu;
  const double a = fabs(x);
  if (isinf(a)) return sbit | 0x7Cu;
  const double r = round_to_grid(a, 5, 2);
  if (r >= 57344.0) return sbit | 0x7Bu;                        /* saturate */
  return sbit | pack_grid_value(r, 5, 2);
}

static void encode_one(int32_t dtype, float y, void *out, int64_t i) {
  switch (dtype) {
    case ORC_F32: ((float *)out)[i] = y; break;
    case ORC_F16: ((uint16_t *)out)[i] = (uint16_t)enc_ieee((double)y, 5, 10); break;
    case ORC_BF16: ((uint16_t *)out)[i] = (uint16_t)enc_ieee((double)y, 8, 7); break;
    case ORC_E4M3: ((uint8_t *)out)[i] = (uint8_t)enc_e4m3fn((double)y); break;
    default: ((uint8_t *)out)[i] = (uint8_t)enc_e5m2((double)y); break;
  }
}

/* out[i] = code of x[i] / scale in `dtype` (F32 stores the quotient itself) */
void orc_encode_array(int32_t dtype, int64_t n, const float *x, float scale, void *out) {
  for (int64_t i = 0; i < n; ++i) encode_one(dtype, x[i] / scale, out, i);  /* one IEEE division */
}

/* Per-vector scales of n vectors of d values (x[n][d]) for an 8-bit format
 * with largest finite value fmax: scales[v] = amax_v / fmax, or 1 if that is 0 */
void orc_vector_scales(int64_t n, int32_t d, const float *x, float fmax, float *scales) {
  for (int64_t v = 0; v < n; ++v) {
    float amax = 0.0f;
    for (int32_t i = 0; i < d; ++i) {
      const float a = fabsf(x[v * d + i]);
      if (isfinite(a) && a > amax) amax = a;
    }
    const float u = amax / fmax;               /* one IEEE single division */
    scales[v] = (u == 0.0f) ? 1.0f : u;
  }
}

/* codes of x[v][i] / scales[v] (each one IEEE single division) */
void orc_encode_vectors(int32_t dtype, int64_t n, int32_t d, const float *x, const float *scales,
                        void *out) {
  for (int64_t v = 0; v < n; ++v)
    for (int32_t i = 0; i < d; ++i) encode_one(dtype, x[v * d + i] / scales[v], out, v * d + i);
}
