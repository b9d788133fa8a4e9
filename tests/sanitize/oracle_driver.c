/*
 * Drives the FP64 oracle (compiled into this file) under AddressSanitizer and
 * UndefinedBehaviorSanitizer on small paged problems that reach every branch
 * of its indexing: shuffled pages, lengths beyond the page table's capacity,
 * ragged rows, a block mask smaller than the sequence's block count, per-head
 * masks, sinks, per-vector scales, every storage format, the split + merge
 * form and the encoders on special values.  Exits non-zero if an output is
 * not finite where it must be (a sanitizer report aborts the run by itself).
 */
#include "../../oracle/attn_oracle.c"

#include <stdio.h>

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (uint32_t)(rng >> 16);
}
static double unit(void) { return (next_u32() & 0xffffff) / 16777216.0 * 2.0 - 1.0; }

/* a random code of `dtype` for a value in about [-2, 2] */
static void put_code(int32_t dtype, void *base, int64_t i) {
  float x = (float)(2.0 * unit());
  switch (dtype) {
    case ORC_F32: ((float *)base)[i] = x; break;
    case ORC_F16: ((uint16_t *)base)[i] = (uint16_t)enc_ieee(x, 5, 10); break;
    case ORC_BF16: ((uint16_t *)base)[i] = (uint16_t)enc_ieee(x, 8, 7); break;
    case ORC_E4M3: ((uint8_t *)base)[i] = (uint8_t)enc_e4m3fn(x * 100.0); break;
    default: ((uint8_t *)base)[i] = (uint8_t)enc_e5m2(x * 100.0); break;
  }
}

static int elt(int32_t dtype) { return dtype == ORC_F32 ? 4 : dtype <= ORC_BF16 ? 2 : 1; }

static int run_case(int32_t kv_dtype, int n_q, int use_mask, int use_vs, int ragged) {
  enum { B = 3, HQ = 4, HKV = 2, D = 16, PS = 16, STRIDE = 5, NPAGES = 16 };
  const int64_t tile = (int64_t)PS * D;
  void *k = calloc((size_t)NPAGES * HKV * tile, (size_t)elt(kv_dtype));
  void *v = calloc((size_t)NPAGES * HKV * tile, (size_t)elt(kv_dtype));
  for (int64_t i = 0; i < (int64_t)NPAGES * HKV * tile; ++i) {
    put_code(kv_dtype, k, i);
    put_code(kv_dtype, v, i);
  }
  int32_t pt[B * STRIDE];
  for (int i = 0; i < B * STRIDE; ++i) pt[i] = (int32_t)((i * 7 + 3) % NPAGES);
  /* one sequence past the capacity (80 tokens), one empty-ish, one ragged tail */
  int32_t lens[B] = {STRIDE * PS + 33, 3, 45};
  int32_t rows[B] = {n_q, 1, n_q > 1 ? n_q - 1 : 0};
  uint16_t *q = calloc((size_t)B * n_q * HQ * D, 2);
  for (int64_t i = 0; i < (int64_t)B * n_q * HQ * D; ++i) q[i] = (uint16_t)enc_ieee(unit(), 8, 7);
  float sinks[HQ];
  for (int h = 0; h < HQ; ++h) sinks[h] = (float)unit();
  /* mask of 2 x 1 blocks of 32 tokens: smaller than the sequences' block counts */
  const int mnq = 2, mnk = 1, mh = 2;
  uint8_t *mask = calloc((size_t)B * mh * mnq * mnk, 1);
  for (int i = 0; i < B * mh * mnq * mnk; ++i) mask[i] = (uint8_t)(next_u32() & 1);
  float *kvs = NULL, *vvs = NULL;
  if (use_vs) {
    kvs = malloc(sizeof(float) * NPAGES * HKV * PS);
    vvs = malloc(sizeof(float) * NPAGES * HKV * PS);
    for (int i = 0; i < NPAGES * HKV * PS; ++i) {
      kvs[i] = (float)(0.01 * (1.5 + unit()));
      vvs[i] = (float)(0.01 * (1.5 + unit()));
    }
  }
  orc_problem P;
  memset(&P, 0, sizeof P);
  P.kv_dtype = kv_dtype;
  P.k_pool = k;
  P.v_pool = v;
  P.k_stride_page = HKV * tile;
  P.k_stride_head = tile;
  P.v_stride_page = HKV * tile;
  P.v_stride_head = tile;
  P.num_pages = NPAGES;
  P.num_kv_heads = HKV;
  P.head_dim = D;
  P.page_size = PS;
  P.k_scale = kv_dtype >= ORC_E4M3 && !use_vs ? 0.01 : 1.0;
  P.v_scale = P.k_scale;
  P.page_table = pt;
  P.page_table_stride = STRIDE;
  P.seq_lens = lens;
  P.q_dtype = ORC_BF16;
  P.q = q;
  P.batch = B;
  P.n_q = n_q;
  P.num_q_heads = HQ;
  P.softmax_scale = 0.3;
  P.sinks = sinks;
  if (use_mask) {
    P.mask = mask;
    P.mask_heads = mh;
    P.mask_block = 32;
    P.mask_nqb = mnq;
    P.mask_nkb = mnk;
  }
  P.rows_per_seq = ragged ? rows : NULL;
  P.k_vs = kvs;
  P.v_vs = vvs;
  P.vs_stride_page = HKV * PS;
  P.vs_stride_head = PS;

  const int64_t nrows = (int64_t)B * n_q * HQ;
  int32_t *list = malloc(sizeof(int32_t) * 3 * nrows);
  int64_t r = 0;
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < n_q; ++i)
      for (int h = 0; h < HQ; ++h) {
        list[3 * r] = b;
        list[3 * r + 1] = i;
        list[3 * r + 2] = h;
        ++r;
      }
  double *o = malloc(sizeof(double) * nrows * D), *lse = malloc(sizeof(double) * nrows);
  orc_attend_rows(&P, nrows, list, o, lse, 3);
  int bad = 0;
  for (r = 0; r < nrows; ++r) {
    const int b = list[3 * r], i = list[3 * r + 1];
    const int exists = !ragged || i < rows[b];
    for (int c = 0; c < D; ++c)
      if (exists && !isfinite(o[r * D + c])) bad = 1;
  }
  /* split + merge of one row over uneven partitions (one empty) */
  double op[3 * D], m[3], l[3], om[D], lm;
  const int64_t cuts[4] = {0, 17, 17, 80};
  for (int p = 0; p < 3; ++p) orc_attend_partial(&P, 0, n_q - 1, 1, cuts[p], cuts[p + 1], op + p * D, &m[p], &l[p]);
  orc_merge(3, D, op, m, l, sinks[1], om, &lm);
  for (int c = 0; c < D; ++c)
    if (!isfinite(om[c])) bad = 1;
  /* gather of the sequence past the capacity */
  double *kg = malloc(sizeof(double) * STRIDE * PS * D), *vg = malloc(sizeof(double) * STRIDE * PS * D);
  orc_gather(&P, 0, 1, kg, vg);
  free(kg); free(vg);
  free(k); free(v); free(q); free(mask); free(kvs); free(vvs); free(list); free(o); free(lse);
  return bad;
}

int main(void) {
  int bad = 0;
  const int32_t dts[5] = {ORC_F32, ORC_F16, ORC_BF16, ORC_E4M3, ORC_E5M2};
  for (int t = 0; t < 5; ++t)
    for (int n_q = 1; n_q <= 40; n_q += 39)
      for (int mask = 0; mask < 2; ++mask)
        for (int ragged = 0; ragged < 2; ++ragged) {
          bad |= run_case(dts[t], n_q, mask, 0, ragged);
          if (dts[t] >= ORC_E4M3) bad |= run_case(dts[t], n_q, mask, 1, ragged);
        }
  /* encoders on special values */
  const float sp[10] = {0.0f, -0.0f, 1e-30f, -1e-30f, 448.0f, 464.0f, 1e9f, -1e9f, INFINITY, NAN};
  uint8_t c8[10];
  uint16_t c16[10];
  float sc[1];
  orc_encode_array(ORC_E4M3, 10, sp, 1.0f, c8);
  orc_encode_array(ORC_E5M2, 10, sp, 1.0f, c8);
  orc_encode_array(ORC_BF16, 10, sp, 1.0f, c16);
  orc_encode_array(ORC_F16, 10, sp, 1.0f, c16);
  orc_vector_scales(1, 10, sp, 448.0f, sc);
  orc_encode_vectors(ORC_E4M3, 1, 10, sp, sc, c8);
  double dec[256];
  uint8_t all[256];
  for (int i = 0; i < 256; ++i) all[i] = (uint8_t)i;
  orc_decode_array(ORC_E4M3, all, 256, dec);
  orc_decode_array(ORC_E5M2, all, 256, dec);
  printf("oracle driver: %s\n", bad ? "non-finite output" : "ok");
  return bad;
}
