/*
 * sanitize_driver.c -- runs every entry point of the CPU oracle (oracle.c)
 * over small seeded cases, built together with it under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  TEST INFRASTRUCTURE ONLY (run by
 * tests/test_oracle_sanitized.py).
 *
 * Every buffer is a heap allocation of exactly the size the oracle's contract
 * gives it, so a read or write one element outside it is reported.  The
 * cases include the edges of the contract: empty bags (first and last, CSR),
 * tables with no indices, L = 0, one table, D = 1, the two narrow storage
 * types with every code, mean pooling, per-sample weights, strided linear
 * operands, and rejected arguments (which must return an error code without
 * touching memory out of bounds).  A few facts that do not depend on the
 * arithmetic's rounding are checked on the way (bag of k copies of one row,
 * dense copy, pair map against the double loop); the values themselves are
 * pinned by the Python pins.
 *
 * Exit status 0 when every case ran and every check held; the sanitizers
 * abort the process on the first error they find.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static int g_checks = 0;
static int g_failed = 0;

static uint64_t next_u64(void) {
  /* xorshift64* (Vigna) */
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return g_state * 0x2545F4914F6CDD1Dull;
}
static int32_t rand_below(int32_t n) { return (int32_t)(next_u64() % (uint64_t)n); }
static float rand_unit(void) {  /* dyadic values n / 256, |n| < 128 */
  return (float)((int32_t)(next_u64() % 255u) - 127) / 256.0f;
}

static void *xmalloc(size_t n) {
  void *p = malloc(n ? n : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}
static float *rand_floats(size_t n) {
  float *p = (float *)xmalloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) p[i] = rand_unit();
  return p;
}
static int32_t *rand_indices(size_t n, int32_t rows) {
  int32_t *p = (int32_t *)xmalloc(n * sizeof(int32_t));
  for (size_t i = 0; i < n; ++i) p[i] = rand_below(rows);
  return p;
}

static void check(int ok, const char *what) {
  ++g_checks;
  if (!ok) {
    ++g_failed;
    fprintf(stderr, "check failed: %s\n", what);
  }
}

/* ---------------------------------------------------------------- pairs -- */
static void run_pairs(void) {
  for (int64_t F = 1; F <= 300; F += (F < 20 ? 1 : 37)) {
    const int64_t P = oracle_pair_count(F);
    int32_t *pi = (int32_t *)xmalloc((size_t)P * sizeof(int32_t));
    int32_t *pj = (int32_t *)xmalloc((size_t)P * sizeof(int32_t));
    int32_t *ci = (int32_t *)xmalloc((size_t)P * sizeof(int32_t));
    int32_t *cj = (int32_t *)xmalloc((size_t)P * sizeof(int32_t));
    check(oracle_pair_enumerate(F, pi, pj) == 0, "pair_enumerate");
    check(oracle_pair_closed_form_range(0, P, ci, cj) == 0, "pair_closed_form_range");
    int same = 1;
    for (int64_t p = 0; p < P; ++p) same &= (pi[p] == ci[p] && pj[p] == cj[p]);
    check(same, "closed form == double loop");
    free(pi);
    free(pj);
    free(ci);
    free(cj);
  }
  int64_t i, j;
  check(oracle_pair_closed_form((int64_t)1 << 40, &i, &j) == 0, "closed form at 2^40");
  check(i * (i - 1) / 2 <= ((int64_t)1 << 40) && ((int64_t)1 << 40) < i * (i + 1) / 2,
        "row start inequality at 2^40");
}

/* ------------------------------------------------------------- emb-bags -- */
typedef struct {
  int32_t K, B, D;
  int csr;
  float **tab;
  int64_t *rows;
  int32_t **idx;
  int32_t **off;
  int64_t *n_idx;
} bags;

/* K tables; table k has rows_k rows; uniform bags of L_k = k % 3 + lmin, or
 * CSR bags with sizes 0..4 (first and last bag of every table empty). */
static bags make_bags(int32_t K, int32_t B, int32_t D, int csr, int lmin) {
  bags g;
  g.K = K;
  g.B = B;
  g.D = D;
  g.csr = csr;
  g.tab = (float **)xmalloc((size_t)K * sizeof(float *));
  g.rows = (int64_t *)xmalloc((size_t)K * sizeof(int64_t));
  g.idx = (int32_t **)xmalloc((size_t)K * sizeof(int32_t *));
  g.off = csr ? (int32_t **)xmalloc((size_t)K * sizeof(int32_t *)) : NULL;
  g.n_idx = (int64_t *)xmalloc((size_t)K * sizeof(int64_t));
  for (int32_t k = 0; k < K; ++k) {
    g.rows[k] = 1 + rand_below(9);
    g.tab[k] = rand_floats((size_t)g.rows[k] * (size_t)D);
    if (csr) {
      g.off[k] = (int32_t *)xmalloc((size_t)B * sizeof(int32_t));
      int64_t n = 0;
      for (int32_t b = 0; b < B; ++b) {
        g.off[k][b] = (int32_t)n;
        const int32_t len = (b == 0 || b == B - 1) ? 0 : rand_below(5);
        n += len;
      }
      g.n_idx[k] = n;
    } else {
      g.n_idx[k] = (int64_t)B * (k % 3 + lmin);
    }
    g.idx[k] = rand_indices((size_t)g.n_idx[k], (int32_t)g.rows[k]);
  }
  return g;
}

static void free_bags(bags *g) {
  for (int32_t k = 0; k < g->K; ++k) {
    free(g->tab[k]);
    free(g->idx[k]);
    if (g->csr) free(g->off[k]);
  }
  free(g->tab);
  free(g->rows);
  free(g->idx);
  free(g->off);
  free(g->n_idx);
}

static void run_emb_bag_sum(void) {
  const int32_t shapes[][3] = {{3, 7, 5}, {1, 1, 1}, {4, 9, 16}, {2, 3, 3}};
  for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
    for (int csr = 0; csr < 2; ++csr) {
      for (int lmin = 0; lmin < 2; ++lmin) {
        bags g = make_bags(shapes[s][0], shapes[s][1], shapes[s][2], csr, lmin);
        float *out = (float *)xmalloc((size_t)g.K * g.B * g.D * sizeof(float));
        check(oracle_emb_bag_sum(g.K, g.B, g.D, (const float *const *)g.tab, g.rows,
                                 (const int32_t *const *)g.idx,
                                 (const int32_t *const *)g.off, g.n_idx, out) == 0,
              "emb_bag_sum");
        free(out);
        free_bags(&g);
      }
    }
  }
  /* a bag of k copies of one row is k times the row, exactly */
  const int32_t D = 6, kcopies = 7;
  float *t = rand_floats(3 * (size_t)D);
  int32_t *ix = (int32_t *)xmalloc(kcopies * sizeof(int32_t));
  for (int l = 0; l < kcopies; ++l) ix[l] = 2;
  const float *tabs[1] = {t};
  const int32_t *ixs[1] = {ix};
  const int64_t rows[1] = {3}, n[1] = {kcopies};
  float *out = (float *)xmalloc((size_t)D * sizeof(float));
  check(oracle_emb_bag_sum(1, 1, D, tabs, rows, ixs, NULL, n, out) == 0, "k copies");
  int same = 1;
  for (int d = 0; d < D; ++d) same &= out[d] == (float)(kcopies * (double)t[2 * D + d]);
  check(same, "bag of k copies == k x row");
  /* rejected arguments: out-of-range index, bad offsets, n_idx % B */
  ix[3] = 3;
  check(oracle_emb_bag_sum(1, 1, D, tabs, rows, ixs, NULL, n, out) == -2, "index >= rows");
  ix[3] = -1;
  check(oracle_emb_bag_sum(1, 1, D, tabs, rows, ixs, NULL, n, out) == -2, "negative index");
  ix[3] = 2;
  int32_t *bad_off = (int32_t *)xmalloc(2 * sizeof(int32_t));
  bad_off[0] = 5;
  bad_off[1] = 2;
  const int32_t *offs[1] = {bad_off};
  float *out2 = (float *)xmalloc(2 * (size_t)D * sizeof(float));  /* B = 2 */
  check(oracle_emb_bag_sum(1, 2, D, tabs, rows, ixs, offs, n, out2) == -3,
        "decreasing offsets");
  check(oracle_emb_bag_sum(1, 2, D, tabs, rows, ixs, NULL, n, out2) == -4, "n_idx % B");
  free(out2);
  free(bad_off);
  free(out);
  free(ix);
  free(t);
}

static void run_emb_bag_forms(void) {
  /* every bf16 pattern and fp8 code converts without undefined behaviour */
  int nan8 = 0;
  for (int c = 0; c < 256; ++c) nan8 += isnan(oracle_fp8_e4m3_to_f64((uint8_t)c)) ? 1 : 0;
  check(nan8 == 2, "two fp8 NaN codes");
  check(oracle_fp8_e4m3_to_f64(0x7e) == 448.0, "fp8 max 448");
  for (uint32_t b = 0; b < 65536u; ++b) (void)oracle_bf16_to_f32((uint16_t)b);
  check(oracle_bf16_to_f32(0x3f80) == 1.0f, "bf16 1.0");

  const int32_t K = 3, B = 6, D = 5;
  for (int dtype = 0; dtype < 3; ++dtype) {
    for (int csr = 0; csr < 2; ++csr) {
      for (int form = 0; form < 3; ++form) {  /* sum, mean, weighted sum */
        bags g = make_bags(K, B, D, csr, 1);
        void **tabs = (void **)xmalloc((size_t)K * sizeof(void *));
        for (int32_t k = 0; k < K; ++k) {
          const size_t n = (size_t)g.rows[k] * (size_t)D;
          if (dtype == ORACLE_F32) {
            tabs[k] = g.tab[k];
          } else if (dtype == ORACLE_BF16) {
            uint16_t *p = (uint16_t *)xmalloc(n * sizeof(uint16_t));
            for (size_t i = 0; i < n; ++i) p[i] = (uint16_t)next_u64();
            tabs[k] = p;
          } else {
            uint8_t *p = (uint8_t *)xmalloc(n);
            for (size_t i = 0; i < n; ++i) p[i] = (uint8_t)(next_u64() & 0x77u); /* no NaN */
            tabs[k] = p;
          }
        }
        float **w = NULL;
        if (form == 2) {
          w = (float **)xmalloc((size_t)K * sizeof(float *));
          for (int32_t k = 0; k < K; ++k) w[k] = rand_floats((size_t)g.n_idx[k]);
        }
        float *sc = rand_floats((size_t)K);
        float *out = (float *)xmalloc((size_t)K * B * D * sizeof(float));
        check(oracle_emb_bag(K, B, D, dtype, (const void *const *)tabs, g.rows,
                             (const int32_t *const *)g.idx, (const int32_t *const *)g.off,
                             (const float *const *)w, g.n_idx,
                             form == 1 ? ORACLE_POOL_MEAN : ORACLE_POOL_SUM,
                             form == 0 ? NULL : sc, out) == 0,
              "emb_bag form");
        if (form == 1) {
          /* weights with mean pooling are rejected */
          float **w1 = (float **)xmalloc((size_t)K * sizeof(float *));
          for (int32_t k = 0; k < K; ++k) w1[k] = rand_floats((size_t)g.n_idx[k]);
          check(oracle_emb_bag(K, B, D, dtype, (const void *const *)tabs, g.rows,
                               (const int32_t *const *)g.idx, (const int32_t *const *)g.off,
                               (const float *const *)w1, g.n_idx, ORACLE_POOL_MEAN, NULL,
                               out) == -6,
                "weights with mean rejected");
          for (int32_t k = 0; k < K; ++k) free(w1[k]);
          free(w1);
        }
        free(out);
        free(sc);
        if (w) {
          for (int32_t k = 0; k < K; ++k) free(w[k]);
          free(w);
        }
        if (dtype != ORACLE_F32)
          for (int32_t k = 0; k < K; ++k) free(tabs[k]);
        free(tabs);
        free_bags(&g);
      }
    }
  }
}

/* ---------------------------------------------------------- interaction -- */
static void run_interact(void) {
  const int32_t shapes[][3] = {{5, 1, 4}, {3, 6, 7}, {1, 2, 1}, {4, 26, 16}};
  for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
    const int32_t B = shapes[s][0], K = shapes[s][1], D = shapes[s][2];
    const int64_t P = oracle_pair_count(K + 1);
    float *dense = rand_floats((size_t)B * D);
    float *emb = rand_floats((size_t)B * K * D);
    float *out = (float *)xmalloc((size_t)B * (D + P) * sizeof(float));
    check(oracle_interact(B, K, D, dense, emb, out) == 0, "interact");
    int same = 1;
    for (int32_t b = 0; b < B; ++b)
      for (int32_t d = 0; d < D; ++d) same &= out[(size_t)b * (D + P) + d] == dense[b * D + d];
    check(same, "interact copies dense");
    free(dense);
    free(emb);
    free(out);
  }
}

/* --------------------------------------------------------------- linear -- */
static void run_linear(void) {
  const int32_t shapes[][5] = {  /* M, N, K, lda pad, ldc pad */
      {1, 1, 1, 0, 0}, {7, 5, 3, 2, 1}, {4, 9, 13, 0, 3}, {3, 1, 8, 1, 0}};
  for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
    const int32_t M = shapes[s][0], N = shapes[s][1], Kd = shapes[s][2];
    const int64_t lda = Kd + shapes[s][3], ldc = N + shapes[s][4];
    /* the last row of a strided matrix ends at its last used column */
    float *A = rand_floats((size_t)((M - 1) * lda + Kd));
    float *W = rand_floats((size_t)N * Kd);
    float *bias = rand_floats((size_t)N);
    float *C = (float *)xmalloc((size_t)((M - 1) * ldc + N) * sizeof(float));
    for (int act = 0; act < 3; ++act) {
      check(oracle_linear(M, N, Kd, A, lda, W, bias, act, C, ldc) == 0, "linear");
      check(oracle_linear(M, N, Kd, A, lda, W, NULL, act, C, ldc) == 0, "linear no bias");
    }
    free(A);
    free(W);
    free(bias);
    free(C);
  }
}

/* -------------------------------------------------------------- forward -- */
static void run_forward(void) {
  const int32_t B = 5, K = 3, D = 4, in0 = 3;
  const int64_t P = oracle_pair_count(K + 1);
  const int32_t bw[] = {in0, 8, D}, tw[] = {D + (int32_t)P, 6, 1};
  oracle_layer bottom[2], top[2];
  float *mem[8];
  int nm = 0;
  for (int l = 0; l < 2; ++l) {
    bottom[l].in_features = bw[l];
    bottom[l].out_features = bw[l + 1];
    bottom[l].weight = mem[nm++] = rand_floats((size_t)bw[l] * bw[l + 1]);
    bottom[l].bias = mem[nm++] = rand_floats((size_t)bw[l + 1]);
    bottom[l].act = ORACLE_ACT_RELU;
    top[l].in_features = tw[l];
    top[l].out_features = tw[l + 1];
    top[l].weight = mem[nm++] = rand_floats((size_t)tw[l] * tw[l + 1]);
    top[l].bias = mem[nm++] = rand_floats((size_t)tw[l + 1]);
    top[l].act = l == 1 ? ORACLE_ACT_SIGMOID : ORACLE_ACT_RELU;
  }
  for (int csr = 0; csr < 2; ++csr) {
    bags g = make_bags(K, B, D, csr, 1);
    float *dense = rand_floats((size_t)B * in0);
    float *out = (float *)xmalloc((size_t)B * sizeof(float));
    float *r = (float *)xmalloc((size_t)B * (D + P) * sizeof(float));
    float *e = (float *)xmalloc((size_t)B * K * D * sizeof(float));
    check(oracle_forward(B, 2, bottom, 2, top, K, D, (const float *const *)g.tab, g.rows, dense,
                         (const int32_t *const *)g.idx, (const int32_t *const *)g.off, g.n_idx,
                         out, r, e) == 0,
          "forward");
    check(oracle_forward(B, 2, bottom, 2, top, K, D, (const float *const *)g.tab, g.rows, dense,
                         (const int32_t *const *)g.idx, (const int32_t *const *)g.off, g.n_idx,
                         out, NULL, NULL) == 0,
          "forward without copies");
    int ok = 1;
    for (int32_t b = 0; b < B; ++b) ok &= out[b] >= 0.0f && out[b] <= 1.0f;
    check(ok, "sigmoid output in [0, 1]");
    free(dense);
    free(out);
    free(r);
    free(e);
    free_bags(&g);
  }
  for (int i = 0; i < nm; ++i) free(mem[i]);
}

int main(void) {
  run_pairs();
  run_emb_bag_sum();
  run_emb_bag_forms();
  run_interact();
  run_linear();
  run_forward();
  printf("sanitized oracle driver: %d checks, %d failed\n", g_checks, g_failed);
  return g_failed ? 1 : 0;
}
