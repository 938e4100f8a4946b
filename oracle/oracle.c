/*
 * oracle.c -- the CPU oracle of the DLRMv1 forward hot path.  TEST
 * INFRASTRUCTURE ONLY (see oracle.h for who may call it).  Written for a
 * reader checking it against the pages by eye: plain loops, fp64 sums, one
 * rounding to float32 per output element, no blocking, fusion or reordering.
 *
 * Built with: gcc -O2 -ffp-contract=off -fno-fast-math (oracle/build.py), so
 * that no multiply-add is contracted and the compiler keeps IEEE semantics.
 *
 * [FASTPATHS] = page "luminal_python: vanilla-PyTorch DLRMv1 fast paths +
 *               batched FFI + input cache" (compare main...vanilla-pytorch).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

int64_t oracle_pair_count(int64_t F) {
  if (F < 1) return 0;
  return F * (F - 1) / 2;
}

/* [FASTPATHS] dlrm_interact.rs: pairs in strict-lower-triangle order, row
 * by row, the order of torch.tril_indices(F, F, -1): (1,0),(2,0),(2,1),... */
int oracle_pair_enumerate(int64_t F, int32_t *pi, int32_t *pj) {
  if (F < 1 || F > 2147483647LL || !pi || !pj) return -1;
  int64_t p = 0;
  for (int64_t i = 1; i < F; ++i) {
    for (int64_t j = 0; j < i; ++j) {
      pi[p] = (int32_t)i;
      pj[p] = (int32_t)j;
      ++p;
    }
  }
  return 0;
}

/* [FASTPATHS] dlrm_interact.rs, PairwiseDotLowerTriStackedKernel layout
 * notes: row i of the strict lower triangle holds i pairs and starts at
 * linear index i(i-1)/2, hence i = floor((1 + sqrt(1 + 8p)) / 2) and
 * j = p - i(i-1)/2.  The floating square root may land one row off for large
 * p; the two integer corrections below restore i(i-1)/2 <= p < i(i+1)/2. */
int oracle_pair_closed_form(int64_t p, int64_t *i_out, int64_t *j_out) {
  if (p < 0 || !i_out || !j_out) return -1;
  int64_t i = (int64_t)floor((1.0 + sqrt(1.0 + 8.0 * (double)p)) / 2.0);
  while (i * (i - 1) / 2 > p) --i;
  while ((i + 1) * i / 2 <= p) ++i;
  *i_out = i;
  *j_out = p - i * (i - 1) / 2;
  return 0;
}

int oracle_pair_closed_form_range(int64_t p0, int64_t n, int32_t *pi,
                                  int32_t *pj) {
  if (p0 < 0 || n < 0 || !pi || !pj) return -1;
  for (int64_t t = 0; t < n; ++t) {
    int64_t i, j;
    oracle_pair_closed_form(p0 + t, &i, &j);
    pi[t] = (int32_t)i;
    pj[t] = (int32_t)j;
  }
  return 0;
}

/* [FASTPATHS] embedding_bag.rs, module doc "Semantics":
 *   out[b, d] = sum_l table[indices[b, l], d]
 * extended to K tables by MultiTableEmbeddingBagSumKernel (output laid out
 * (batch, num_tables, d)), and to explicit offsets by the reading that an
 * offsets array is torch.nn.EmbeddingBag's CSR bag start list. */
int oracle_emb_bag_sum(int32_t K, int32_t B, int32_t D,
                       const float *const *tables, const int64_t *rows,
                       const int32_t *const *indices,
                       const int32_t *const *offsets, const int64_t *n_idx,
                       float *out) {
  if (K < 1 || B < 1 || D < 1 || !tables || !rows || !indices || !n_idx ||
      !out)
    return -1;
  for (int32_t k = 0; k < K; ++k) {
    if (!tables[k] || rows[k] < 1 || n_idx[k] < 0) return -1;
    if (n_idx[k] > 0 && !indices[k]) return -1;
    if (offsets == NULL && n_idx[k] % B != 0) return -4;
    if (offsets != NULL && !offsets[k]) return -1;
  }
  for (int32_t k = 0; k < K; ++k) {
    const float *W = tables[k];
    const int32_t *idx = indices[k];
    for (int32_t b = 0; b < B; ++b) {
      int64_t start, end;
      if (offsets == NULL) {
        int64_t L = n_idx[k] / B;
        start = (int64_t)b * L;
        end = start + L;
      } else {
        start = offsets[k][b];
        end = (b + 1 < B) ? (int64_t)offsets[k][b + 1] : n_idx[k];
        if (start < 0 || end < start || end > n_idx[k]) return -3;
      }
      for (int32_t d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t l = start; l < end; ++l) {
          int64_t r = idx[l];
          if (r < 0 || r >= rows[k]) return -2;
          acc += (double)W[r * (int64_t)D + d];
        }
        out[((int64_t)b * K + k) * D + d] = (float)acc;
      }
    }
  }
  return 0;
}

float oracle_bf16_to_f32(uint16_t b) {
  uint32_t bits = (uint32_t)b << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

double oracle_fp8_e4m3_to_f64(uint8_t c) {
  const int sign = c >> 7;
  const int expo = (c >> 3) & 15;
  const int man = c & 7;
  double v;
  if (expo == 15 && man == 7) return NAN;
  if (expo == 0)
    v = ldexp((double)man, -9);             /* subnormal: (m / 8) x 2^(1 - 7) */
  else
    v = ldexp((double)(8 + man), expo - 10); /* (1 + m / 8) x 2^(e - 7) */
  return sign ? -v : v;
}

/* The sum of oracle_emb_bag_sum with the two torch.nn.EmbeddingBag options
 * the pages' lowering rejects: mean pooling and per-sample weights, and with
 * bfloat16 table storage.  Every term is formed and summed in double. */
int oracle_emb_bag(int32_t K, int32_t B, int32_t D, int32_t table_dtype,
                   const void *const *tables, const int64_t *rows,
                   const int32_t *const *indices, const int32_t *const *offsets,
                   const float *const *weights, const int64_t *n_idx, int32_t pool,
                   const float *scales, float *out) {
  if (K < 1 || B < 1 || D < 1 || !tables || !rows || !indices || !n_idx || !out)
    return -1;
  if (table_dtype != ORACLE_F32 && table_dtype != ORACLE_BF16 &&
      table_dtype != ORACLE_FP8_E4M3)
    return -6;
  if (pool != ORACLE_POOL_SUM && pool != ORACLE_POOL_MEAN) return -6;
  if (weights && pool != ORACLE_POOL_SUM) return -6;
  for (int32_t k = 0; k < K; ++k) {
    if (!tables[k] || rows[k] < 1 || n_idx[k] < 0) return -1;
    if (n_idx[k] > 0 && !indices[k]) return -1;
    if (weights && n_idx[k] > 0 && !weights[k]) return -1;
    if (offsets == NULL && n_idx[k] % B != 0) return -4;
    if (offsets != NULL && !offsets[k]) return -1;
  }
  for (int32_t k = 0; k < K; ++k) {
    const int32_t *idx = indices[k];
    for (int32_t b = 0; b < B; ++b) {
      int64_t start, end;
      if (offsets == NULL) {
        int64_t L = n_idx[k] / B;
        start = (int64_t)b * L;
        end = start + L;
      } else {
        start = offsets[k][b];
        end = (b + 1 < B) ? (int64_t)offsets[k][b + 1] : n_idx[k];
        if (start < 0 || end < start || end > n_idx[k]) return -3;
      }
      for (int32_t d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t l = start; l < end; ++l) {
          int64_t r = idx[l];
          if (r < 0 || r >= rows[k]) return -2;
          int64_t e = r * (int64_t)D + d;
          double v;
          if (table_dtype == ORACLE_BF16)
            v = (double)oracle_bf16_to_f32(((const uint16_t *)tables[k])[e]);
          else if (table_dtype == ORACLE_FP8_E4M3)
            v = oracle_fp8_e4m3_to_f64(((const uint8_t *)tables[k])[e]);
          else
            v = (double)((const float *)tables[k])[e];
          double w = weights ? (double)weights[k][l] : 1.0;
          acc += w * v;
        }
        if (pool == ORACLE_POOL_MEAN && end > start) acc /= (double)(end - start);
        if (scales) acc *= (double)scales[k];
        out[((int64_t)b * K + k) * D + d] = (float)acc;
      }
    }
  }
  return 0;
}

/* [FASTPATHS] translator dispatch, pairwise-dot peephole:
 *   T = cat([dense.unsqueeze(1)] + [e.unsqueeze(1) for e in ly], dim=1)
 *   Z = bmm(T, T^T);   dots = Z[:, li, lj] with (li, lj) = tril_indices(F, F, -1)
 * and the top MLP's input cat(dense, dots).  Z is formed in full and the
 * strict lower triangle is read out row by row, exactly that definition. */
int oracle_interact(int32_t B, int32_t K, int32_t D, const float *dense,
                    const float *emb, float *out) {
  if (B < 1 || K < 1 || D < 1 || !dense || !emb || !out) return -1;
  const int64_t F = (int64_t)K + 1;
  const int64_t P = oracle_pair_count(F);
  const int64_t width = (int64_t)D + P;
  double *X = (double *)malloc(sizeof(double) * (size_t)(F * D));
  double *Z = (double *)malloc(sizeof(double) * (size_t)(F * F));
  if (!X || !Z) {
    free(X);
    free(Z);
    return -5;
  }
  for (int32_t b = 0; b < B; ++b) {
    /* Feature 0 is the dense vector, features 1..K the pooled tables. */
    for (int32_t d = 0; d < D; ++d) X[d] = (double)dense[(int64_t)b * D + d];
    for (int32_t k = 0; k < K; ++k)
      for (int32_t d = 0; d < D; ++d)
        X[(int64_t)(k + 1) * D + d] =
            (double)emb[((int64_t)b * K + k) * D + d];
    /* Full Gram matrix Z = X X^T. */
    for (int64_t i = 0; i < F; ++i) {
      for (int64_t j = 0; j < F; ++j) {
        double acc = 0.0;
        for (int32_t d = 0; d < D; ++d) acc += X[i * D + d] * X[j * D + d];
        Z[i * F + j] = acc;
      }
    }
    float *row = out + (int64_t)b * width;
    memcpy(row, dense + (int64_t)b * D, sizeof(float) * (size_t)D);
    int64_t p = 0;
    for (int64_t i = 1; i < F; ++i)
      for (int64_t j = 0; j < i; ++j) row[D + p++] = (float)Z[i * F + j];
  }
  free(X);
  free(Z);
  return 0;
}

/* [FASTPATHS] matmul2d.rs: C = act(A B^T + bias) with B the (N, K) weight as
 * stored by nn.Linear; ReLU and Sigmoid applied in the store path. */
int oracle_linear(int32_t M, int32_t N, int32_t Kd, const float *A,
                  int64_t lda, const float *W, const float *bias, int32_t act,
                  float *C, int64_t ldc) {
  if (M < 1 || N < 1 || Kd < 1 || !A || !W || !C || lda < Kd || ldc < N)
    return -1;
  if (act != ORACLE_ACT_NONE && act != ORACLE_ACT_RELU &&
      act != ORACLE_ACT_SIGMOID)
    return -1;
  for (int32_t m = 0; m < M; ++m) {
    for (int32_t n = 0; n < N; ++n) {
      double acc = bias ? (double)bias[n] : 0.0;
      for (int32_t k = 0; k < Kd; ++k)
        acc += (double)A[(int64_t)m * lda + k] *
               (double)W[(int64_t)n * Kd + k];
      if (act == ORACLE_ACT_RELU) acc = acc > 0.0 ? acc : 0.0;
      if (act == ORACLE_ACT_SIGMOID) acc = 1.0 / (1.0 + exp(-acc));
      C[(int64_t)m * ldc + n] = (float)acc;
    }
  }
  return 0;
}

/* Runs a stack of layers; returns a malloc'd (B, last width) buffer. */
static float *run_mlp(int32_t B, int32_t n, const oracle_layer *layers,
                      const float *x, int32_t x_width, int *err) {
  float *cur = (float *)malloc(sizeof(float) * (size_t)B * (size_t)x_width);
  if (!cur) {
    *err = -5;
    return NULL;
  }
  memcpy(cur, x, sizeof(float) * (size_t)B * (size_t)x_width);
  int32_t width = x_width;
  for (int32_t l = 0; l < n; ++l) {
    if (layers[l].in_features != width) {
      free(cur);
      *err = -1;
      return NULL;
    }
    int32_t w_out = layers[l].out_features;
    float *next = (float *)malloc(sizeof(float) * (size_t)B * (size_t)w_out);
    if (!next) {
      free(cur);
      *err = -5;
      return NULL;
    }
    int rc = oracle_linear(B, w_out, width, cur, width, layers[l].weight,
                           layers[l].bias, layers[l].act, next, w_out);
    free(cur);
    if (rc) {
      free(next);
      *err = rc;
      return NULL;
    }
    cur = next;
    width = w_out;
  }
  *err = 0;
  return cur;
}

int oracle_forward(int32_t B, int32_t num_bottom, const oracle_layer *bottom,
                   int32_t num_top, const oracle_layer *top, int32_t K,
                   int32_t D, const float *const *tables, const int64_t *rows,
                   const float *dense_in, const int32_t *const *indices,
                   const int32_t *const *offsets, const int64_t *n_idx,
                   float *out, float *r_out, float *e_out) {
  if (B < 1 || num_bottom < 1 || num_top < 1 || !bottom || !top || !dense_in ||
      !out)
    return -1;
  if (bottom[num_bottom - 1].out_features != D) return -1;
  const int64_t P = oracle_pair_count((int64_t)K + 1);
  if (top[0].in_features != D + P) return -1;
  int err = 0;
  float *d = run_mlp(B, num_bottom, bottom, dense_in, bottom[0].in_features,
                     &err);
  if (!d) return err;
  float *E = (float *)malloc(sizeof(float) * (size_t)B * (size_t)K * (size_t)D);
  float *R = (float *)malloc(sizeof(float) * (size_t)B * (size_t)(D + P));
  if (!E || !R) {
    free(d);
    free(E);
    free(R);
    return -5;
  }
  err = oracle_emb_bag_sum(K, B, D, tables, rows, indices, offsets, n_idx, E);
  if (!err) err = oracle_interact(B, K, D, d, E, R);
  float *y = NULL;
  if (!err) y = run_mlp(B, num_top, top, R, (int32_t)(D + P), &err);
  if (!err) {
    int32_t w = top[num_top - 1].out_features;
    memcpy(out, y, sizeof(float) * (size_t)B * (size_t)w);
    if (r_out) memcpy(r_out, R, sizeof(float) * (size_t)B * (size_t)(D + P));
    if (e_out) memcpy(e_out, E, sizeof(float) * (size_t)B * (size_t)K * D);
  }
  free(d);
  free(E);
  free(R);
  free(y);
  return err;
}
