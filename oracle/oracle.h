/*
 * oracle.h -- plain, slow, obviously-correct CPU implementation of the DLRMv1
 * forward hot path.  TEST INFRASTRUCTURE ONLY: it is called by tests/, by the
 * smoke check in __graft_entry__.py and by the cpu_baseline leg of bench.py,
 * and by nothing else.  It shares no code, header, table or constant with the
 * HIP library in dlrm_embedding_bag_amd/, and it never includes or links it.
 *
 * Citations name the web page they follow and the section on it:
 *   [FASTPATHS] = page "luminal_python: vanilla-PyTorch DLRMv1 fast paths +
 *                 batched FFI + input cache" (compare main...vanilla-pytorch)
 * followed by the file diff on that page and the item inside it.
 *
 * Precision: every sum is accumulated in double (fp64) and rounded once to
 * float32 per output element; every stage's output is float32, as on the
 * pages, where every tensor of the path is F32.
 *
 * All pointers are host pointers.  Return value: 0 on success, a negative
 * number when an argument is invalid (the oracle checks index and offset
 * ranges, which the GPU path takes as a precondition).
 */
#ifndef DLRM_ORACLE_H
#define DLRM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_ACT_NONE = 0, ORACLE_ACT_RELU = 1, ORACLE_ACT_SIGMOID = 2 };

/* Number of strict-lower-triangle pairs of an F x F matrix: F(F-1)/2. */
int64_t oracle_pair_count(int64_t F);

/* Enumerate the strict lower triangle row by row: i = 1..F-1, j = 0..i-1,
 * writing pair p's row into pi[p] and column into pj[p].  This is the order
 * of torch.tril_indices(F, F, -1) ([FASTPATHS] dlrm_interact.rs, doc of
 * dlrm_pairwise_dot_lower_tri). */
int oracle_pair_enumerate(int64_t F, int32_t *pi, int32_t *pj);

/* Recover (i, j) from the linear pair index p with the closed form the pages
 * give ([FASTPATHS] dlrm_interact.rs, PairwiseDotLowerTriStackedKernel
 * layout notes): row i starts at i(i-1)/2, so i = floor((1+sqrt(1+8p))/2),
 * j = p - i(i-1)/2.  The square root is taken in double and the row is then
 * corrected by integer tests so that i(i-1)/2 <= p < i(i+1)/2 holds exactly. */
int oracle_pair_closed_form(int64_t p, int64_t *i, int64_t *j);

/* The closed form applied to p = p0 .. p0+n-1 (for brute-force checks). */
int oracle_pair_closed_form_range(int64_t p0, int64_t n, int32_t *pi,
                                  int32_t *pj);

/* Multi-table EmbeddingBag, sum pooling ([FASTPATHS] embedding_bag.rs,
 * module doc "Semantics" and MultiTableEmbeddingBagSumKernel doc):
 *   out[b, k, :] = sum over l in bag(b, k) of tables[k][indices[k][l], :]
 * with bag(b, k) = [b*L_k, (b+1)*L_k), L_k = n_idx[k] / B, when offsets is
 * NULL (uniform stride), else the CSR bag [offsets[k][b], offsets[k][b+1])
 * whose last bag ends at n_idx[k] (torch.nn.EmbeddingBag offsets with
 * include_last_offset = False).  An empty bag pools to zeros.
 *   tables[k]  : (rows[k], D) float32 row-major
 *   indices[k] : (n_idx[k],) int32
 *   offsets    : NULL, or K pointers to (B,) int32
 *   out        : (B, K, D) float32 row-major
 * Errors: -1 bad sizes, -2 index out of [0, rows[k]), -3 bad offsets,
 *         -4 n_idx[k] not a multiple of B in uniform mode. */
int oracle_emb_bag_sum(int32_t K, int32_t B, int32_t D,
                       const float *const *tables, const int64_t *rows,
                       const int32_t *const *indices,
                       const int32_t *const *offsets, const int64_t *n_idx,
                       float *out);

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_FP8_E4M3 = 2 };
enum { ORACLE_POOL_SUM = 0, ORACLE_POOL_MEAN = 1 };

/* bfloat16 (the upper 16 bits of an IEEE float32) to float32: exact. */
float oracle_bf16_to_f32(uint16_t b);

/* FP8 E4M3 as the OCP 8-bit floating point format defines it (the "fn"
 * variant: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
 * subnormals at exponent 0, no infinities, S.1111.111 is NaN, largest finite
 * 448) to double: exact. */
double oracle_fp8_e4m3_to_f64(uint8_t c);

/* Generalised EmbeddingBag pooling, the adjacent semantics of the pages'
 * sum-only kernel ([FASTPATHS] translator dispatch, _embedding_bag lowering:
 * mode must be sum, per_sample_weights are rejected; torch.nn.EmbeddingBag
 * defines the rest):
 *   sum:  out[b,k,:] = sum over l in bag of w_l * row(idx[l])
 *   mean: out[b,k,:] = (sum over l in bag of row(idx[l])) / |bag|, 0 if empty
 * with w_l = weights[k][l] when weights is not NULL (sum only, as in torch),
 * else 1.  table_dtype ORACLE_BF16 means tables[k] holds uint16_t bfloat16
 * values, converted exactly to f32 before use; ORACLE_FP8_E4M3 means uint8_t
 * FP8 E4M3 codes (oracle_fp8_e4m3_to_f64).  scales: NULL, or K per-table
 * factors applied to the pooled value (out = scales[k] x pool(...)), which
 * lets narrow storage hold tables of any magnitude.  Bags as in
 * oracle_emb_bag_sum.  Errors: as oracle_emb_bag_sum, and -6 for weights
 * with mean pooling or an unknown dtype or pool. */
int oracle_emb_bag(int32_t K, int32_t B, int32_t D, int32_t table_dtype,
                   const void *const *tables, const int64_t *rows,
                   const int32_t *const *indices, const int32_t *const *offsets,
                   const float *const *weights, const int64_t *n_idx, int32_t pool,
                   const float *scales,
                   float *out);

/* Strict-lower-triangle pairwise-dot interaction ([FASTPATHS]
 * dlrm_interact.rs, PairwiseDotLowerTriStackedKernel; translator dispatch,
 * the Z[:, li, lj] over bmm(cat, permute) pattern).  Per sample b:
 *   X = [dense[b]; emb[b, 0]; ...; emb[b, K-1]]       (F x D, F = K + 1)
 *   Z = X X^T                                         (full F x F, fp64)
 *   out[b] = [dense[b] (copied bit for bit), Z[1][0], Z[2][0], Z[2][1], ...]
 *   dense : (B, D), emb : (B, K, D), out : (B, D + F(F-1)/2). */
int oracle_interact(int32_t B, int32_t K, int32_t D, const float *dense,
                    const float *emb, float *out);

/* Fused linear layer ([FASTPATHS] matmul2d.rs, Activation epilogue and the
 * linear_bias_relu / linear_bias_sigmoid frontends):
 *   C[m][n] = act(bias[n] + sum_k A[m][k] * W[n][k])
 * A : (M, Kd) row-major with row stride lda, W : (N, Kd) row-major (the
 * nn.Linear weight layout), bias : (N,) or NULL, C : (M, N) row stride ldc.
 * relu(x) = x > 0 ? x : 0; sigmoid(x) = 1 / (1 + exp(-x)), both in double. */
int oracle_linear(int32_t M, int32_t N, int32_t Kd, const float *A,
                  int64_t lda, const float *W, const float *bias, int32_t act,
                  float *C, int64_t ldc);

/* One MLP layer description for oracle_forward. */
typedef struct oracle_layer {
  int32_t in_features;
  int32_t out_features;
  const float *weight; /* (out_features, in_features) */
  const float *bias;   /* (out_features,) or NULL */
  int32_t act;         /* ORACLE_ACT_* */
} oracle_layer;

/* DLRMv1 forward ([FASTPATHS] commit message and translator notes: bottom MLP
 * on the dense input, one EmbeddingBag(sum) per table, pairwise-dot
 * interaction with the dense vector as feature 0, top MLP on
 * cat(dense, dots) ending in a sigmoid):
 *   d = bottom(dense_in)            (B, D)
 *   E = emb_bag_sum(...)            (B, K, D)
 *   R = interact(d, E)              (B, D + P)
 *   out = top(R)                    (B, top[last].out_features)
 * r_out (B, D + P) and e_out (B, K, D) are optional copies of R and E. */
int oracle_forward(int32_t B, int32_t num_bottom, const oracle_layer *bottom,
                   int32_t num_top, const oracle_layer *top, int32_t K,
                   int32_t D, const float *const *tables, const int64_t *rows,
                   const float *dense_in, const int32_t *const *indices,
                   const int32_t *const *offsets, const int64_t *n_idx,
                   float *out, float *r_out, float *e_out);

#ifdef __cplusplus
}
#endif

#endif /* DLRM_ORACLE_H */
