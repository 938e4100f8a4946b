/*
 * dlrm_embedding_bag.h -- C ABI of the MI355X (gfx950) DLRMv1 forward hot path.
 *
 * Library: libdlrm_mi355x.so (hand-written HIP kernels for CDNA4).
 *
 * Citations name the web page an operation follows and the section on it:
 *   [FASTPATHS] = page "luminal_python: vanilla-PyTorch DLRMv1 fast paths +
 *                 batched FFI + input cache" (compare main...vanilla-pytorch)
 *
 * Conventions shared by every call
 *  - Pointers are DEVICE pointers unless marked [host].  [host] arrays are
 *    read during the call only and may be freed as soon as it returns.
 *  - The caller owns every buffer.  The compute calls allocate no device
 *    memory and keep no pointer after they return ([FASTPATHS] runtime.rs:
 *    non-owning views over caller memory); dlrm_plan_create allocates host
 *    memory for the plan it returns.  The library holds two pieces of
 *    mutable state: the calling thread's kernel-timing events
 *    (dlrm_set_kernel_timing_events, measurement support, off unless a
 *    thread sets it) and the per-GPU scratch array of dlrm_forward_noalloc
 *    (shared by that call only).  Apart from them, calls on different
 *    streams or threads are independent and re-entrant.
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *    Every call only enqueues work on `stream` and never synchronizes
 *    ([FASTPATHS] runtime.rs: execute() stays capturable, no trailing sync).
 *  - Floating point data is float32, row-major and dense unless a leading
 *    dimension says otherwise.  Indices and offsets are int32 (the caller
 *    narrows int64 indices, as the pages' Python bridge does).
 *  - Outputs must not overlap inputs.
 *  - Return value: a dlrm_status.  Argument errors are reported before any
 *    work is enqueued; DLRM_ERR_HIP reports a failed launch.  A zero batch
 *    (or m == 0) is a no-op that returns DLRM_OK and reads no data pointer.
 *  - Index values are trusted, as on the pages ([FASTPATHS] embedding_bag.rs:
 *    the kernel trusts user indices): every index of table k must lie in
 *    [0, rows[k]); an index outside it is undefined behaviour.  Explicit
 *    offsets are clamped into [0, n_idx[k]] on the device, so a bad offset
 *    gives a wrong bag, never an out-of-bounds index read.
 *  - Vectorised paths are used when dim % 4 == 0 and the relevant pointers
 *    and leading dimensions are 16-byte aligned; anything else takes a scalar
 *    path.  Alignment is never an error.
 */
#ifndef DLRM_EMBEDDING_BAG_H
#define DLRM_EMBEDDING_BAG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define DLRM_API __attribute__((visibility("default")))
#else
#define DLRM_API
#endif

typedef enum dlrm_status {
  DLRM_OK = 0,
  DLRM_ERR_NULL = 1,        /* a required pointer is NULL                    */
  DLRM_ERR_SHAPE = 2,       /* a size is out of range or sizes disagree      */
  DLRM_ERR_UNSUPPORTED = 3, /* valid request beyond a documented limit       */
  DLRM_ERR_WORKSPACE = 4,   /* workspace smaller than required               */
  DLRM_ERR_HIP = 5          /* the HIP runtime reported an error             */
} dlrm_status;

typedef enum dlrm_act {
  DLRM_ACT_NONE = 0,
  DLRM_ACT_RELU = 1,   /* x > 0 ? x : 0                                     */
  DLRM_ACT_SIGMOID = 2 /* 1 / (1 + exp(-x))                                 */
} dlrm_act;

/* Documented limits. */
#define DLRM_MAX_TABLES 64        /* K per call (pointer table travels by value) */
#define DLRM_MAX_DIM 1024         /* embedding dim D                             */

/* Human-readable name of a status code (static string, never NULL). */
DLRM_API const char *dlrm_status_string(int status);

/* ABI version of this header (bumped on any incompatible change). */
DLRM_API int dlrm_abi_version(void);
#define DLRM_ABI_VERSION 2

/*
 * dlrm_set_kernel_timing_events -- per-kernel timing for benchmarks.
 * (Measurement support, not a step of the method: the pages time whole
 * forwards with CUDA events, RESULTS.md of [FASTPATHS]; this times one
 * kernel without the dispatch gap that events recorded around a call
 * include.)
 *
 *   start, stop  hipEvent_t handles created by the caller (default flags),
 *                or both NULL to switch timing off (the initial state).
 *
 * While set, every kernel that this library launches from the calling
 * thread is dispatched with hipExtLaunchKernel, which records `start` and
 * `stop` with that dispatch, so after a call that launches one kernel,
 * hipEventElapsedTime(start, stop) times that kernel without the gap that
 * events recorded around the call include (measured within a few percent
 * of a profiler's dispatch time); after a call that launches several, it
 * times the last one.  This is thread-local state of the library (the only
 * mutable state it keeps): it changes how the calling thread's later
 * launches are dispatched, never what they compute, and other threads are
 * unaffected.  The events stay owned by the caller, who must switch timing
 * off before destroying them.  Graph-mode plans capture plain launches
 * whatever the setting; a caller capturing its own stream must switch
 * timing off first.  Returns DLRM_ERR_NULL when exactly one of the two is
 * NULL (nothing changes), else DLRM_OK.
 */
DLRM_API int dlrm_set_kernel_timing_events(void *start, void *stop);

/*
 * dlrm_stream_read -- reads a device buffer once with a streaming-read
 * kernel (measurement support, not a step of the method: the practical HBM
 * read rate the gather's bytes are compared with, and a dispatch of known
 * read bytes for calibrating memory-traffic counters).
 *
 *   buf    device buffer, 16-byte aligned
 *   bytes  its size, a multiple of 16 (0: nothing to do, DLRM_OK)
 *   sink   device float32; written only when the bytes read hash to a value
 *          chosen not to occur (it keeps the reads from being optimised
 *          away), so its content is unspecified afterwards
 * One launch of 16-byte loads, 8 in flight per lane, up to 2048 workgroups
 * of 256 lanes.  Returns DLRM_ERR_NULL for a NULL buf or sink,
 * DLRM_ERR_SHAPE for a misaligned buffer or size.
 */
DLRM_API int dlrm_stream_read(const void *buf, size_t bytes, float *sink, void *stream);

/*
 * emb_bag_sum_multi -- K EmbeddingBag(sum) lookups in one launch
 * ([FASTPATHS] embedding_bag.rs, module doc "Semantics" and
 * MultiTableEmbeddingBagSumKernel doc; translator dispatch,
 * aten._embedding_bag_forward_only lowering):
 *
 *   out[b, k, :] = sum over l in bag(b, k) of tables[k][indices[k][l], :]
 *
 *   num_tables  K, 1 <= K <= DLRM_MAX_TABLES
 *   batch       B >= 0 (0: nothing to do, DLRM_OK)
 *   dim         D, 1 <= D <= DLRM_MAX_DIM (shared by all tables)
 *   tables      [host] K device pointers; table k is (rows[k], D) float32
 *   rows        [host] K row counts (>= 1; row counts may differ per table)
 *   indices     [host] K device pointers; indices[k] is (n_idx[k],) int32
 *   offsets     [host] NULL for uniform stride: bag(b, k) = [b*L_k, (b+1)*L_k)
 *               with L_k = n_idx[k] / B (n_idx[k] must be a multiple of B);
 *               or K device pointers to (B,) int32 bag starts (CSR, as
 *               torch.nn.EmbeddingBag with include_last_offset = False: the
 *               last bag ends at n_idx[k]; an empty bag pools to 0).
 *   n_idx       [host] K index counts, 0 <= n_idx[k] <= INT32_MAX
 *   out         (B, K, D) float32
 * Sum mode only; per-sample weights, padding_idx and include_last_offset are
 * not part of the pages' path and have no parameter here.
 */
DLRM_API int emb_bag_sum_multi(int32_t num_tables, int32_t batch, int32_t dim,
                      const float *const *tables, const int64_t *rows,
                      const int32_t *const *indices,
                      const int32_t *const *offsets, const int64_t *n_idx,
                      float *out, void *stream);

/*
 * dlrm_interact_lower_tri -- strict-lower-triangle pairwise-dot interaction
 * ([FASTPATHS] dlrm_interact.rs, PairwiseDotLowerTriStackedKernel: feature 0
 * is the dense vector, features 1..N the stacked embeddings; pair p = (i, j),
 * i > j, in torch.tril_indices(F, F, -1) order; translator dispatch: the top
 * MLP reads cat(dense, dots)):
 *
 *   X_b = [dense[b]; emb[b, 0]; ...; emb[b, N-1]]           F = N + 1 rows
 *   out[b, 0:D]       = dense[b]                             (exact copy)
 *   out[b, D + p]     = dot(X_b[i], X_b[j]),  (i, j) = pair p
 *
 *   batch    B >= 0 (0: nothing to do, DLRM_OK)
 *   num_emb  N, 1 <= N <= DLRM_MAX_TABLES
 *   dim      D, 1 <= D <= DLRM_MAX_DIM, with F * D * 4 bytes of features per
 *            sample fitting the 64 KiB shared-memory budget (else
 *            DLRM_ERR_UNSUPPORTED)
 *   dense    (B, D) float32
 *   emb      (B, N, D) float32
 *   out      (B, D + F(F-1)/2) float32
 */
DLRM_API int dlrm_interact_lower_tri(int32_t batch, int32_t num_emb, int32_t dim,
                            const float *dense, const float *emb, float *out,
                            void *stream);

/*
 * dlrm_emb_interact -- emb_bag_sum_multi fused with dlrm_interact_lower_tri
 * in one launch: the pooled vectors stay on chip and go straight into the
 * interaction ([FASTPATHS] commit message: the multi-table emb-bag kernel
 * feeding the stacked pairwise-dot kernel).  Arguments as in the two calls
 * above; emb_out, if not NULL, also receives the (B, K, D) pooled tensor.
 *   dense    (B, D) float32
 *   out      (B, D + F(F-1)/2) float32, F = K + 1
 * Long bags: when emb_out is given (16-byte aligned, D % 4 == 0) and the mean
 * bag pools at least 4096 elements (L x D), the call runs as two launches on
 * `stream`, the gather into emb_out and then the interaction reading it,
 * which is faster there; out and emb_out hold the same values either way.
 * emb_out must not overlap dense or out.
 */
DLRM_API int dlrm_emb_interact(int32_t num_tables, int32_t batch, int32_t dim,
                      const float *const *tables, const int64_t *rows,
                      const int32_t *const *indices,
                      const int32_t *const *offsets, const int64_t *n_idx,
                      const float *dense, float *out, float *emb_out,
                      void *stream);

/* Storage type of embedding-table rows. */
typedef enum dlrm_dtype {
  DLRM_F32 = 0,      /* IEEE float32                                          */
  DLRM_BF16 = 1,     /* bfloat16: the high 16 bits of a float32, widened exactly */
  DLRM_FP8_E4M3 = 2  /* OCP FP8 E4M3 ("fn": bias 7, subnormals, no infinities,
                        S.1111.111 NaN, max 448), one byte, decoded exactly   */
} dlrm_dtype;

/* How a bag's rows are combined (the modes of torch.nn.EmbeddingBag). */
typedef enum dlrm_pool {
  DLRM_POOL_SUM = 0,  /* sum of the rows (times their weights, if given)   */
  DLRM_POOL_MEAN = 1  /* sum divided by the bag size; an empty bag gives 0 */
} dlrm_pool;

/*
 * A set of K EmbeddingBag lookups over one batch, the general form of the
 * arguments of emb_bag_sum_multi.  Every array of this struct is [host]; the
 * tables, indices, offsets and weights they point to are device memory.
 *
 *   num_tables   K, 1 <= K <= DLRM_MAX_TABLES
 *   batch        B >= 0
 *   dim          D, 1 <= D <= DLRM_MAX_DIM
 *   table_dtype  a dlrm_dtype, shared by all K tables
 *   pool         a dlrm_pool
 *   tables       K device pointers; table k is (rows[k], D) of table_dtype
 *   rows, indices, offsets, n_idx   as in emb_bag_sum_multi (offsets NULL:
 *                uniform stride; else CSR bag starts)
 *   weights      NULL, or K device pointers: weights[k] is (n_idx[k],)
 *                float32, the per-sample weight of each index (the
 *                per_sample_weights of torch.nn.EmbeddingBag); sum pooling
 *                only (with DLRM_POOL_MEAN it is DLRM_ERR_UNSUPPORTED, as in
 *                torch)
 *   scales       NULL, or [host] K float32 factors: table k's pooled value is
 *                multiplied by scales[k] (what lets fp8 storage hold tables
 *                of any magnitude: store w / scale, get scale x pool)
 *
 * Pooling ([FASTPATHS] translator dispatch, aten._embedding_bag lowering:
 * the pages' path takes sum mode only and rejects per-sample weights; the
 * other options follow torch.nn.EmbeddingBag):
 *   sum   out[b, k, :] = sum_{l in bag(b,k)} w_l * row(tables[k], indices[k][l])
 *         with w_l = weights[k][l], or 1 without weights
 *   mean  out[b, k, :] = (sum_{l in bag(b,k)} row(...)) / |bag(b,k)|, 0 if empty
 * Rows of bfloat16 and fp8 tables are widened to float32 exactly;
 * accumulation is float32 in bag order, then mean and scale.
 * The vector path needs 16-byte rows chunks (dim % 4 == 0 for float32, 8 for
 * bfloat16, 16 for fp8) and 16-byte aligned tables and outputs; anything else
 * takes the scalar path.
 */
typedef struct dlrm_bags {
  int32_t num_tables;
  int32_t batch;
  int32_t dim;
  int32_t table_dtype;
  int32_t pool;
  const void *const *tables;
  const int64_t *rows;
  const int32_t *const *indices;
  const int32_t *const *offsets;
  const int64_t *n_idx;
  const float *const *weights;
  const float *scales;
} dlrm_bags;

/*
 * emb_bag_pool -- K EmbeddingBag lookups of any dlrm_bags form in one launch.
 *   bags   [host] the lookups
 *   out    (B, K, D) float32
 * A zero batch is a no-op.  emb_bag_sum_multi is this call with float32
 * tables, sum pooling and no weights.
 */
DLRM_API int emb_bag_pool(const dlrm_bags *bags, float *out, void *stream);

/*
 * dlrm_emb_interact_pool -- emb_bag_pool fused with dlrm_interact_lower_tri
 * in one launch, as dlrm_emb_interact is for float32 sum bags.
 *   bags     [host] the lookups (K = bags->num_tables, D = bags->dim)
 *   dense    (B, D) float32
 *   out      (B, D + F(F-1)/2) float32, F = K + 1
 *   emb_out  NULL, or (B, K, D) float32 receiving the pooled vectors; long
 *            bags then take two launches, as for dlrm_emb_interact
 */
DLRM_API int dlrm_emb_interact_pool(const dlrm_bags *bags, const float *dense, float *out,
                                    float *emb_out, void *stream);

/*
 * dlrm_emb_interact_dots -- the fused gather + interaction writing only the
 * dots, the (B, P) layout of the pages' stacked pairwise-dot kernel
 * ([FASTPATHS] dlrm_interact.rs, PairwiseDotLowerTriStackedKernel output;
 * the top MLP then reads the dense vector and the dots through a split A,
 * see linear_bias_act_split):
 *   dots[b, p] = dot(X_b[i], X_b[j]),  (i, j) = pair p,  X_b as above
 *   bags     [host] the lookups (any dlrm_bags form)
 *   dense    (B, D) float32, feature 0 (read, not copied)
 *   dots     (B, P) float32 with row stride ld_dots >= P = F(F-1)/2
 *   emb_out  NULL, or (B, K, D) float32 receiving the pooled vectors; long
 *            bags then take two launches, as for dlrm_emb_interact
 */
DLRM_API int dlrm_emb_interact_dots(const dlrm_bags *bags, const float *dense, float *dots,
                                    int64_t ld_dots, float *emb_out, void *stream);

/*
 * linear_bias_act -- fused linear layer ([FASTPATHS] matmul2d.rs, Activation
 * epilogue; linear_bias / linear_bias_relu / linear_bias_sigmoid):
 *
 *   c[m, n] = act(bias[n] + sum_k a[m, k] * w[n, k])
 *
 *   m >= 0 (0: nothing to do), n >= 1, k >= 1
 *   a        (m, k) float32 with row stride lda >= k
 *   w        (n, k) float32, dense (the nn.Linear weight layout)
 *   bias     (n,) float32, or NULL for no bias
 *   act      a dlrm_act
 *   c        (m, n) float32 with row stride ldc >= n
 */
DLRM_API int linear_bias_act(int32_t m, int32_t n, int32_t k, const float *a,
                    int64_t lda, const float *w, const float *bias, int32_t act,
                    float *c, int64_t ldc, void *stream);

/*
 * linear_bias_act_split -- linear_bias_act whose input is the concatenation
 * [a_lo | a_hi] of two matrices, read in place ([FASTPATHS] matmul2d.rs,
 * a_split and the linear_bias / linear_bias_relu / linear_bias_sigmoid
 * *_split_a frontends: the first top-MLP layer reads cat(dense, dots)):
 *
 *   c[m, n] = act(bias[n] + sum_{k < k_lo} a_lo[m, k] w[n, k]
 *                         + sum_{k < k_hi} a_hi[m, k] w[n, k_lo + k])
 *
 *   m >= 0 (0: nothing to do), n >= 1, k_lo >= 1, k_hi >= 1
 *   a_lo     (m, k_lo) float32 with row stride lda_lo >= k_lo
 *   a_hi     (m, k_hi) float32 with row stride lda_hi >= k_hi
 *   w        (n, k_lo + k_hi) float32, dense
 *   bias     (n,) float32, or NULL
 *   c        (m, n) float32 with row stride ldc >= n
 * For n > 8 the k order of every sum is the one linear_bias_act uses on the
 * concatenated matrix, so both give the same bits; for n <= 8 the order may
 * differ (within float rounding).
 */
DLRM_API int linear_bias_act_split(int32_t m, int32_t n, int32_t k_lo, const float *a_lo,
                                   int64_t lda_lo, int32_t k_hi, const float *a_hi,
                                   int64_t lda_hi, const float *w, const float *bias, int32_t act,
                                   float *c, int64_t ldc, void *stream);

/*
 * linear_bias_act_head -- a linear layer followed by a one-output head in one
 * launch, the end of the DLRMv1 top MLP ([FASTPATHS] matmul2d.rs, Activation
 * epilogue and linear_bias_sigmoid; commit message: the top MLP ends in a
 * sigmoid):
 *
 *   h[m, n] = act(bias[n] + sum_k a[m, k] * w[n, k])          (never stored)
 *   out[m]  = head_act(head_bias + sum_n h[m, n] * head_w[n])
 *
 *   m >= 0 (0: nothing to do), 1 <= n <= 256, k >= 1
 *   a          (m, k) float32 with row stride lda >= k
 *   w          (n, k) float32, dense;  bias (n,) or NULL;  act a dlrm_act
 *   head_w     (n,) float32 (the (1, n) weight of the head);  head_bias (1,)
 *              or NULL;  head_act a dlrm_act
 *   out        (m,) float32 with stride ldo >= 1 (out[m * ldo])
 * n > 256 is DLRM_ERR_UNSUPPORTED.  A workgroup owns 32 whole rows, so the
 * head's sum over n runs in a fixed order (deterministic); it differs from
 * the order of linear_bias_act on the stored h within float rounding.
 */
DLRM_API int linear_bias_act_head(int32_t m, int32_t n, int32_t k, const float *a, int64_t lda,
                                  const float *w, const float *bias, int32_t act,
                                  const float *head_w, const float *head_bias, int32_t head_act,
                                  float *out, int64_t ldo, void *stream);

/* One MLP layer (of a dlrm_model or an mlp_forward stack). */
typedef struct dlrm_layer {
  int32_t in_features;
  int32_t out_features;
  const float *weight; /* (out_features, in_features) float32, device */
  const float *bias;   /* (out_features,) float32, device, or NULL    */
  int32_t act;         /* a dlrm_act                                  */
} dlrm_layer;

/*
 * mlp_forward -- a stack of linear_bias_act layers in one launch, the hidden
 * activations kept on chip ([FASTPATHS] matmul2d.rs, Activation epilogue;
 * the DLRMv1 bottom and top MLPs):
 *
 *   h_0 = a;  h_{l+1} = act_l(h_l W_l^T + b_l);  c = h_{num_layers}
 *
 *   m           rows, >= 0 (0: nothing to do)
 *   num_layers  1..4
 *   layers      [host] num_layers layers; layer l+1's in_features equals
 *               layer l's out_features
 *   a           (m, layers[0].in_features) float32, row stride lda
 *   c           (m, layers[last].out_features) float32, row stride ldc
 * Kernels: a three-layer stack with 4 <= in_features <= 15, a first layer
 * as wide as a multiple of 64 (>= 128), a second of at most 256 and a third
 * of at most 64 outputs (multiples of 16), second and third weights 16-byte
 * aligned (the DLRMv1 bottom MLP 13-512-256-64) runs in the fused bottom
 * kernel: 32 rows per workgroup, the hidden layers in registers and LDS.
 * Any other stack runs in the chain kernel, whose supported widths are:
 * every layer but a last one of out_features <= 8 must have out_features in
 * {64, 128, 256, 512}, and 16-byte aligned biases; at least one layer must
 * precede an out_features <= 8 layer.  Anything else returns
 * DLRM_ERR_UNSUPPORTED (linear_bias_act per layer always works).
 */
DLRM_API int mlp_forward(int32_t m, int32_t num_layers, const dlrm_layer *layers,
                         const float *a, int64_t lda, float *c, int64_t ldc, void *stream);

/* How dlrm_forward composes its launches (bits of dlrm_model.options; 0
 * lets the library choose).  Every composition computes the same function
 * within float rounding; these exist to compare them. */
#define DLRM_FORWARD_LAYERED 1u  /* never the one-launch small-model kernel   */
#define DLRM_FORWARD_UNFUSED_HEAD 2u /* the last top layer as its own launch  */
#define DLRM_FORWARD_UNFUSED_BOTTOM 4u /* each bottom layer as its own launch */
#define DLRM_FORWARD_UNSPLIT_K 8u /* no partial sums across workgroups      */

/* A DLRMv1 model: bottom MLP, K embedding tables, top MLP.  All arrays of
 * this struct are [host]; the weights and tables they point to are device
 * memory owned by the caller. */
typedef struct dlrm_model {
  int32_t num_bottom;        /* >= 1                                       */
  const dlrm_layer *bottom;  /* [host] bottom[last].out_features == dim    */
  int32_t num_top;           /* >= 1                                       */
  const dlrm_layer *top;     /* [host] top[0].in_features == dim + P       */
  int32_t num_tables;        /* K                                          */
  int32_t dim;               /* D                                          */
  const float *const *tables;/* [host] K device pointers, (rows[k], D)     */
  const int64_t *rows;       /* [host] K row counts                        */
  uint32_t options;          /* DLRM_FORWARD_* bits, 0 = automatic; other
                                bits are DLRM_ERR_SHAPE                    */
} dlrm_model;

/* Bytes of device workspace dlrm_forward needs for `batch` samples. */
DLRM_API size_t dlrm_forward_workspace_bytes(const dlrm_model *model, int32_t batch);

/*
 * dlrm_forward -- the DLRMv1 forward ([FASTPATHS] commit message and
 * translator notes: bottom MLP on the dense features, one EmbeddingBag(sum)
 * per table, pairwise-dot interaction with the bottom-MLP output as feature
 * 0, top MLP on cat(dense, dots) ending in a sigmoid):
 *
 *   d   = bottom(dense_in)                      (B, D)
 *   R   = dlrm_emb_interact(tables, indices, d) (B, D + P)
 *   out = top(R)                                (B, top[last].out_features)
 *
 *   dense_in   (B, bottom[0].in_features) float32
 *   indices, offsets, n_idx as in emb_bag_sum_multi
 *   out        (B, top[last].out_features) float32
 *   workspace  device memory of at least dlrm_forward_workspace_bytes bytes,
 *              256-byte aligned; its contents are scratch
 * Composition: a model whose MLPs hold at most 64 Ki weights in all (widths
 * <= 1024, <= 4 layers each) runs as ONE launch with every intermediate on
 * chip; larger models run each layer as its own tiled GEMM launch around the
 * fused gather + interaction, except:
 *   - when the batch is about one 32-row band per compute unit
 *     (7,137..8,192 samples), a three-layer bottom MLP of the fused kernel's
 *     shapes (see mlp_forward) runs as one launch and a one-output last top
 *     layer after a layer at most 256 wide runs in that layer's launch
 *     (linear_bias_act_head): 4 launches for 3 + 3 layers;
 *   - at small batches (the full-size model: up to 1,536 samples), a
 *     three-layer bottom MLP (first layer <= 15 inputs, hidden widths
 *     multiples of 64, N0 <= 512, output <= 256 a multiple of 16) runs as
 *     one launch cut by its hidden layer's columns (16-column slices up to
 *     512 samples, 64-column ones above), whose partial sums of the output
 *     the interaction adds as it loads the dense feature;
 *   - a layer whose tiles would leave compute units idle splits its k over
 *     up to 8 workgroups storing partial sums, which the next layer adds in
 *     a fixed order as it loads them (when it can: K a multiple of 4 and at
 *     least 128, or a matrix-vector last layer).
 * Every composition gives the same function within float rounding, and the
 * same bits on every call.  model->options may force the layered
 * composition (DLRM_FORWARD_LAYERED), the head or the bottom MLP as their
 * own launches (DLRM_FORWARD_UNFUSED_HEAD, DLRM_FORWARD_UNFUSED_BOTTOM) or
 * no partial sums across workgroups (DLRM_FORWARD_UNSPLIT_K: each layer a
 * launch of its own that finishes its outputs; with
 * DLRM_FORWARD_UNFUSED_HEAD its bits equal linear_bias_act layer by layer).
 */
DLRM_API int dlrm_forward(const dlrm_model *model, int32_t batch, const float *dense_in,
                 const int32_t *const *indices, const int32_t *const *offsets,
                 const int64_t *n_idx, float *out, void *workspace,
                 size_t workspace_bytes, void *stream);

/*
 * dlrm_forward_noalloc -- dlrm_forward without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * validation and results as dlrm_forward, with the workspace taken from a
 * fixed device array of the library of DLRM_NOALLOC_SCRATCH_BYTES bytes
 * (every GPU the library runs on holds its own copy until the process ends).
 * The call allocates nothing: no hipMalloc, hipFree or allocating library
 * routine.  Its first call on a device looks up that device's array address
 * once (hipGetSymbolAddress, with the device current).
 *   Limit: when the forward's workspace (dlrm_forward_workspace_bytes)
 *          exceeds DLRM_NOALLOC_SCRATCH_BYTES, the call runs the composition
 *          without partial sums across workgroups (DLRM_FORWARD_UNSPLIT_K
 *          added to model->options; same function within float rounding);
 *          when that too exceeds it, DLRM_ERR_WORKSPACE before any work is
 *          enqueued (the full-size model 13-512-256-64 / 26 tables /
 *          415-512-256-1 fits up to 11,650 samples).
 *   Sharing: all calls on one GPU share its array, which keeps the last
 *          call's contents; calls that overlap on one GPU (other streams or
 *          threads without ordering between them) race and give undefined
 *          results.  Calls ordered on one stream are safe.
 */
#define DLRM_NOALLOC_SCRATCH_BYTES (64u << 20)
DLRM_API int dlrm_forward_noalloc(const dlrm_model *model, int32_t batch, const float *dense_in,
                                  const int32_t *const *indices, const int32_t *const *offsets,
                                  const int64_t *n_idx, float *out, void *stream);

/*
 * Plans -- the forward recorded once into a HIP graph and replayed
 * ([FASTPATHS] runtime.rs and the commit message: the runtime captures the
 * whole graph and replays it on every execute, and the per-iteration host
 * overhead of re-registering input pointers dominated small cells until
 * pointers were cached).  A plan binds one model, one batch size and one
 * set of caller buffers; the caller writes each new batch into those same
 * buffers and calls dlrm_plan_run.
 *
 * dlrm_plan_create -- validates exactly as dlrm_forward does (same argument
 *   meanings; batch >= 1) and records the forward's launches once:
 *     DLRM_PLAN_DIRECT  the launches with their packed kernel arguments;
 *                       a run issues them with no validation or packing
 *     DLRM_PLAN_GRAPH   a HIP graph (recorded on a private stream and
 *                       instantiated); a run is one graph launch
 *   The model's host arrays are copied into the plan; every device pointer
 *   (weights, tables, dense_in, indices, offsets, out, workspace) must stay
 *   valid while the plan lives.  Allocates host memory (and HIP graph
 *   objects in graph mode), no device buffers.  An unknown mode is
 *   DLRM_ERR_SHAPE.  On success *plan receives the plan; on error it is set
 *   to NULL.
 *
 * dlrm_plan_update -- rebinds the per-batch buffers (dense_in, indices,
 *   offsets, n_idx, out) of a plan, same model, batch and workspace: the
 *   forward is recorded again (in graph mode the executable graph is updated
 *   in place, or re-instantiated if the launch shapes changed).  Must not
 *   race a run of the same plan.
 *
 * dlrm_plan_run -- enqueues one forward on `stream` (the recorded launches,
 *   or one graph launch); no other host work and no synchronization.  Runs of one plan
 *   share its workspace and output, so runs on different streams must be
 *   ordered by the caller.
 *
 * dlrm_plan_destroy -- releases the plan (NULL is a no-op).  Pending runs on
 *   a stream complete normally; the caller must not destroy a plan that a
 *   graph still being recorded refers to.
 */
typedef struct dlrm_plan dlrm_plan;

typedef enum dlrm_plan_mode {
  DLRM_PLAN_DIRECT = 0, /* replay the recorded launches          */
  DLRM_PLAN_GRAPH = 1   /* replay a HIP graph of the launches    */
} dlrm_plan_mode;

DLRM_API int dlrm_plan_create(const dlrm_model *model, int32_t batch, const float *dense_in,
                              const int32_t *const *indices, const int32_t *const *offsets,
                              const int64_t *n_idx, float *out, void *workspace,
                              size_t workspace_bytes, int32_t mode, dlrm_plan **plan);
DLRM_API int dlrm_plan_update(dlrm_plan *plan, const float *dense_in,
                              const int32_t *const *indices, const int32_t *const *offsets,
                              const int64_t *n_idx, float *out);
DLRM_API int dlrm_plan_run(dlrm_plan *plan, void *stream);
DLRM_API int dlrm_plan_destroy(dlrm_plan *plan);

#ifdef __cplusplus
}
#endif

#endif /* DLRM_EMBEDDING_BAG_H */
