// kernels.hpp -- host-side launchers of the HIP kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace dlrm {

// Geometry and buffers of one interaction launch.
struct InteractParams {
  int B, K, D, P;   // batch, pooled vectors per sample, dim, pairs F(F-1)/2
  int S;            // samples per workgroup
  int DP;           // LDS row stride in floats
  int FR;           // LDS tile rows per sample (F, or F rounded up to 4)
  int G;            // lanes per gathered row
  int Q;            // quads per 4 x 4 dot block (blocked interaction)
  int lds_bytes;    // dynamic LDS per workgroup
  int copy_dense;   // write dense into out[:, 0:D]
  int dot_off;      // column of the first dot in an out row: D, or 0 for dots only
  int out_vec;      // out rows are 16-byte aligned (vector dense copy)
  const float *dense;
  int64_t ld_dense;
  float *out;
  int64_t ld_out;
  float *emb_out;        // optional (B, K, D) copy of the pooled vectors
  const float *emb_in;   // (B, K, D) input of the interaction-only kernel
  // dense_nred >= 1: dense holds dense_nred partial sums of the bottom MLP's
  // last layer (its pre-activation when there is one), dense_stride floats
  // apart, and feature 0 is dense_act(dense_bias + (P_0 + P_1 + ...))
  // (dense_bias may be null); 0: dense is feature 0.
  int dense_nred;
  int64_t dense_stride;
  const float *dense_bias;
  int dense_act;
};

// How a gather reads its bags: table storage type, vector (16-byte chunk) or
// scalar path, CSR offsets, per-sample weights.
struct GatherConfig {
  int dtype = kF32;
  bool vec = false;
  bool csr = false;
  bool psw = false;
};

hipError_t launch_emb_bag(const TableSet &ts, const GatherConfig &gc, int B, int K, int D,
                          float *out, hipStream_t stream);

// Fills the geometry fields of `ip` for a gather whose row chunks hold `el`
// elements (1 when there is no gather); false if one sample's tile exceeds LDS.
bool plan_interact(int B, int K, int D, bool vec4, int el, InteractParams &ip, int &threads);

// ts == nullptr: interaction over ip.emb_in (gc.vec selects the vector path);
// otherwise fused gather + interaction.
hipError_t launch_interact(const TableSet *ts, const GatherConfig &gc, const InteractParams &ip,
                           int threads, hipStream_t stream);

// The whole forward in one launch (forward_small.hip) for small MLPs.
constexpr int kMaxSmallLayers = 4;           // per MLP
constexpr int kSmallMaxWidth = 1024;         // widest layer input or output
constexpr int kSmallWeightFloats = 64 * 1024;  // all MLP weights together (256 KiB)

struct SmallLayer {
  const float *W;     // (N, K) dense
  const float *bias;  // (N,) or nullptr
  int K, N, act;
};

struct SmallForwardParams {
  InteractParams ip;  // gather + interaction geometry (ip.out etc. unused)
  int nb, nt;         // bottom and top layer counts
  SmallLayer layer[2 * kMaxSmallLayers];  // bottom in [0, nb), top from kMaxSmallLayers
  const float *dense_in;  // (B, in0)
  int in0;
  float *out;  // (B, n_out)
  int n_out;
  int ld_buf, ldR;            // LDS row strides (floats)
  int r_off, a_off, b_off;    // LDS offsets (floats); the tile starts at 0
  int w_lds;                  // weights and biases are staged in LDS
  int w_off[2 * kMaxSmallLayers], bias_off[2 * kMaxSmallLayers];  // their LDS offsets
};

// Fills `p` (all but dense_in, out, n_out) for batch B; false if the model
// is too large for the one-launch forward.
bool plan_forward_small(int B, int K, int D, bool vec4, int in0, int nb, const SmallLayer *bottom,
                        int nt, const SmallLayer *top, SmallForwardParams &p, int &threads);
hipError_t launch_forward_small(const TableSet &ts, bool csr, bool vec4,
                                const SmallForwardParams &p, int threads, hipStream_t stream);

constexpr int kMaxChainLayers = 4;
constexpr int kMaxChainWidth = 512;  // widest layer the MLP chain keeps in LDS

// One layer of an MLP chain: out = act(in W^T + bias), W (N, K) dense.
struct ChainLayer {
  const float *W;
  const float *bias;  // (N,) or nullptr
  int K, N, act;
};

// A stack of layers run by one launch over rows [0, M).
struct ChainParams {
  int M, nlayers;
  const float *A;  // (M, layer[0].K), row stride lda
  int64_t lda;
  float *C;        // (M, layer[last].N), row stride ldc
  int64_t ldc;
  int c_vec;       // filled by the launcher
  int ld_hidden;   // filled by the launcher
  ChainLayer layer[kMaxChainLayers];
};

// True when the chain kernel can run these layers: every layer but a final
// N <= 8 head has N a multiple of 64 with N/64 a power of two and N <= 512,
// biases 16-byte aligned, widths chain.
bool chain_supported(const ChainParams &p);
hipError_t launch_mlp_chain(ChainParams p, hipStream_t stream);

// C = act(A W^T + bias); A (M, K) stride lda, W (N, K) dense, C stride ldc.
hipError_t launch_linear(int M, int N, int K, const float *A, int64_t lda, const float *W,
                         const float *bias, int act, float *C, int64_t ldc, hipStream_t stream);
// The same with A = [A_lo | A_hi]: A_lo (M, K_lo) stride lda_lo, A_hi (M, K_hi)
// stride lda_hi, W (N, K_lo + K_hi).
hipError_t launch_linear_split(int M, int N, int K_lo, const float *A_lo, int64_t lda_lo,
                               int K_hi, const float *A_hi, int64_t lda_hi, const float *W,
                               const float *bias, int act, float *C, int64_t ldc,
                               hipStream_t stream);

// One layer with the k split across workgroups and the split's partial sums
// reduced by the next layer (linear.hip).  A is either a plain (M, K) matrix
// (a_nred <= 1) or a_nred partial sums of the layer before, a_stride floats
// apart, read as a_act(a_bias[k] + (P_0 + P_1 + ...)[m][k]) (a_bias may be
// null).  With nsplit >= 2 the layer stores nsplit raw partial sums (no bias,
// no activation: its reader applies them) at C + s c_stride, else
// C = act(A W^T + bias).
struct LinearCall {
  int M, N, K;
  const float *A;
  int64_t lda;
  int a_nred;
  int64_t a_stride;
  const float *a_bias;
  int a_act;
  const float *W;
  const float *bias;
  int act;
  float *C;
  int64_t ldc;
  int nsplit;
  int64_t c_stride;
};
hipError_t launch_linear_call(const LinearCall &c, hipStream_t stream);
// How many partial sums an M x N x K layer is split into so that its tiles
// fill the chip (a power of two up to 8; 1 = not split).
int linear_split_count(int M, int N, int K);
// Whether an M x N x K layer with weights W can read its A as nred partials.
bool linear_reduce_supported(int M, int N, int K, const float *W, int nred);

// The three-layer bottom MLP in one launch (bottom_mlp.hip):
// y = act2(act1(act0(x W0^T + b0) W1^T + b1) W2^T + b2), hidden layers on chip.
struct BottomParams {
  int M, K0, N0, N1, N2;
  const float *x;  // (M, K0), row stride ldx
  int64_t ldx;
  const float *W0, *b0, *W1, *b1, *W2, *b2;  // (N_l, K_l) dense; biases (N_l,) or nullptr
  int act0, act1, act2;
  float *y;        // (M, N2), row stride ldy
  int64_t ldy;
};
// True when the kernel takes these shapes: 4 <= K0 <= 15, N0 a multiple of 64
// (>= 128), N1 <= 256 and N2 <= 64 multiples of 16, W1 and W2 16-byte
// aligned.
bool bottom_mlp_supported(const BottomParams &p);
// Whether it beats three layer launches inside the forward at M rows (its
// grid is M / 32 bands, one per CU at a time).
bool bottom_mlp_preferred(int M);
hipError_t launch_bottom_mlp(const BottomParams &p, hipStream_t stream);

// The three-layer bottom MLP in one launch cut by h1's columns into slices
// of sw = 64 or 16 columns (slice_mlp.hip): workgroup (16-row band, slice s)
// stores P_s = act1(act0(x W0^T + b0) W1[slice]^T + b1[slice]) W2[:, slice]^T,
// and the N1 / sw partials summed in slice order are y's pre-activation (b2
// and act2 are the reader's).
struct SliceParams {
  int M, K0, N0, N1, N2;
  int sw;          // slice width: 64, or 16 for the smallest batches
  const float *x;  // (M, K0), row stride ldx
  int64_t ldx;
  const float *W0, *b0, *W1, *b1, *W2;  // (N_l, K_l) dense; biases (N_l,) or nullptr
  int act0, act1;
  float *P;        // partial s at P + s pstride, row stride ldp
  int64_t ldp, pstride;
};
int slice_mlp_count(const SliceParams &p);         // partials written (N1 / sw)
int64_t slice_mlp_workgroups(const SliceParams &p);
// True for sw 64 or 16, 1 <= K0 <= 15, N0 a multiple of 64 up to 512, N1 a
// multiple of sw, N2 a multiple of 16 up to 256, P 16-byte aligned with ldp,
// pstride multiples of 4.
bool slice_mlp_supported(const SliceParams &p);
hipError_t launch_slice_mlp(const SliceParams &p, hipStream_t stream);

// Two layers in one launch: h = act(A W^T + bias) (N <= 256 columns, never
// stored) followed by a one-output head, out[m] = head_act(head_bias +
// sum_n h[m][n] head_w[n]), out row stride ldo.
bool linear_head_supported(int N, int K);
// Whether the fused launch beats the two layer launches at M rows.
bool linear_head_preferred(int M);
hipError_t launch_linear_head(int M, int N, int K, const float *A, int64_t lda, const float *W,
                              const float *bias, int act, const float *head_w,
                              const float *head_bias, int head_act, float *out, int64_t ldo,
                              hipStream_t stream);

}  // namespace dlrm
