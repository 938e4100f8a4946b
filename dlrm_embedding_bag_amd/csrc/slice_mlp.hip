// slice_mlp.hip -- the three-layer bottom MLP as one launch for small
// batches on gfx950 ([FASTPATHS] matmul2d.rs, Activation epilogue; the
// commit message and translator notes: the bottom MLP turns the dense
// features into the interaction's feature 0), where [FASTPATHS] = page
// "luminal_python: vanilla-PyTorch DLRMv1 fast paths + batched FFI + input
// cache".
//
//   h0 = act0(x W0^T + b0)     x (M, K0), K0 <= 15        h0 (M, N0)
//   h1 = act1(h0 W1^T + b1)                                h1 (M, N1)
//   y  = act2(h1 W2^T + b2)                                y  (M, N2)
//
// The grid is cut by h1's columns, so that a batch of a few hundred rows
// still gives the chip a few hundred workgroups.  Workgroup (16-row band,
// slice s) computes
//   h1_s = act1(h0 W1[slice]^T + b1[slice])     (16 x 64, never stored)
//   P_s  = h1_s W2[:, slice]^T                   (16 x N2)
// and stores P_s, the part of y's pre-activation that its 64 columns of h1
// contribute.  Summed in slice order, the N1 / 64 partials are y's
// pre-activation; the reader (the interaction, as it loads the dense
// feature) adds them, then b2, and applies act2.  h0 is never read from
// memory either: each 64-column slab of it is produced where the slab is
// stored to LDS, by four f32 MFMAs per wave over x and the slab's rows of W0
// (the bias in a spare k slot), then act0; every slice recomputes it (16 x
// N0 x 16 multiply-adds, a quarter of layer 1's).
//
// Everything a workgroup reads is requested at its start: the whole
// 64-row slice of W1 into LDS, this lane's W0 fragments of every slab and
// its W2 fragments into registers; then layer 1 runs slab by slab from LDS
// (two wave groups splitting each slab's k, adding their partial tiles in
// group order), and layer 2 reads h1_s from LDS.  W is the first MFMA
// operand throughout, so a lane's 4 accumulators are 4 consecutive output
// columns of one row.
#include <math.h>

#include <type_traits>

#include "../../include/dlrm_embedding_bag.h"
#include "common.hpp"
#include "kernels.hpp"

namespace dlrm {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float float4_a4 __attribute__((ext_vector_type(4), aligned(4)));

constexpr int kBM = 16;         // rows per workgroup
constexpr int kSW = 64;         // h1 columns per workgroup (the slice)
constexpr int kKS = 2;          // wave groups splitting each slab's k
constexpr int kBK = 32;         // k per wave group per slab
constexpr int kSK = kBK * kKS;  // k (h0 columns) per slab
constexpr int kSTR = kSK + 4;   // LDS row stride of an h0 slab (floats)
constexpr int kThreads = 64 * 4 * kKS;
constexpr int kAE = kBM * kSTR;  // floats per h0 slab buffer
constexpr int kHS = kSW + 4;    // LDS row stride of the h1_s tile
constexpr int kMaxN2 = 256;     // widest y (16 column blocks over 8 waves)
constexpr int kMaxN0 = 512;     // widest h0 (the whole W1 slice sits in LDS)
constexpr int kMaxSlabs = kMaxN0 / kSK;
constexpr int kPark = 4 * 4 * 64;   // floats of group 1's parked partial tiles
static_assert(kPark + kBM * kHS <= 2 * kAE, "parked tiles and h1_s fit the h0 slabs");

__device__ __forceinline__ float act_of(float x, int act) {
  if (act == 1) return x > 0.0f ? x : 0.0f;
  if (act == 2) return 1.0f / (1.0f + expf(-x));
  return x;
}

__device__ __forceinline__ floatx4 mfma4(float4 w, float4 a, floatx4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(w.x, a.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(w.y, a.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(w.z, a.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(w.w, a.w, c, 0, 0, 0);
  return c;
}

// k .. k+3 of a row of len floats (len >= 1) read at clamped addresses;
// quad_fix zeroes the ones past the row end.  The two are kept apart so that
// every load of a workgroup's start is in flight before any select (a select
// right behind each load made the compiler reuse one register and wait for
// every load in turn).
struct RawQuad {
  float v[4];
};
__device__ __forceinline__ RawQuad raw_quad(const float *__restrict__ row, int k, int len) {
  RawQuad r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r.v[e] = row[min(k + e, len - 1)];
  return r;
}
// The quad with elements past len zeroed and element `slot` (if among
// k .. k+3) set to x.
__device__ __forceinline__ float4 quad_fix(const RawQuad &r, int k, int len, int slot, float x) {
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (k + e == slot) ? x : (k + e < len) ? r.v[e] : 0.0f;
  return make_float4(v[0], v[1], v[2], v[3]);
}

// Four floats at a 4-byte-aligned address as one 16-byte load.
__device__ __forceinline__ float4 load4(const float *p) {
  const float4_a4 t = *reinterpret_cast<const float4_a4 *>(p);
  return make_float4(t.x, t.y, t.z, t.w);
}

// NS = N0 / 64 slabs, a compile-time count: every unrolled loop runs its full
// trip count (no early exits from loops that carry MFMA accumulators).
template <int NS>
__global__ __launch_bounds__(kThreads) void slice_mlp_kernel(SliceParams p, int nslice,
                                                             int xcd_chunk) {
  extern __shared__ float4 lds_raw[];
  float *lds = reinterpret_cast<float *>(lds_raw);

  const int M = p.M, N0 = p.N0, N1 = p.N1, N2 = p.N2, K0 = p.K0;
  int bid = blockIdx.x;
  if (xcd_chunk > 0) bid = (bid & 7) * xcd_chunk + (bid >> 3);
  const int band = bid / nslice;
  const int s = bid - band * nslice;
  const int m0 = band * kBM, n0 = s * kSW;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kg = wave >> 2;  // k group of layer 1
  const int wn = wave & 3;   // 16-column block of the slice
  const int l16 = lane & 15, lq = lane >> 4;

  static_assert(NS >= 1 && NS <= kMaxSlabs, "slab count (N0 / kSK)");
  const int SW1 = N0 + 4;         // LDS row stride of the W1 slice
  float *W1s = lds;               // 64 x SW1
  float *Abuf = lds + kSW * SW1;  // two h0 slabs of 16 x kSTR (then the h1_s tile)

  // Waves 0..3 produce columns [16 w, +16) of each h0 slab from x (one x
  // fragment for every slab; k slot K0 carries 1, the matching W0 slot the
  // bias).  Rows past M compute on row M - 1 and are never stored.  The
  // loads are issued in the order their data is needed: x and W0, the W1
  // slice, W2.
  RawQuad xr{}, w0q[NS];
  float blv[NS];
  if (wave < 4) {
    xr = raw_quad(p.x + (int64_t)min(m0 + l16, M - 1) * p.ldx, 4 * lq, K0);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int n = j * kSK + 16 * wn + l16;  // h0 column of the W0 row
      w0q[j] = raw_quad(p.W0 + (int64_t)n * K0, 4 * lq, K0);
      blv[j] = *(p.b0 ? p.b0 + n : p.W0);
    }
  }

  // W1 slice: thread t loads row t / 8 of it, quads t % 8 + 8 i (2 NS
  // loads per thread, all issued before any is stored).
  const int wr = tid >> 3, wc0 = tid & 7;
  const float *wrow = p.W1 + (int64_t)(n0 + wr) * N0;
  float4 wq[2 * NS];
#pragma unroll
  for (int i = 0; i < 2 * NS; ++i) wq[i] = load4(wrow + 4 * (wc0 + 8 * i));

  // Layer 2's W2 fragments: wave w multiplies 16-column blocks w, w + 8 of
  // P (N2 / 16 blocks), k over the slice in 16-wide steps.
  constexpr int KQ = kSW / 16;
  const int nblk = N2 / 16;
  float4 wb[2][KQ];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int cb = min(wave + 8 * j, nblk - 1);
    const float *row = p.W2 + (int64_t)(16 * cb + l16) * N1 + n0;
#pragma unroll
    for (int q = 0; q < KQ; ++q) wb[j][q] = load4(row + 16 * q + 4 * lq);
  }
  __builtin_amdgcn_sched_barrier(0);  // every load above is issued before any use

  float4 xf = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 w0r[NS];
  if (wave < 4) {
    xf = quad_fix(xr, 4 * lq, K0, K0, 1.0f);
#pragma unroll
    for (int j = 0; j < NS; ++j) w0r[j] = quad_fix(w0q[j], 4 * lq, K0, K0, p.b0 ? blv[j] : 0.0f);
  }

  // the W1 slice to LDS
#pragma unroll
  for (int i = 0; i < 2 * NS; ++i)
    *reinterpret_cast<float4 *>(&W1s[wr * SW1 + 4 * (wc0 + 8 * i)]) = wq[i];

  // h0 slab j goes to buffer j & 1.
  auto put_slab = [&](int j) __attribute__((always_inline)) {
    if (wave >= 4) return;
    float *As = Abuf + (j & 1) * kAE;
    const floatx4 h = mfma4(w0r[j], xf, floatx4{0.f, 0.f, 0.f, 0.f});
    float4 o;
    o.x = act_of(h[0], p.act0);
    o.y = act_of(h[1], p.act0);
    o.z = act_of(h[2], p.act0);
    o.w = act_of(h[3], p.act0);
    *reinterpret_cast<float4 *>(&As[l16 * kSTR + 16 * wn + 4 * lq]) = o;
  };

  // Layer 1: two accumulator chains per wave (the two 16-wide k quads of its
  // half of each slab), added at the end.  Each interval between barriers
  // multiplies slab j and produces slab j + 1 (into the buffer slab j - 1
  // was read from, released by the barrier).
  floatx4 acc[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
  const int kgo = kg * kBK;
  put_slab(0);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const float *As = Abuf + (j & 1) * kAE;
    const float *Wj = W1s + j * kSK;
    float4 af[2], wf[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = kgo + 16 * h + 4 * lq;
      af[h] = *reinterpret_cast<const float4 *>(&As[l16 * kSTR + k]);
      wf[h] = *reinterpret_cast<const float4 *>(&Wj[(16 * wn + l16) * SW1 + k]);
    }
    if (j + 1 < NS) put_slab(j + 1);
    acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[0].x, af[0].x, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[1].x, af[1].x, acc[1], 0, 0, 0);
    acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[0].y, af[0].y, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[1].y, af[1].y, acc[1], 0, 0, 0);
    acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[0].z, af[0].z, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[1].z, af[1].z, acc[1], 0, 0, 0);
    acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[0].w, af[0].w, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[1].w, af[1].w, acc[1], 0, 0, 0);
    __syncthreads();
  }
  const floatx4 accs = acc[0] + acc[1];

  // Group 1 parks its partial tile; group 0 adds it (fixed order), applies
  // b1 and act1 and writes h1_s to LDS.
  float *H = Abuf + kPark;  // 16 x kHS
  if (kg == 1) {
    float *red = Abuf + (size_t)wn * 4 * 64 + lane;
#pragma unroll
    for (int v = 0; v < 4; ++v) red[v * 64] = accs[v];
  }
  __syncthreads();
  if (kg == 0) {
    const float *red = Abuf + (size_t)wn * 4 * 64 + lane;
    const int n = n0 + 16 * wn + 4 * lq;  // h1 column of the lane's first value
    float o[4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
      o[v] = act_of(accs[v] + red[v * 64] + (p.b1 ? p.b1[n + v] : 0.0f), p.act1);
    *reinterpret_cast<float4 *>(&H[l16 * kHS + 16 * wn + 4 * lq]) =
        make_float4(o[0], o[1], o[2], o[3]);
  }
  __syncthreads();

  // Layer 2 on the slice: P_s[m][c] = sum_k h1_s[m][k] W2[c][n0 + k], the
  // wave's two column blocks as two chains.
  float *P = p.P + (int64_t)s * p.pstride;
  floatx4 y[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int q = 0; q < KQ; ++q) {
    const float4 hf = *reinterpret_cast<const float4 *>(&H[l16 * kHS + 16 * q + 4 * lq]);
    y[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(wb[0][q].x, hf.x, y[0], 0, 0, 0);
    y[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(wb[1][q].x, hf.x, y[1], 0, 0, 0);
    y[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(wb[0][q].y, hf.y, y[0], 0, 0, 0);
    y[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(wb[1][q].y, hf.y, y[1], 0, 0, 0);
    y[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(wb[0][q].z, hf.z, y[0], 0, 0, 0);
    y[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(wb[1][q].z, hf.z, y[1], 0, 0, 0);
    y[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(wb[0][q].w, hf.w, y[0], 0, 0, 0);
    y[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(wb[1][q].w, hf.w, y[1], 0, 0, 0);
  }
  const int m = m0 + l16;
  if (m >= M) return;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int cb = wave + 8 * j;
    if (cb >= nblk) continue;
    *reinterpret_cast<float4 *>(P + (int64_t)m * p.ldp + 16 * cb + 4 * lq) =
        make_float4(y[j][0], y[j][1], y[j][2], y[j][3]);
  }
}

// LDS bytes of a launch: the W1 slice and two h0 slabs.
size_t slice_lds_bytes(int N0) { return sizeof(float) * ((size_t)kSW * (N0 + 4) + 2 * kAE); }

// ---------------------------------------------------------------------------
// Narrow slices: 16 columns of h1 per workgroup of 4 waves, for the smallest
// batches, where 64-column slices leave most CUs idle and each workgroup's
// 64 x N0 slice of W1 takes many memory round trips to arrive.  A workgroup
// (16-row band, slice s) reads a quarter of the W1 bytes of a 64-column one:
//   1. every load is issued at the start: the lane's x fragment, its W0
//      fragments (wave w produces h0 column blocks w, w + 4, ...), its W1
//      fragments (wave w multiplies k in [w N0/4, (w + 1) N0/4)) and its W2
//      fragments;
//   2. h0 (16 x N0) is produced into LDS by four f32 MFMAs per 16 x 16 block
//      (bias in the spare k slot K0), then act0;
//   3. layer 1: each wave one 16 x 16 partial tile over its k quarter;
//      waves 1..3 park theirs in LDS and wave 0 adds them in wave order,
//      then b1 and act1: h1_s (16 x 16) in LDS;
//   4. layer 2: P_s = h1_s W2[:, slice]^T, wave w the column blocks w,
//      w + 4, ... of P_s (k = 16: four MFMAs).
// ---------------------------------------------------------------------------
constexpr int kNSW = 16;                // h1 columns per workgroup
constexpr int kNThreads = 256;          // 4 waves
constexpr int kNMaxQ = kMaxN0 / 4 / 16;  // W1 k-quad blocks per wave (N0 / 64)
constexpr int kNMaxB2 = kMaxN2 / 16 / 4;  // P column blocks per wave

// NQ = N0 / 64 (h0 column blocks and layer-1 k blocks per wave), a
// compile-time count as in slice_mlp_kernel.
template <int NQ>
__global__ __launch_bounds__(kNThreads) void narrow_slice_kernel(SliceParams p, int nslice,
                                                                int xcd_chunk) {
  extern __shared__ float4 lds_raw[];
  float *lds = reinterpret_cast<float *>(lds_raw);

  const int M = p.M, N0 = p.N0, N1 = p.N1, N2 = p.N2, K0 = p.K0;
  int bid = blockIdx.x;
  if (xcd_chunk > 0) bid = (bid & 7) * xcd_chunk + (bid >> 3);
  const int band = bid / nslice;
  const int s = bid - band * nslice;
  const int m0 = band * kBM, n0 = s * kNSW;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;

  const int SH = N0 + 4;             // LDS row stride of h0
  float *H0 = lds;                   // 16 x SH
  float *red = lds + kBM * SH;       // 3 parked 16 x 16 tiles
  float *H1 = red + 3 * 4 * 64;      // 16 x (kNSW + 4)
  constexpr int SH1 = kNSW + 4;

  static_assert(NQ >= 1 && NQ <= kNMaxQ, "block count");
  const int nblk2 = N2 / 16;

  // 1. loads.  Rows past M compute on row M - 1 and are never stored.
  const RawQuad xr = raw_quad(p.x + (int64_t)min(m0 + l16, M - 1) * p.ldx, 4 * lq, K0);
  RawQuad w0q[NQ];
  float blv[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int n = 16 * (w + 4 * j) + l16;  // h0 column of the W0 row
    w0q[j] = raw_quad(p.W0 + (int64_t)n * K0, 4 * lq, K0);
    blv[j] = *(p.b0 ? p.b0 + n : p.W0);
  }
  const int kw = w * (N0 / 4);  // this wave's k quarter of layer 1
  const float *w1row = p.W1 + (int64_t)(n0 + l16) * N0 + kw + 4 * lq;
  float4 w1f[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) w1f[q] = load4(w1row + 16 * q);
  float4 w2f[kNMaxB2];
#pragma unroll
  for (int j = 0; j < kNMaxB2; ++j) {
    const int cb = min(w + 4 * j, nblk2 - 1);
    w2f[j] = load4(p.W2 + (int64_t)(16 * cb + l16) * N1 + n0 + 4 * lq);
  }
  __builtin_amdgcn_sched_barrier(0);  // every load above is issued before any use
  const float4 xf = quad_fix(xr, 4 * lq, K0, K0, 1.0f);
  float4 w0r[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) w0r[j] = quad_fix(w0q[j], 4 * lq, K0, K0, p.b0 ? blv[j] : 0.0f);

  // 2. h0 into LDS
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const floatx4 h = mfma4(w0r[j], xf, floatx4{0.f, 0.f, 0.f, 0.f});
    float4 o;
    o.x = act_of(h[0], p.act0);
    o.y = act_of(h[1], p.act0);
    o.z = act_of(h[2], p.act0);
    o.w = act_of(h[3], p.act0);
    *reinterpret_cast<float4 *>(&H0[l16 * SH + 16 * (w + 4 * j) + 4 * lq]) = o;
  }
  __syncthreads();

  // 3. layer 1 over the wave's k quarter, two accumulator chains
  floatx4 acc[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const float4 af = *reinterpret_cast<const float4 *>(&H0[l16 * SH + kw + 16 * q + 4 * lq]);
    acc[q & 1] = mfma4(w1f[q], af, acc[q & 1]);
  }
  const floatx4 accs = acc[0] + acc[1];
  if (w > 0) {
    float *r = red + (size_t)(w - 1) * 4 * 64 + lane;
#pragma unroll
    for (int v = 0; v < 4; ++v) r[v * 64] = accs[v];
  }
  __syncthreads();
  if (w == 0) {
    const int n = n0 + 4 * lq;  // h1 column of the lane's first value
    float o[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float t = accs[v];
#pragma unroll
      for (int g = 0; g < 3; ++g) t += red[(size_t)g * 4 * 64 + v * 64 + lane];
      o[v] = act_of(t + (p.b1 ? p.b1[n + v] : 0.0f), p.act1);
    }
    *reinterpret_cast<float4 *>(&H1[l16 * SH1 + 4 * lq]) = make_float4(o[0], o[1], o[2], o[3]);
  }
  __syncthreads();

  // 4. layer 2 on the slice
  const float4 hf = *reinterpret_cast<const float4 *>(&H1[l16 * SH1 + 4 * lq]);
  float *P = p.P + (int64_t)s * p.pstride;
  const int m = m0 + l16;
#pragma unroll
  for (int j = 0; j < kNMaxB2; ++j) {
    const int cb = w + 4 * j;
    const floatx4 y = mfma4(w2f[j], hf, floatx4{0.f, 0.f, 0.f, 0.f});
    if (cb < nblk2 && m < M)
      *reinterpret_cast<float4 *>(P + (int64_t)m * p.ldp + 16 * cb + 4 * lq) =
          make_float4(y[0], y[1], y[2], y[3]);
  }
}

size_t narrow_lds_bytes(int N0) {
  return sizeof(float) * ((size_t)kBM * (N0 + 4) + 3 * 4 * 64 + kBM * (kNSW + 4));
}

}  // namespace

int slice_mlp_count(const SliceParams &p) { return p.sw > 0 ? p.N1 / p.sw : 0; }

int64_t slice_mlp_workgroups(const SliceParams &p) {
  return (int64_t)((p.M + kBM - 1) / kBM) * slice_mlp_count(p);
}

bool slice_mlp_supported(const SliceParams &p) {
  return (p.sw == kSW || p.sw == kNSW) && p.M >= 1 && p.K0 >= 1 && p.K0 <= 15 &&
         p.N0 >= kSK && p.N0 <= kMaxN0 && p.N0 % kSK == 0 && p.N1 >= p.sw &&
         p.N1 % p.sw == 0 && p.N2 >= 16 && p.N2 <= kMaxN2 &&
         p.N2 % 16 == 0 && p.x && p.W0 && p.W1 && p.W2 && p.P && p.ldx >= p.K0 &&
         p.ldp >= p.N2 && p.ldp % 4 == 0 && p.pstride % 4 == 0 && aligned16(p.P);
}

hipError_t launch_slice_mlp(const SliceParams &p, hipStream_t stream) {
  if (!slice_mlp_supported(p)) return hipErrorInvalidValue;
  const int nslice = slice_mlp_count(p);
  const int64_t wgs = slice_mlp_workgroups(p);
  const int xcd_chunk = (wgs % 8 == 0) ? (int)(wgs / 8) : 0;
  const dim3 grid((unsigned)wgs);
  // the kernels' loops run N0 / 64 times, fixed at compile time
  auto run = [&](auto ns) -> hipError_t {
    constexpr int NS = decltype(ns)::value;
    if (p.sw == kNSW) {
      launch_kernel(narrow_slice_kernel<NS>, grid, dim3(kNThreads), narrow_lds_bytes(p.N0), stream,
                    p, nslice, xcd_chunk);
      return hipGetLastError();
    }
    // up to 140 KiB of LDS per workgroup (the CU has 160 KiB): raise the
    // 64 KiB default once per instantiation
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(slice_mlp_kernel<NS>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)slice_lds_bytes(NS * kSK));
    if (attr != hipSuccess) return attr;
    launch_kernel(slice_mlp_kernel<NS>, grid, dim3(kThreads), slice_lds_bytes(p.N0), stream, p,
                  nslice, xcd_chunk);
    return hipGetLastError();
  };
  switch (p.N0 / kSK) {
    case 1: return run(std::integral_constant<int, 1>{});
    case 2: return run(std::integral_constant<int, 2>{});
    case 3: return run(std::integral_constant<int, 3>{});
    case 4: return run(std::integral_constant<int, 4>{});
    case 5: return run(std::integral_constant<int, 5>{});
    case 6: return run(std::integral_constant<int, 6>{});
    case 7: return run(std::integral_constant<int, 7>{});
    default: return run(std::integral_constant<int, 8>{});
  }
}

}  // namespace dlrm
