// bottom_mlp.hip -- the DLRMv1 bottom MLP (three fused linear + bias +
// activation layers, 13 -> 512 -> 256 -> 64 in the full-size model) as one
// launch for gfx950 ([FASTPATHS] matmul2d.rs, Activation epilogue; the
// commit message and translator notes: the bottom MLP turns the dense
// features into the interaction's feature 0), where [FASTPATHS] = page
// "luminal_python: vanilla-PyTorch DLRMv1 fast paths + batched FFI + input
// cache".
//
//   h0 = act0(x W0^T + b0)     x (M, K0), K0 <= 16       h0 (M, N0)
//   h1 = act1(h0 W1^T + b1)                               h1 (M, N1), N1 <= 256
//   y  = act2(h1 W2^T + b2)                               y  (M, N2), N2 <= 64
//
// A workgroup owns 32 whole rows.  Layer 1 is the contraction that carries
// the work: the f32 matrix-core tile of linear.hip (32 x 256 on 8 waves, two
// wave groups splitting each 64-wide k slab, slabs of W1 staged through two
// LDS buffers two slabs ahead).  Its A operand, h0, is never read from
// memory: each 64-column slab of h0 is produced where the slab would be
// stored to LDS, by four f32 MFMAs per wave over x (kept in registers) and
// the slab's rows of W0 (4 <= K0 <= 15: four k per lane, and a spare k
// slot that carries the bias), then the activation.  Layer 2 runs in the epilogue: group 0 writes h1 to LDS
// and each wave computes one 16 x 16 block of y from it and W2 (read
// straight from L2), storing y to the caller's matrix.  The (M, N0) and
// (M, N1) activations of the two hidden layers never reach HBM, and the
// three layers cost one launch.
//
// As in linear.hip, W is the first MFMA operand (a lane's 4 accumulators are
// 4 consecutive output columns of one row) and each lane feeds the 4
// components of a float4 of 4 consecutive k to 4 successive MFMAs.
#include <math.h>

#include "../../include/dlrm_embedding_bag.h"
#include "common.hpp"
#include "kernels.hpp"

namespace dlrm {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 32;          // rows per workgroup
constexpr int kBN = 256;         // widest layer-1 output (4 waves x 64 columns)
constexpr int kKS = 2;           // wave groups splitting each slab's k
constexpr int kBK = 32;          // k per wave group per slab
constexpr int kSK = kBK * kKS;   // k (= layer-0 output columns) per staged slab
constexpr int kSTR = kSK + 4;    // LDS row stride of a slab (floats)
constexpr int kThreads = 64 * 4 * kKS;
constexpr int kA = kBM * kSTR, kW = kBN * kSTR;  // floats per slab buffer
constexpr int kHS = kBN + 4;     // LDS row stride of the h1 tile
constexpr int kPark = 4 * 2 * 4 * 4 * 64;        // floats of group 1's parked partial tile
static_assert(kPark + kBM * kHS <= 2 * (kA + kW), "h1 tile must fit beside the parked tile");

__device__ __forceinline__ float mlp_act(float x, int act) {
  if (act == 1) return x > 0.0f ? x : 0.0f;
  if (act == 2) return 1.0f / (1.0f + expf(-x));
  return x;
}

// The same activation without a branch (both forms computed, one selected),
// for use inside the k loop, where a branch would make the compiler's
// wait-count pass drain the outstanding prefetch loads where it joins.
__device__ __forceinline__ float mlp_act_select(float x, int act) {
  const float r = (act == 1 && !(x > 0.0f)) ? 0.0f : x;
  const float sg = 1.0f / (1.0f + expf(-x));
  return act == 2 ? sg : r;
}

// k .. k+3 of a row of `len` floats; past the row end reads zero.  Four
// loads at clamped addresses (every one inside the row) and selects, with
// no branch: a load under a lane-dependent branch inside the k loop would
// make the compiler wait for every outstanding load (the W1 prefetch
// included) where the branches join.
__device__ __forceinline__ float4 row_quad(const float *__restrict__ row, int k, int len) {
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float t = row[min(k + e, len - 1)];
    v[e] = (k + e < len) ? t : 0.0f;
  }
  return make_float4(v[0], v[1], v[2], v[3]);
}

// The same for a row of len >= 4 floats with one 16-byte load at dword
// alignment, in two steps so that the load can be issued well before its
// value is needed: quad_load reads the four floats at min(k, len - 4),
// inside the row; quad_pick selects the lane's elements out of them.
typedef float float4_a4 __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ floatx4 quad_load(const float *__restrict__ row, int k, int len) {
  const float4_a4 t = *reinterpret_cast<const float4_a4 *>(row + min(k, len - 4));
  return floatx4{t.x, t.y, t.z, t.w};
}
__device__ __forceinline__ float4 quad_pick(floatx4 t, int k, int len) {
  const int o = min(k, len - 4);
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = k + e - o;  // 0..3 for the elements inside the row
    const float x = i == 0 ? t[0] : i == 1 ? t[1] : i == 2 ? t[2] : t[3];
    v[e] = (k + e < len) ? x : 0.0f;
  }
  return make_float4(v[0], v[1], v[2], v[3]);
}

// Element e (0..3) of v set to x; any other e leaves v unchanged.
__device__ __forceinline__ void set_elem(float4 &v, int e, float x) {
  v.x = e == 0 ? x : v.x;
  v.y = e == 1 ? x : v.y;
  v.z = e == 2 ? x : v.z;
  v.w = e == 3 ? x : v.w;
}

__device__ __forceinline__ floatx4 mfma4(float4 w, float4 a, floatx4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(w.x, a.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(w.y, a.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(w.z, a.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(w.w, a.w, c, 0, 0, 0);
  return c;
}

template <bool VC, bool B0>
__global__ __launch_bounds__(kThreads) void bottom_mlp_kernel(BottomParams p, int xcd_chunk) {
  __shared__ float lds[2 * (kA + kW)];

  const int M = p.M, K0 = p.K0, N0 = p.N0, N1 = p.N1, N2 = p.N2;
  int bid = blockIdx.x;
  if (xcd_chunk > 0) bid = (bid & 7) * xcd_chunk + (bid >> 3);
  const int m0 = bid * kBM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kg = wave >> 2;  // k group of layer 1
  const int wn = wave & 3;   // 64-column quarter of layer 1's output
  const int l16 = lane & 15, lq = lane >> 4;

  // Layer 0 producer: wave w makes rows [16 (w >> 2), +16) x columns
  // [16 (w & 3), +16) of every h0 slab.  Its x fragment (one float4 of k per
  // lane) is the same for every slab.
  // The bias rides in the MFMA: k slot K0 (free, K0 <= 15) holds 1 in x and
  // b0[n] in W0's fragment, so the sum over k adds it.
  const int prb = wave >> 2, pcb = wave & 3;
  float4 xf = row_quad(p.x + (int64_t)min(m0 + 16 * prb + l16, M - 1) * p.ldx, 4 * lq, K0);
  set_elem(xf, K0 - 4 * lq, 1.0f);

  // Layer 1 staging: each thread loads 8 float4 of a W1 slab, rows
  // tid / 16 + 32 i at column 4 (tid % 16) (rows past N1 are clamped to its
  // last row; their outputs are masked).
  constexpr int W_V4 = kBN * kSK / 4 / kThreads;
  static_assert(kThreads % (kSK / 4) == 0, "one column per thread");
  constexpr int kRowStep = kThreads / (kSK / 4);
  const int wr0 = tid / (kSK / 4), wc = 4 * (tid % (kSK / 4));

  floatx4 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nslab = N0 / kSK;  // N0 % 64 == 0: every slab is full
  // fetch: the slab's W1 rows, and this lane's W0 fragment and bias for the
  // h0 slab it produces.  (Every helper is forced inline: one that is not
  // would receive the register arrays by address, i.e. through scratch.)
  // W0Frag: the raw loads behind this lane's W0 fragment of a slab.
  struct W0Frag {
    floatx4 q;  // the four floats of quad_load
    float bn;   // the bias of the h0 column the lane's W0 row feeds
  };
  auto fetch = [&](int sl, floatx4 (&rw)[W_V4], W0Frag &w0) __attribute__((always_inline)) {
    const int kb = sl * kSK;
#pragma unroll
    for (int i = 0; i < W_V4; ++i)
      rw[i] = *reinterpret_cast<const floatx4 *>(
          p.W1 + (int64_t)min(wr0 + kRowStep * i, N1 - 1) * N0 + kb + wc);
    const int n = kb + 16 * pcb + l16;  // h0 column this lane's W0 row feeds
    w0.q = quad_load(p.W0 + (int64_t)n * K0, 4 * lq, K0);
    // every lane loads the bias (a load under a lane-dependent test would be
    // a divergent branch in the k loop, see row_quad)
    w0.bn = B0 ? p.b0[n] : 0.0f;
  };
  // stash: W1 rows to the LDS buffer, and the produced h0 slab beside them.
  auto stash = [&](int buf, const floatx4 (&rw)[W_V4], const W0Frag &w0) __attribute__((always_inline)) {
    float *As = lds + buf * (kA + kW);
    float *Ws = As + kA;
#pragma unroll
    for (int i = 0; i < W_V4; ++i)
      *reinterpret_cast<floatx4 *>(&Ws[(wr0 + kRowStep * i) * kSTR + wc]) = rw[i];
    float4 w0f = quad_pick(w0.q, 4 * lq, K0);
    set_elem(w0f, K0 - 4 * lq, w0.bn);  // no-op unless slot K0 is in this lane's quad
    floatx4 h = mfma4(w0f, xf, floatx4{0.f, 0.f, 0.f, 0.f});
    float4 o;
    o.x = mlp_act_select(h[0], p.act0);
    o.y = mlp_act_select(h[1], p.act0);
    o.z = mlp_act_select(h[2], p.act0);
    o.w = mlp_act_select(h[3], p.act0);
    *reinterpret_cast<float4 *>(&As[(16 * prb + l16) * kSTR + 16 * pcb + 4 * lq]) = o;
  };
  const int kgo = kg * kBK;
  auto frags = [&](const float *As, const float *Ws, int kq, float4 (&af)[2], float4 (&wf)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
      af[a] = *reinterpret_cast<const float4 *>(&As[(a * 16 + l16) * kSTR + kgo + kq + 4 * lq]);
#pragma unroll
    for (int b = 0; b < 4; ++b)
      wf[b] = *reinterpret_cast<const float4 *>(
          &Ws[(wn * 64 + b * 16 + l16) * kSTR + kgo + kq + 4 * lq]);
  };
  auto mfmas = [&](const float4 (&af)[2], const float4 (&wf)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[b].x, af[a].x, acc[a][b], 0, 0, 0);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[b].y, af[a].y, acc[a][b], 0, 0, 0);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[b].z, af[a].z, acc[a][b], 0, 0, 0);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[b].w, af[a].w, acc[a][b], 0, 0, 0);
  };
  auto compute = [&](int buf) __attribute__((always_inline)) {
    const float *As = lds + buf * (kA + kW);
    const float *Ws = As + kA;
    float4 af0[2], wf0[4], af1[2], wf1[4];
    frags(As, Ws, 0, af0, wf0);
#pragma unroll
    for (int kq = 0; kq < kBK; kq += 32) {
      frags(As, Ws, kq + 16, af1, wf1);
      mfmas(af0, wf0);
      if (kq + 32 < kBK) frags(As, Ws, kq + 32, af0, wf0);
      mfmas(af1, wf1);
    }
    __builtin_amdgcn_iglp_opt(1);
  };

  // Slab s + 1 is loaded into registers while slab s is multiplied from LDS
  // buffer s & 1, then stored to the other buffer: one register set (two
  // would exceed the 256 registers of two waves per SIMD, and the compiler
  // would then wait on every load), each load covered by a slab of MFMAs.
  floatx4 rw[W_V4];
  W0Frag w0f;
  fetch(0, rw, w0f);
  stash(0, rw, w0f);
  __syncthreads();
  int sl = 0;
  // (the scheduling barriers keep each slab's loads ahead of the MFMAs that
  // are to cover them)
  for (; sl + 2 < nslab; sl += 2) {  // steady state: both fetches exist
    fetch(sl + 1, rw, w0f);
    __builtin_amdgcn_sched_barrier(0);
    compute(0);
    __builtin_amdgcn_sched_barrier(0);
    stash(1, rw, w0f);
    __syncthreads();
    fetch(sl + 2, rw, w0f);
    __builtin_amdgcn_sched_barrier(0);
    compute(1);
    __builtin_amdgcn_sched_barrier(0);
    stash(0, rw, w0f);
    __syncthreads();
  }
  for (; sl < nslab; ++sl) {
    const bool more = sl + 1 < nslab;
    if (more) fetch(sl + 1, rw, w0f);
    compute(sl & 1);
    if (more) stash((sl + 1) & 1, rw, w0f);
    __syncthreads();
  }

  // Layer 2's W2 fragments: wave w computes rows [16 (w >> 2), +16) x
  // columns [16 (w & 3), +16) of y, k over h1's N1 columns in 16-wide steps.
  // All of the lane's W2 quads are loaded now (they do not depend on layer
  // 1), so their trip to L2 overlaps the reduction of layer 1 below.
  const int rb = wave >> 2, cb = wave & 3;
  const bool has_block = 16 * cb < N2;
  const float *w2row = p.W2 + (int64_t)(16 * min(cb, N2 / 16 - 1) + l16) * N1;
  constexpr int KQ = kBN / 16;
  float4 wf[KQ];
#pragma unroll
  for (int q = 0; q < KQ; ++q)
    wf[q] = 16 * q < N1 ? *reinterpret_cast<const float4 *>(w2row + 16 * q + 4 * lq)
                        : make_float4(0.f, 0.f, 0.f, 0.f);

  // Group 1 parks its partial tile in the idle slab buffers; group 0 adds it
  // (fixed order), applies bias and activation, and writes h1 to LDS (columns
  // at or past N1 as zeros, so layer 2 may read whole 16-column blocks).
  constexpr int PER = 2 * 4 * 4;  // floats per lane of a wave's tile
  if (kg == 1) {
    float *red = lds + (size_t)wn * PER * 64 + lane;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[((a * 4 + b) * 4 + v) * 64] = acc[a][b][v];
  }
  __syncthreads();
  float *H = lds + kPark;
  if (kg == 0) {
    const float *red = lds + (size_t)wn * PER * 64 + lane;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int n = wn * 64 + b * 16 + 4 * lq;
      float bv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) bv[v] = (p.b1 && n + v < N1) ? p.b1[n + v] : 0.0f;
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        float o[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float t = acc[a][b][v] + red[((a * 4 + b) * 4 + v) * 64];
          o[v] = (n + v < N1) ? mlp_act(t + bv[v], p.act1) : 0.0f;
        }
        *reinterpret_cast<float4 *>(&H[(a * 16 + l16) * kHS + n]) =
            make_float4(o[0], o[1], o[2], o[3]);
      }
    }
  }
  __syncthreads();

  // Layer 2 from h1 in LDS and the W2 fragments loaded above.
  if (!has_block) return;
  floatx4 y = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < KQ; ++q) {
    if (16 * q < N1) {
      const float4 hf =
          *reinterpret_cast<const float4 *>(&H[(16 * rb + l16) * kHS + 16 * q + 4 * lq]);
      y = mfma4(wf[q], hf, y);
    }
  }
  const int m = m0 + 16 * rb + l16;
  if (m >= M) return;
  const int n = 16 * cb + 4 * lq;
  float o[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) o[v] = mlp_act(y[v] + (p.b2 ? p.b2[n + v] : 0.0f), p.act2);
  float *cp = p.y + (int64_t)m * p.ldy + n;
  if (VC) {
    *reinterpret_cast<float4 *>(cp) = make_float4(o[0], o[1], o[2], o[3]);
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v) cp[v] = o[v];
  }
}

}  // namespace

bool bottom_mlp_supported(const BottomParams &p) {
  return p.K0 >= 4 && p.K0 <= 15 && p.N0 >= 2 * kSK && p.N0 % kSK == 0 && p.N1 >= 16 &&
         p.N1 <= kBN && p.N1 % 16 == 0 && p.N2 >= 16 && p.N2 <= 64 && p.N2 % 16 == 0 &&
         p.ldx >= p.K0 && p.ldy >= p.N2 && aligned16(p.W1) && aligned16(p.W2);
}

// One workgroup per 32 rows and per CU (157 KB of LDS): inside the forward
// the fused launch beats three layer launches when its grid is about one band
// per CU, 224..256 bands (measured at M = 8192: 34-35 us against 39.5 us;
// at M = 16384 the forward's fused MLP launches took 183.6 us against 178.7
// us for the layer launches, the second wave of bands costing more).
bool bottom_mlp_preferred(int M) {
  const int64_t bands = (int64_t)(M + kBM - 1) / kBM;
  return bands >= 224 && bands <= 256;
}

hipError_t launch_bottom_mlp(const BottomParams &p, hipStream_t stream) {
  if (!bottom_mlp_supported(p)) return hipErrorInvalidValue;
  const int tiles = (p.M + kBM - 1) / kBM;
  const int xcd_chunk = (tiles % 8 == 0) ? tiles / 8 : 0;
  const bool vc = aligned16(p.y) && p.ldy % 4 == 0;
  const dim3 grid((unsigned)tiles), block(kThreads);
  if (vc && p.b0)
    launch_kernel(bottom_mlp_kernel<true, true>, grid, block, 0, stream, p, xcd_chunk);
  else if (vc)
    launch_kernel(bottom_mlp_kernel<true, false>, grid, block, 0, stream, p, xcd_chunk);
  else if (p.b0)
    launch_kernel(bottom_mlp_kernel<false, true>, grid, block, 0, stream, p, xcd_chunk);
  else
    launch_kernel(bottom_mlp_kernel<false, false>, grid, block, 0, stream, p, xcd_chunk);
  return hipGetLastError();
}

}  // namespace dlrm
