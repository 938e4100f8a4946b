// mlp_chain.hip -- a stack of fused linear + bias + activation layers in one
// launch, for gfx950:
//   h_0 = A;  h_{l+1} = act_l(h_l W_l^T + b_l);  C = h_L
// ([FASTPATHS] matmul2d.rs, Activation epilogue; the DLRMv1 bottom and top
// MLPs of the commit message and translator notes), where [FASTPATHS] = page
// "luminal_python: vanilla-PyTorch DLRMv1 fast paths + batched FFI + input
// cache".
//
// Each workgroup carries BM = 32 rows through every layer.  The hidden
// activations of those rows stay in LDS (at most 32 x 512 floats), so no
// intermediate layer touches HBM and the whole stack pays one prologue and one
// epilogue.  With 4 waves (kWM = 2 would give 8), wave w
// owns output columns [(w%4) N/4, (w%4 + 1) N/4) of every row: a 32 x N/4 tile
// of v_mfma_f32_16x16x4f32 accumulators (TN = N/64 blocks of 16 columns).
//
// Where it pays: weights are read by every workgroup straight from L2, 16
// rows of 64 B per wave-load, so a wide first layer (415 -> 512) is paced by
// the vector memory path and runs slower than the tiled GEMM of linear.hip
// (top MLP 415-512-256-1 at 8192 rows: 136 us, against 64 us for the three
// layers as tiled launches).  With a narrow first layer (13 -> 512) the
// chain took 47 us against 40 us for three launches, and inside the full
// forward the three launches win as well; so dlrm_forward does not
// use it and mlp_forward, its own entry point, runs it for any supported
// stack.  Its A fragments (activation rows) come from LDS; its weight
// fragments come straight from global memory (every workgroup reads each
// weight once, the L2 serves the repeats), one k-quad ahead of the MFMAs that
// use them.  Layer 0 reads A from global through a double-buffered LDS slab.
// A last layer of N <= 8 columns (the 256 -> 1 sigmoid head) is a dot product
// per row, done on the VALU from the LDS activations.
//
// As in linear.hip, each lane feeds the 4 components of a float4 of 4
// consecutive k to 4 successive MFMAs (a permutation of the k order), and W
// is the first MFMA operand so a lane's accumulators are 4 consecutive output
// columns of one row.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dlrm {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 32;                 // rows per workgroup
constexpr int kWM = 1;                  // waves along the rows (1 or 2)
constexpr int kTM = 2 / kWM;            // 16-row MFMA blocks per wave
constexpr int kThreads = 256 * kWM;     // 4 column quarters x kWM row groups
constexpr int kSlab = 32;               // k per staged slab of the input
constexpr int kSlabStride = kSlab + 4;  // LDS row stride of the staged slab

__device__ __forceinline__ float chain_act(float x, int act) {
  if (act == 1) return x > 0.0f ? x : 0.0f;
  if (act == 2) return 1.0f / (1.0f + expf(-x));
  return x;
}

// float4 of k..k+3 of a row; columns at or past K read as zero (addresses
// clamped inside the row).
__device__ __forceinline__ float4 row_k4(const float *__restrict__ row, int k, int K, bool vec) {
  if (vec && k + 3 < K) return *reinterpret_cast<const float4 *>(row + k);
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int kk = k + e;
    const float x = row[kk < K ? kk : K - 1];
    v[e] = kk < K ? x : 0.0f;
  }
  return make_float4(v[0], v[1], v[2], v[3]);
}

// One MFMA layer.  A_GLOBAL: the input is p.A (global, staged through `slab`);
// else the input is the LDS activation tile h (row stride ldh).  The result,
// act(acc + bias), goes to LDS h (row stride ldo) when TO_LDS, else to p.C.
template <int TN, bool A_GLOBAL, bool TO_LDS>
__device__ __forceinline__ void chain_layer(const ChainParams &p, const ChainLayer &L, int m0,
                                            float *h, int ldh, int ldo, float *slab) {
  const int K = L.K, N = L.N;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int wq = wave & 3, wr = wave >> 2;  // column quarter, row group
  const int nw0 = wq * (N / 4);             // first output column of this wave
  const int r0 = wr * 16 * kTM;             // first row of this wave
  const bool wvec = ((K & 3) == 0) && aligned16(L.W);

  floatx4 acc[kTM][TN];
#pragma unroll
  for (int a = 0; a < kTM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  // weight row of block b: wbase + b * wstep
  const float *wbase = L.W + (int64_t)(nw0 + l16) * K;
  const int64_t wstep = (int64_t)16 * K;

  // Layer 0: rows of A staged one 32-k slab at a time (one float4 per thread
  // of the first 256).
  const bool stager = tid < 256;
  const int srow = (tid & 255) >> 3, scol = 4 * (tid & 7);
  const float *arow = A_GLOBAL ? p.A + (int64_t)min(m0 + srow, p.M - 1) * p.lda : nullptr;
  const bool avec = A_GLOBAL && ((p.lda & 3) == 0) && aligned16(p.A);
  if (A_GLOBAL) {
    if (stager)
      *reinterpret_cast<float4 *>(&slab[srow * kSlabStride + scol]) = row_k4(arow, scol, K, avec);
    __syncthreads();
  }

  float4 wf[TN], wn[TN];
#pragma unroll
  for (int b = 0; b < TN; ++b) wf[b] = row_k4(wbase + b * wstep, 4 * lq, K, wvec);
  float4 snext = make_float4(0.f, 0.f, 0.f, 0.f);

  for (int kq = 0; kq < K; kq += 16) {
    const bool more = kq + 16 < K;
    // weights of the next k-quad, in flight while this one's MFMAs run
    if (more) {
#pragma unroll
      for (int b = 0; b < TN; ++b) wn[b] = row_k4(wbase + b * wstep, kq + 16 + 4 * lq, K, wvec);
    }
    // the next input slab, loaded at the start of each slab
    const int kin = kq & (kSlab - 1);
    if (A_GLOBAL && stager && kin == 0 && kq + kSlab < K)
      snext = row_k4(arow, kq + kSlab + scol, K, avec);
    float4 af[kTM];
#pragma unroll
    for (int a = 0; a < kTM; ++a) {
      if (A_GLOBAL)
        af[a] = *reinterpret_cast<const float4 *>(
            &slab[((kq / kSlab) & 1) * kBM * kSlabStride + (r0 + a * 16 + l16) * kSlabStride +
                  kin + 4 * lq]);
      else
        af[a] = *reinterpret_cast<const float4 *>(&h[(r0 + a * 16 + l16) * ldh + kq + 4 * lq]);
    }
#pragma unroll
    for (int a = 0; a < kTM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[b].x, af[a].x, acc[a][b], 0, 0, 0);
#pragma unroll
    for (int a = 0; a < kTM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[b].y, af[a].y, acc[a][b], 0, 0, 0);
#pragma unroll
    for (int a = 0; a < kTM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[b].z, af[a].z, acc[a][b], 0, 0, 0);
#pragma unroll
    for (int a = 0; a < kTM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[b].w, af[a].w, acc[a][b], 0, 0, 0);
    if (more) {
#pragma unroll
      for (int b = 0; b < TN; ++b) wf[b] = wn[b];
    }
    // slab hand-over: the next slab goes to the other buffer after this one's
    // last k-quad; a barrier makes it visible (and retires the old buffer)
    if (A_GLOBAL && kin == kSlab - 16 && kq + 16 < K) {
      if (stager)
        *reinterpret_cast<float4 *>(
            &slab[(((kq / kSlab) + 1) & 1) * kBM * kSlabStride + srow * kSlabStride + scol]) =
            snext;
      __syncthreads();
    }
  }

  // Epilogue: lane holds rows a*16 + l16, columns nw0 + b*16 + 4*lq + 0..3.
  if (TO_LDS) __syncthreads();  // every wave is done reading the input tile
#pragma unroll
  for (int b = 0; b < TN; ++b) {
    const int n = nw0 + b * 16 + 4 * lq;
    const float4 bv = L.bias ? *reinterpret_cast<const float4 *>(L.bias + n)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int a = 0; a < kTM; ++a) {
      const int r = r0 + a * 16 + l16;
      const float4 o = make_float4(chain_act(acc[a][b][0] + bv.x, L.act),
                                   chain_act(acc[a][b][1] + bv.y, L.act),
                                   chain_act(acc[a][b][2] + bv.z, L.act),
                                   chain_act(acc[a][b][3] + bv.w, L.act));
      if (TO_LDS) {
        *reinterpret_cast<float4 *>(&h[r * ldo + n]) = o;
      } else if (m0 + r < p.M) {
        float *cp = p.C + (int64_t)(m0 + r) * p.ldc + n;
        if (p.c_vec) {
          *reinterpret_cast<float4 *>(cp) = o;
        } else {
          cp[0] = o.x;
          cp[1] = o.y;
          cp[2] = o.z;
          cp[3] = o.w;
        }
      }
    }
  }
  if (TO_LDS) __syncthreads();  // the new tile is visible to every wave
}

template <bool A_GLOBAL, bool TO_LDS>
__device__ __forceinline__ void chain_layer_tn(const ChainParams &p, const ChainLayer &L, int m0,
                                               float *h, int ldh, int ldo, float *slab) {
  switch (L.N / 64) {
    case 1: chain_layer<1, A_GLOBAL, TO_LDS>(p, L, m0, h, ldh, ldo, slab); break;
    case 2: chain_layer<2, A_GLOBAL, TO_LDS>(p, L, m0, h, ldh, ldo, slab); break;
    case 4: chain_layer<4, A_GLOBAL, TO_LDS>(p, L, m0, h, ldh, ldo, slab); break;
    default: chain_layer<8, A_GLOBAL, TO_LDS>(p, L, m0, h, ldh, ldo, slab); break;
  }
}

// Last layer with N <= 8: per row, N dot products of length K on the VALU
// from the LDS activations; 8 lanes per row (4 waves) or 16 (8 waves), DPP
// sums within those lanes.
__device__ __forceinline__ void chain_head(const ChainParams &p, const ChainLayer &L, int m0,
                                           const float *h, int ldh) {
  const int K = L.K;
  constexpr int LPR = 8 * kWM;  // lanes per row
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = wave * (64 / LPR) + lane / LPR;
  const int part = lane % LPR;
  const float *hr = h + r * ldh;
  for (int n = 0; n < L.N; ++n) {
    const float *w = L.W + (int64_t)n * K;
    float acc = 0.0f;
    for (int k = 4 * part; k < K; k += 4 * LPR) {
      const float4 x = *reinterpret_cast<const float4 *>(hr + k);
      acc = vdot_acc(x, row_k4(w, k, K, false), acc);
    }
    if (LPR == 16) {
      acc = row16_sum(acc);
    } else {
      // sum over the 8 lanes of the row: quad sum, then the other quad
      acc = quad_sum(acc);
      acc += __int_as_float(
          __builtin_amdgcn_update_dpp(0, __float_as_int(acc), 0x141, 0xF, 0xF, false));
    }
    if (part == 0 && m0 + r < p.M)
      p.C[(int64_t)(m0 + r) * p.ldc + n] = chain_act(acc + (L.bias ? L.bias[n] : 0.0f), L.act);
  }
}

__global__ __launch_bounds__(kThreads) void mlp_chain_kernel(ChainParams p) {
  extern __shared__ float4 lds_raw[];
  float *h = reinterpret_cast<float *>(lds_raw);           // kBM x (max hidden + 4)
  float *slab = h + kBM * p.ld_hidden;                    // 2 x kBM x kSlabStride
  const int m0 = blockIdx.x * kBM;
  const int last = p.nlayers - 1;
  int ldh = 0;
  // The layer loop is unrolled so every access to p.layer has a constant index
  // (a runtime index would copy the argument block to scratch).
#pragma unroll
  for (int l = 0; l < kMaxChainLayers; ++l) {
    if (l <= last) {
      const ChainLayer &L = p.layer[l];
      const int ldo = L.N + 4;
      if (l == last && L.N <= 8) {
        chain_head(p, L, m0, h, ldh);
      } else if (l == 0) {
        if (l < last)
          chain_layer_tn<true, true>(p, L, m0, h, 0, ldo, slab);
        else
          chain_layer_tn<true, false>(p, L, m0, h, 0, ldo, slab);
      } else {
        if (l < last)
          chain_layer_tn<false, true>(p, L, m0, h, ldh, ldo, slab);
        else
          chain_layer_tn<false, false>(p, L, m0, h, ldh, ldo, slab);
      }
      ldh = ldo;
    }
  }
}

}  // namespace

bool chain_supported(const ChainParams &p) {
  if (p.nlayers < 1 || p.nlayers > kMaxChainLayers) return false;
  const int last = p.nlayers - 1;
  for (int l = 0; l < p.nlayers; ++l) {
    const ChainLayer &L = p.layer[l];
    if (l > 0 && L.K != p.layer[l - 1].N) return false;
    const bool head = (l == last) && L.N <= 8;
    if (head) {
      if (l == 0 || (L.K & 3) != 0) return false;  // the head reads LDS rows
      continue;
    }
    const int tn = L.N / 64;
    if (L.N % 64 != 0 || L.N > kMaxChainWidth || (tn & (tn - 1)) != 0) return false;
    if (L.bias && !aligned16(L.bias)) return false;
  }
  return true;
}

hipError_t launch_mlp_chain(ChainParams p, hipStream_t stream) {
  int widest = 4;
  for (int l = 0; l + 1 < p.nlayers; ++l) widest = widest > p.layer[l].N ? widest : p.layer[l].N;
  p.ld_hidden = widest + 4;
  p.c_vec = (p.ldc % 4 == 0) && aligned16(p.C);
  const size_t lds = sizeof(float) * ((size_t)kBM * p.ld_hidden + 2 * kBM * kSlabStride);
  // up to 75 KiB of LDS per workgroup (the CU has 160 KiB): raise the limit
  // from the 64 KiB default once
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(mlp_chain_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)(sizeof(float) * ((size_t)kBM * (kMaxChainWidth + 4) + 2 * kBM * kSlabStride)));
  if (attr != hipSuccess) return attr;
  dim3 grid((unsigned)((p.M + kBM - 1) / kBM)), block(kThreads);
  launch_kernel(mlp_chain_kernel, grid, block, lds, stream, p);
  return hipGetLastError();
}

}  // namespace dlrm
