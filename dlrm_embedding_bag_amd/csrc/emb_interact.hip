// emb_interact.hip -- multi-table EmbeddingBag(sum) gather and the
// strict-lower-triangle pairwise-dot interaction, for gfx950.
//
// [FASTPATHS] = page "luminal_python: vanilla-PyTorch DLRMv1 fast paths +
//               batched FFI + input cache" (compare main...vanilla-pytorch).
//
// Gather ([FASTPATHS] embedding_bag.rs, "Semantics" and the multi-table
// kernel): every bag (b, k) is pooled by a group of G lanes; lane c of the
// group owns 16-byte column chunks c, c+G, ... of the row, so one wave-wide
// load instruction fetches 64 x 16 B of table rows, and each lane keeps up to
// eight independent row loads in flight before it adds them (in bag order).
// Row addresses are 64-bit: a table may exceed 2^31 elements.
//
// Interaction ([FASTPATHS] dlrm_interact.rs, the block-per-sample stacked
// kernel): a workgroup stages the F x D feature tile of S samples in LDS
// (row stride D+4 floats so rows start on different banks), then each quad of
// lanes computes one dot at a time: each lane sums a quarter of the D
// products and two DPP quad permutations finish the reduction.  Pair p is
// mapped to (i, j) in closed form.  The fused kernel pools straight into the
// LDS tile, so the (B, K, D) pooled tensor never round-trips through HBM.
#include "common.hpp"
#include "kernels.hpp"

namespace dlrm {

namespace {

constexpr int kUnroll = 8;

__device__ __forceinline__ void store_unaligned(float *p, float4 v) {
  p[0] = v.x;
  p[1] = v.y;
  p[2] = v.z;
  p[3] = v.w;
}
__device__ __forceinline__ void store_unaligned(float *p, float v) { p[0] = v; }

template <bool CSR>
__device__ __forceinline__ void bag_bounds(const TableSet &ts, int k, int b, int B,
                                           int &s, int &e) {
  if (CSR) {
    const int n = ts.nidx[k];
    const int32_t *o = ts.off[k];
    int lo = o[b];
    int hi = (b + 1 < B) ? o[b + 1] : n;
    lo = min(max(lo, 0), n);
    hi = min(max(hi, lo), n);
    s = lo;
    e = hi;
  } else {
    const int L = ts.bag[k];
    s = b * L;  // b * L <= n_idx <= INT32_MAX, checked on the host
    e = s + L;
  }
}

// Pools bag [s, e) of `tab` for column chunk c (VW floats wide) of a row of
// nvec chunks.  Rows are added in bag order.
template <int VW>
__device__ __forceinline__ typename Vec<VW>::T pool_chunk(const float *__restrict__ tab,
                                                          const int32_t *__restrict__ idx,
                                                          int s, int e, int nvec, int c) {
  using V = typename Vec<VW>::T;
  const V *col = reinterpret_cast<const V *>(tab) + c;
  V acc = vzero<V>();
  int l = s;
  for (; l + kUnroll <= e; l += kUnroll) {
    int r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) r[u] = idx[l + u];
    V v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = col[(size_t)(uint32_t)r[u] * (size_t)nvec];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc = operator_add(acc, v[u]);
  }
  const int rem = e - l;
  if (rem > 0) {
    // Tail of up to kUnroll - 1 rows: predicated loads stay in flight together.
    int r[kUnroll - 1];
#pragma unroll
    for (int u = 0; u < kUnroll - 1; ++u) r[u] = (u < rem) ? idx[l + u] : 0;
    V v[kUnroll - 1];
#pragma unroll
    for (int u = 0; u < kUnroll - 1; ++u)
      v[u] = (u < rem) ? col[(size_t)(uint32_t)r[u] * (size_t)nvec] : vzero<V>();
#pragma unroll
    for (int u = 0; u < kUnroll - 1; ++u)
      if (u < rem) acc = operator_add(acc, v[u]);
  }
  return acc;
}

// ---------------------------------------------------------------------------
// emb_bag_sum_multi: grid over bags, one group of G lanes per bag (b, k).
// ---------------------------------------------------------------------------
template <int VW, bool CSR>
__global__ __launch_bounds__(256) void emb_bag_kernel(TableSet ts, int B, int K, int D,
                                                      int G, float *__restrict__ out) {
  using V = typename Vec<VW>::T;
  const int groups = blockDim.x / G;
  const int g = threadIdx.x / G;
  const int c0 = threadIdx.x - g * G;
  if (g >= groups) return;
  const int64_t task = (int64_t)blockIdx.x * groups + g;
  if (task >= (int64_t)B * K) return;
  const int b = (int)(task / K);
  const int k = (int)(task - (int64_t)b * K);
  int s, e;
  bag_bounds<CSR>(ts, k, b, B, s, e);
  const int nvec = D / VW;
  V *dst = reinterpret_cast<V *>(out + task * D);
  for (int c = c0; c < nvec; c += G) dst[c] = pool_chunk<VW>(ts.table[k], ts.idx[k], s, e, nvec, c);
}

// ---------------------------------------------------------------------------
// Interaction (and fused gather + interaction): one workgroup per S samples.
// MODE_FUSED pools the bags into the LDS tile; MODE_LOAD reads a (B, K, D)
// pooled tensor.
// ---------------------------------------------------------------------------
enum { MODE_FUSED = 0, MODE_LOAD = 1 };

template <int VW, int MODE, bool CSR>
__global__ __launch_bounds__(1024) void interact_kernel(TableSet ts, InteractParams ip) {
  using V = typename Vec<VW>::T;
  extern __shared__ float4 lds_raw[];
  float *X = reinterpret_cast<float *>(lds_raw);
  const int B = ip.B, K = ip.K, D = ip.D, S = ip.S, DP = ip.DP;
  const int F = K + 1;
  const int P = ip.P;
  const int nvec = D / VW;
  const int b0 = blockIdx.x * S;
  const int nthreads = blockDim.x;

  // Phase 1a: dense rows -> feature 0 of each sample (and the output copy).
  for (int t = threadIdx.x; t < S * nvec; t += nthreads) {
    const int s = t / nvec;
    const int c = t - s * nvec;
    const int b = b0 + s;
    if (b >= B) continue;
    const V v = reinterpret_cast<const V *>(ip.dense + (int64_t)b * ip.ld_dense)[c];
    reinterpret_cast<V *>(X + (size_t)(s * F) * DP)[c] = v;
    if (ip.copy_dense) {
      float *o = ip.out + (int64_t)b * ip.ld_out;
      if (VW == 1 || ip.out_vec)
        reinterpret_cast<V *>(o)[c] = v;
      else
        store_unaligned(o + c * VW, v);
    }
  }

  // Phase 1b: pooled rows -> features 1..K.
  const int G = ip.G;
  const int groups = nthreads / G;
  const int g = threadIdx.x / G;
  const int c0 = threadIdx.x - g * G;
  if (g < groups) {
    for (int t = g; t < S * K; t += groups) {
      const int s = t / K;
      const int k = t - s * K;
      const int b = b0 + s;
      if (b >= B) continue;
      V *row = reinterpret_cast<V *>(X + (size_t)(s * F + 1 + k) * DP);
      if (MODE == MODE_FUSED) {
        int bs, be;
        bag_bounds<CSR>(ts, k, b, B, bs, be);
        V *eo = ip.emb_out ? reinterpret_cast<V *>(ip.emb_out + ((int64_t)b * K + k) * D) : nullptr;
        for (int c = c0; c < nvec; c += G) {
          const V v = pool_chunk<VW>(ts.table[k], ts.idx[k], bs, be, nvec, c);
          row[c] = v;
          if (eo) eo[c] = v;
        }
      } else {
        const V *src = reinterpret_cast<const V *>(ip.emb_in + ((int64_t)b * K + k) * D);
        for (int c = c0; c < nvec; c += G) row[c] = src[c];
      }
    }
  }
  __syncthreads();

  // Phase 2: one quad of lanes per dot product.
  const int quads = nthreads >> 2;
  const int q = threadIdx.x >> 2;
  const int r = threadIdx.x & 3;
  const int total = S * P;
  for (int t = q; t < total; t += quads) {
    const int s = t / P;
    const int p = t - s * P;
    int i, j;
    pair_from_index((uint32_t)p, i, j);
    const V *xi = reinterpret_cast<const V *>(X + (size_t)(s * F + i) * DP);
    const V *xj = reinterpret_cast<const V *>(X + (size_t)(s * F + j) * DP);
    float acc = 0.0f;
    for (int c = r; c < nvec; c += 4) acc = vdot_acc(xi[c], xj[c], acc);
    acc = quad_sum(acc);
    const int b = b0 + s;
    if (r == 0 && b < B) ip.out[(int64_t)b * ip.ld_out + D + p] = acc;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
static int lanes_per_row(int D, int VW) {
  const int nvec = D / VW;
  return nvec < kWave ? nvec : kWave;
}

hipError_t launch_emb_bag(const TableSet &ts, bool csr, int B, int K, int D, bool vec4,
                          float *out, hipStream_t stream) {
  const int VW = vec4 ? 4 : 1;
  const int G = lanes_per_row(D, VW);
  const int threads = 256;
  const int groups = threads / G;
  const int64_t tasks = (int64_t)B * K;
  const int64_t blocks = (tasks + groups - 1) / groups;
  dim3 grid((unsigned)blocks), block(threads);
  if (vec4) {
    if (csr)
      hipLaunchKernelGGL((emb_bag_kernel<4, true>), grid, block, 0, stream, ts, B, K, D, G, out);
    else
      hipLaunchKernelGGL((emb_bag_kernel<4, false>), grid, block, 0, stream, ts, B, K, D, G, out);
  } else {
    if (csr)
      hipLaunchKernelGGL((emb_bag_kernel<1, true>), grid, block, 0, stream, ts, B, K, D, G, out);
    else
      hipLaunchKernelGGL((emb_bag_kernel<1, false>), grid, block, 0, stream, ts, B, K, D, G, out);
  }
  return hipGetLastError();
}

bool plan_interact(int B, int K, int D, bool vec4, InteractParams &ip, int &threads) {
  const int VW = vec4 ? 4 : 1;
  const int F = K + 1;
  ip.B = B;
  ip.K = K;
  ip.D = D;
  ip.P = F * (F - 1) / 2;
  ip.DP = D + (vec4 ? 4 : 1);
  ip.G = lanes_per_row(D, VW);
  const size_t per_sample = (size_t)F * ip.DP * sizeof(float);
  if (per_sample > kLdsBudget) return false;
  const int lanes_per_sample = K * ip.G;
  int S = 1;
  while (S * lanes_per_sample < 256 && (size_t)(2 * S) * per_sample <= kLdsBudget / 2 &&
         S < B)
    S *= 2;
  ip.S = S;
  int want = S * lanes_per_sample;
  if (want > 1024) want = 1024;
  threads = ((want + kWave - 1) / kWave) * kWave;
  if (threads < 256) threads = 256;
  ip.lds_bytes = (int)(S * per_sample);
  return true;
}

hipError_t launch_interact(const TableSet *ts, bool csr, const InteractParams &ip, int threads,
                           bool vec4, hipStream_t stream) {
  dim3 grid((unsigned)((ip.B + ip.S - 1) / ip.S)), block(threads);
  const size_t lds = (size_t)ip.lds_bytes;
  TableSet empty{};
  const TableSet &t = ts ? *ts : empty;
  if (ts) {
    if (vec4) {
      if (csr)
        hipLaunchKernelGGL((interact_kernel<4, MODE_FUSED, true>), grid, block, lds, stream, t, ip);
      else
        hipLaunchKernelGGL((interact_kernel<4, MODE_FUSED, false>), grid, block, lds, stream, t, ip);
    } else {
      if (csr)
        hipLaunchKernelGGL((interact_kernel<1, MODE_FUSED, true>), grid, block, lds, stream, t, ip);
      else
        hipLaunchKernelGGL((interact_kernel<1, MODE_FUSED, false>), grid, block, lds, stream, t, ip);
    }
  } else {
    if (vec4)
      hipLaunchKernelGGL((interact_kernel<4, MODE_LOAD, false>), grid, block, lds, stream, t, ip);
    else
      hipLaunchKernelGGL((interact_kernel<1, MODE_LOAD, false>), grid, block, lds, stream, t, ip);
  }
  return hipGetLastError();
}

}  // namespace dlrm
