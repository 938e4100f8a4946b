// emb_interact.hip -- multi-table EmbeddingBag(sum) gather and the
// strict-lower-triangle pairwise-dot interaction, for gfx950.
//
// [FASTPATHS] = page "luminal_python: vanilla-PyTorch DLRMv1 fast paths +
//               batched FFI + input cache" (compare main...vanilla-pytorch).
//
// Gather ([FASTPATHS] embedding_bag.rs, "Semantics" and the multi-table
// kernel).  Every bag (b, k) is pooled by a group of G lanes; lane c of the
// group owns 16-byte column chunks c, c+G, ... of a row, so one wave-wide load
// instruction fetches 64 x 16 B of table rows.  A group first loads up to R of
// the bag's indices with one coalesced load per lane, broadcasts them inside
// the group with ds_bpermute (the LDS crossbar, no LDS storage), and then has
// all R row loads of the round in flight at once; the rows are added in bag
// order.  A bag of L <= R rows therefore costs one index round trip and one
// row round trip.  Row addresses are 64-bit: a table may exceed 2^31 floats.
// Shapes whose row is not a power-of-two number of 16-byte chunks (or not
// 16-byte aligned) take a generic path where each lane reads the indices
// itself.
//
// Interaction ([FASTPATHS] dlrm_interact.rs, the block-per-sample stacked
// kernel: all F feature rows of a sample cached on chip, then every pair).
// A workgroup stages the F x D tile of S samples in LDS (row stride D+4 floats
// so that consecutive rows start on different banks).  The strict lower
// triangle of Z = X X^T is cut into 4 x 4 blocks of (row i, row j) pairs; a
// quad of lanes owns one block at a time, each lane multiplying a quarter of
// the D columns of the 4 + 4 rows into 16 partial dots (so every LDS read of a
// row serves 4 dots), and a transposed quad reduction with DPP permutations
// leaves each lane with 4 finished dots.  Block t of the lower triangle maps
// to block row I = floor((sqrt(8t+1) - 1) / 2), the closed form of the pages'
// pair map applied to blocks; a dot (i, j) lands at p = i(i-1)/2 + j.  The
// scalar path keeps one quad per dot with p -> (i, j) in closed form.
// The fused kernel pools straight into the LDS tile, so the (B, K, D) pooled
// tensor never round-trips through HBM.
#include "common.hpp"
#include "kernels.hpp"

namespace dlrm {

namespace {

#ifndef DLRM_GATHER_ROUND
#define DLRM_GATHER_ROUND 12
#endif
#ifndef DLRM_ROW_NT
#define DLRM_ROW_NT 0
#endif
#ifndef DLRM_MIN_THREADS
#define DLRM_MIN_THREADS 256
#endif

constexpr int kUnroll = 8;                  // generic path: loads in flight per lane
constexpr int kRound = DLRM_GATHER_ROUND;   // shuffle path: row loads in flight per lane

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

// Generic path: pools bag [s, e) of `tab` for column chunk c (VW floats wide)
// of a row of nvec chunks, each lane reading the indices itself.
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

// Shuffle path (G lanes per group, G a power of two <= 64, nvec % G == 0):
// pools bag [s, e) for column chunk c of float4 width.  Every lane of the
// group must call this together (the index broadcast reads the other lanes);
// gbase is the wave lane of the group's first lane.
template <int G>
__device__ __forceinline__ float4 pool_group(const float *__restrict__ tab,
                                             const int32_t *__restrict__ idx, int s, int e,
                                             int nvec, int c_lane, int c, int gbase) {
  constexpr int T = (kRound + G - 1) / G;  // index registers per lane
  const float4 *col = reinterpret_cast<const float4 *>(tab) + c;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int l0 = s; l0 < e; l0 += kRound) {
    const int n = min(kRound, e - l0);
    int mine[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int l = c_lane + G * t;
      mine[t] = (l < n) ? idx[l0 + l] : 0;
    }
    float4 v[kRound];
#pragma unroll
    for (int u = 0; u < kRound; ++u) {
      const int r = __builtin_amdgcn_ds_bpermute((gbase + (u % G)) << 2, mine[u / G]);
#if DLRM_ROW_NT
      typedef float f4v __attribute__((ext_vector_type(4)));
      f4v tv = (u < n) ? __builtin_nontemporal_load(reinterpret_cast<const f4v *>(
                             col + (size_t)(uint32_t)r * (size_t)nvec))
                       : f4v{0.f, 0.f, 0.f, 0.f};
      v[u] = make_float4(tv.x, tv.y, tv.z, tv.w);
#else
      v[u] = (u < n) ? col[(size_t)(uint32_t)r * (size_t)nvec] : make_float4(0.f, 0.f, 0.f, 0.f);
#endif
    }
#pragma unroll
    for (int u = 0; u < kRound; ++u)
      if (u < n) acc = operator_add(acc, v[u]);
  }
  return acc;
}

// Pools bag (b, k) into `row` (nvec chunks of VW floats) and optionally `eo`.
// All G lanes of the group call it together.
template <int VW, int GS, bool CSR>
__device__ __forceinline__ void pool_bag(const TableSet &ts, int k, int b, int B, int nvec,
                                         int G, int c0, typename Vec<VW>::T *row,
                                         typename Vec<VW>::T *eo) {
  using V = typename Vec<VW>::T;
  int bs, be;
  bag_bounds<CSR>(ts, k, b, B, bs, be);
  for (int c = c0; c < nvec; c += G) {
    V v;
    if constexpr (GS > 0) {
      const int gbase = (threadIdx.x & 63) & ~(GS - 1);
      v = pool_group<GS>(ts.table[k], ts.idx[k], bs, be, nvec, c0, c, gbase);
    } else {
      v = pool_chunk<VW>(ts.table[k], ts.idx[k], bs, be, nvec, c);
    }
    row[c] = v;
    if (eo) eo[c] = v;
  }
}

// ---------------------------------------------------------------------------
// emb_bag_sum_multi: grid over bags, one group of G lanes per bag (b, k).
// ---------------------------------------------------------------------------
template <int VW, int GS, bool CSR>
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
  V *dst = reinterpret_cast<V *>(out + task * D);
  pool_bag<VW, GS, CSR>(ts, k, b, B, D / VW, G, c0, dst, nullptr);
}

// ---------------------------------------------------------------------------
// Interaction (and fused gather + interaction): one workgroup per S samples.
// MODE_FUSED pools the bags into the LDS tile; MODE_LOAD reads a (B, K, D)
// pooled tensor.
// ---------------------------------------------------------------------------
enum { MODE_FUSED = 0, MODE_LOAD = 1 };

// One quad per dot, p -> (i, j) in closed form (any D; used by the scalar path).
template <int VW>
__device__ __forceinline__ void dots_per_pair(const float *X, const InteractParams &ip, int b0,
                                              int FR) {
  using V = typename Vec<VW>::T;
  const int D = ip.D, P = ip.P, DP = ip.DP, nvec = D / VW;
  const int quads = blockDim.x >> 2;
  const int q = threadIdx.x >> 2;
  const int r = threadIdx.x & 3;
  const int total = ip.S * P;
  for (int t = q; t < total; t += quads) {
    const int s = t / P;
    const int p = t - s * P;
    int i, j;
    pair_from_index((uint32_t)p, i, j);
    const V *xi = reinterpret_cast<const V *>(X + (size_t)(s * FR + i) * DP);
    const V *xj = reinterpret_cast<const V *>(X + (size_t)(s * FR + j) * DP);
    float acc = 0.0f;
    for (int c = r; c < nvec; c += 4) acc = vdot_acc(xi[c], xj[c], acc);
    acc = quad_sum(acc);
    const int b = b0 + s;
    if (r == 0 && b < ip.B) ip.out[(int64_t)b * ip.ld_out + D + p] = acc;
  }
}

// Quad exchange helper: value of `v` in lane (lane ^ 1) or (lane ^ 2).
__device__ __forceinline__ float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
// Value of `v` in lane (lane + n) of the same 16-lane row (0 past the row end).
__device__ __forceinline__ float dpp_row_shl(float v, int n) {
  const int x = __float_as_int(v);
  return __int_as_float(n == 4 ? __builtin_amdgcn_update_dpp(0, x, 0x104, 0xF, 0xF, false)
                               : __builtin_amdgcn_update_dpp(0, x, 0x108, 0xF, 0xF, false));
}

// 4 x 4 blocked dots (float4 path).  The tile holds FR = 4*ceil(F/4) rows per
// sample; rows F..FR-1 are never stored out.  A team of Q quads (Q = 1, 2 or
// 4, so a team never straddles a 16-lane DPP row) owns one block: its lanes
// split the D columns, each quad reduces its 16 partial dots to 4 per lane,
// and row shifts of 4 and 8 lanes add the quads' results into the first quad.
__device__ __forceinline__ void dots_blocked(const float *X, const InteractParams &ip, int b0,
                                             int FR) {
  const int D = ip.D, DP = ip.DP, F = ip.K + 1, nvec = D / 4;
  const int nb = FR >> 2;
  const int nblk = nb * (nb + 1) / 2;  // lower-triangle blocks incl. the diagonal
  const int Q = ip.Q;
  const int lanes = 4 * Q;
  const int teams = blockDim.x / lanes;
  const int team = threadIdx.x / lanes;
  const int tl = threadIdx.x - team * lanes;  // lane within the team
  const int r = tl & 3;
  const int total = ip.S * nblk;
  for (int t = team; t < total; t += teams) {
    const int s = t / nblk;
    const int tb = t - s * nblk;
    // block row I: largest I with I(I+1)/2 <= tb, i.e. (isqrt(8 tb + 1) - 1) / 2
    int I, J;
    {
      const uint32_t qv = 8u * (uint32_t)tb + 1u;
      uint32_t rt = (uint32_t)__builtin_sqrtf((float)qv);
      rt -= (rt * rt > qv) ? 1u : 0u;
      rt += ((rt + 1) * (rt + 1) <= qv) ? 1u : 0u;
      I = (int)((rt - 1) >> 1);
      J = tb - I * (I + 1) / 2;
    }
    const float *base = X + (size_t)(s * FR) * DP;
    const float4 *xi = reinterpret_cast<const float4 *>(base + (size_t)(4 * I) * DP);
    const float4 *xj = reinterpret_cast<const float4 *>(base + (size_t)(4 * J) * DP);
    const int st = DP >> 2;  // row stride in float4
    float acc[16];
#pragma unroll
    for (int n = 0; n < 16; ++n) acc[n] = 0.0f;
    for (int c = tl; c < nvec; c += lanes) {
      float4 a[4], bv[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) a[x] = xi[x * st + c];
#pragma unroll
      for (int y = 0; y < 4; ++y) bv[y] = xj[y * st + c];
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x * 4 + y] = vdot_acc(a[x], bv[y], acc[x * 4 + y]);
    }
    // Transposed quad reduction: 16 partial sums per lane -> 4 totals per lane.
    const bool o1 = (r & 1) != 0, o2 = (r & 2) != 0;
    float w[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const float send = o1 ? acc[n] : acc[8 + n];
      const float keep = o1 ? acc[8 + n] : acc[n];
      w[n] = keep + dpp_xor1(send);
    }
    float z[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const float send = o2 ? w[n] : w[4 + n];
      const float keep = o2 ? w[4 + n] : w[n];
      z[n] = keep + dpp_xor2(send);
    }
    // Add the other quads of the team into quad 0 (lane i += lane i + 4, + 8).
    if (Q >= 2) {
#pragma unroll
      for (int n = 0; n < 4; ++n) z[n] += dpp_row_shl(z[n], 4);
    }
    if (Q >= 4) {
#pragma unroll
      for (int n = 0; n < 4; ++n) z[n] += dpp_row_shl(z[n], 8);
    }
    // lane r of quad 0 holds dots (4I + x, 4J + y), y = 0..3, x = 2*(r&1) + ((r>>1)&1)
    const int i = 4 * I + 2 * (r & 1) + ((r >> 1) & 1);
    const int b = b0 + s;
    if (tl < 4 && b < ip.B && i < F) {
      float *o = ip.out + (int64_t)b * ip.ld_out + D + i * (i - 1) / 2;
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int j = 4 * J + y;
        if (j < i) o[j] = z[y];
      }
    }
  }
}

template <int VW, int MODE, bool CSR, int GS>
__global__ __launch_bounds__(1024) void interact_kernel(TableSet ts, InteractParams ip) {
  using V = typename Vec<VW>::T;
  extern __shared__ float4 lds_raw[];
  float *X = reinterpret_cast<float *>(lds_raw);
  const int B = ip.B, K = ip.K, D = ip.D, S = ip.S, DP = ip.DP;
  const int FR = ip.FR;  // tile rows per sample (F, or F rounded up to 4)
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
    reinterpret_cast<V *>(X + (size_t)(s * FR) * DP)[c] = v;
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
      V *row = reinterpret_cast<V *>(X + (size_t)(s * FR + 1 + k) * DP);
      if (MODE == MODE_FUSED) {
        V *eo = ip.emb_out ? reinterpret_cast<V *>(ip.emb_out + ((int64_t)b * K + k) * D) : nullptr;
        pool_bag<VW, GS, CSR>(ts, k, b, B, nvec, G, c0, row, eo);
      } else {
        const V *src = reinterpret_cast<const V *>(ip.emb_in + ((int64_t)b * K + k) * D);
        for (int c = c0; c < nvec; c += G) row[c] = src[c];
      }
    }
  }
  __syncthreads();

  // Phase 2: the strict-lower-triangle dots.
  if constexpr (VW == 4)
    dots_blocked(X, ip, b0, FR);
  else
    dots_per_pair<VW>(X, ip, b0, FR);
}

// Shuffle-path group size for a row of nvec float4 chunks (0: generic path).
// Rows narrower than 4 chunks keep the generic path: with 1 or 2 lanes per
// group the index registers of a round would not fit beside the row loads.
int shuffle_group(int nvec) {
  if (nvec < 4) return 0;
  if (nvec <= 64 && (nvec & (nvec - 1)) == 0) return nvec;
  if (nvec % 64 == 0) return 64;
  return 0;
}

}  // namespace

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
static int lanes_per_row(int D, int VW) {
  const int nvec = D / VW;
  return nvec < kWave ? nvec : kWave;
}

#define DLRM_GS_SWITCH(gs, BODY)            \
  switch (gs) {                             \
    case 4: { constexpr int GSV = 4; BODY; } break;   \
    case 8: { constexpr int GSV = 8; BODY; } break;   \
    case 16: { constexpr int GSV = 16; BODY; } break; \
    case 32: { constexpr int GSV = 32; BODY; } break; \
    case 64: { constexpr int GSV = 64; BODY; } break; \
    default: { constexpr int GSV = 0; BODY; } break;  \
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
    const int gs = shuffle_group(D / 4);
    if (csr) {
      DLRM_GS_SWITCH(gs, hipLaunchKernelGGL((emb_bag_kernel<4, GSV, true>), grid, block, 0,
                                            stream, ts, B, K, D, G, out));
    } else {
      DLRM_GS_SWITCH(gs, hipLaunchKernelGGL((emb_bag_kernel<4, GSV, false>), grid, block, 0,
                                            stream, ts, B, K, D, G, out));
    }
  } else {
    if (csr)
      hipLaunchKernelGGL((emb_bag_kernel<1, 0, true>), grid, block, 0, stream, ts, B, K, D, G,
                         out);
    else
      hipLaunchKernelGGL((emb_bag_kernel<1, 0, false>), grid, block, 0, stream, ts, B, K, D, G,
                         out);
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
  ip.FR = vec4 ? ((F + 3) & ~3) : F;
  ip.G = lanes_per_row(D, VW);
  const size_t per_sample = (size_t)ip.FR * ip.DP * sizeof(float);
  if (per_sample > kLdsBudget) return false;
  const int lanes_per_sample = K * ip.G;
  int S = 1;
  while (S * lanes_per_sample < DLRM_MIN_THREADS &&
         (size_t)(2 * S) * per_sample <= kLdsBudget / 2 &&
         S < B)
    S *= 2;
  ip.S = S;
  int want = S * lanes_per_sample;
  if (want > 1024) want = 1024;
  threads = ((want + kWave - 1) / kWave) * kWave;
  if (threads < DLRM_MIN_THREADS) threads = DLRM_MIN_THREADS;
  ip.lds_bytes = (int)(S * per_sample);
  // Quads per 4 x 4 block team: the most that still covers every block of the
  // workgroup in one pass, so the interaction phase runs on as many waves as
  // possible with each lane doing the least work.
  const int nbr = ip.FR / 4;
  const int work = S * nbr * (nbr + 1) / 2;
  const int quads = threads / 4;
  ip.Q = (work * 4 <= quads) ? 4 : (work * 2 <= quads) ? 2 : 1;
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
      const int gs = shuffle_group(ip.D / 4);
      if (csr) {
        DLRM_GS_SWITCH(gs, hipLaunchKernelGGL((interact_kernel<4, MODE_FUSED, true, GSV>), grid,
                                              block, lds, stream, t, ip));
      } else {
        DLRM_GS_SWITCH(gs, hipLaunchKernelGGL((interact_kernel<4, MODE_FUSED, false, GSV>), grid,
                                              block, lds, stream, t, ip));
      }
    } else {
      if (csr)
        hipLaunchKernelGGL((interact_kernel<1, MODE_FUSED, true, 0>), grid, block, lds, stream, t,
                           ip);
      else
        hipLaunchKernelGGL((interact_kernel<1, MODE_FUSED, false, 0>), grid, block, lds, stream,
                           t, ip);
    }
  } else {
    if (vec4)
      hipLaunchKernelGGL((interact_kernel<4, MODE_LOAD, false, 0>), grid, block, lds, stream, t,
                         ip);
    else
      hipLaunchKernelGGL((interact_kernel<1, MODE_LOAD, false, 0>), grid, block, lds, stream, t,
                         ip);
  }
  return hipGetLastError();
}

}  // namespace dlrm
