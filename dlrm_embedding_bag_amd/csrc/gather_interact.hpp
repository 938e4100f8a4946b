// gather_interact.hpp -- device building blocks of the gather and the
// interaction, shared by the kernels of emb_interact.hip and
// forward_small.hip (internal; gfx950).
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
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace dlrm {


// Row loads in flight per lane on the shuffle path, by table storage type
// (measured on MI355X: 10, 12 and 16 float32 rows gave the same time, 20
// spilled; fp8 keeps 8, since its weighted instantiations spill at 12).
constexpr int kRoundF32 = 12, kRoundBF16 = 12, kRoundFP8 = 8;
// Smallest workgroup of the interaction kernels.
constexpr int kMinThreads = 128;

constexpr int kUnroll = 8;  // generic path: loads in flight per lane
// Shuffle path: row loads in flight per lane, by table storage type.
template <typename TT>
constexpr int kRound = sizeof(TT) == 1 ? kRoundFP8 : sizeof(TT) == 2 ? kRoundBF16 : kRoundF32;

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

// A row chunk: what one lane loads per row.  On the vector path it is 16
// bytes (4 float32 or 8 bfloat16 elements), on the scalar path one element.
// bfloat16 is widened to float32 exactly (its bits are the high half of the
// float32), and the bag is accumulated in float32.
template <typename TT, int VW>
struct RowChunk;

template <>
struct RowChunk<float, 4> {
  using Raw = float4;
  static constexpr int EL = 4;
  static __device__ __forceinline__ Raw zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  static __device__ __forceinline__ void add(float *a, Raw r) {
    a[0] += r.x;
    a[1] += r.y;
    a[2] += r.z;
    a[3] += r.w;
  }
  static __device__ __forceinline__ void fma(float *a, float w, Raw r) {
    a[0] = __builtin_fmaf(w, r.x, a[0]);
    a[1] = __builtin_fmaf(w, r.y, a[1]);
    a[2] = __builtin_fmaf(w, r.z, a[2]);
    a[3] = __builtin_fmaf(w, r.w, a[3]);
  }
};

template <>
struct RowChunk<float, 1> {
  using Raw = float;
  static constexpr int EL = 1;
  static __device__ __forceinline__ Raw zero() { return 0.f; }
  static __device__ __forceinline__ void add(float *a, Raw r) { a[0] += r; }
  static __device__ __forceinline__ void fma(float *a, float w, Raw r) {
    a[0] = __builtin_fmaf(w, r, a[0]);
  }
};

// bfloat16 element 2i of a chunk is the low half of 32-bit word i.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <>
struct RowChunk<uint16_t, 4> {
  using Raw = uint4;
  static constexpr int EL = 8;
  static __device__ __forceinline__ Raw zero() { return make_uint4(0u, 0u, 0u, 0u); }
  static __device__ __forceinline__ void add(float *a, Raw r) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[2 * i] += bf16_lo(w[i]);
      a[2 * i + 1] += bf16_hi(w[i]);
    }
  }
  static __device__ __forceinline__ void fma(float *a, float wt, Raw r) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[2 * i] = __builtin_fmaf(wt, bf16_lo(w[i]), a[2 * i]);
      a[2 * i + 1] = __builtin_fmaf(wt, bf16_hi(w[i]), a[2 * i + 1]);
    }
  }
};

template <>
struct RowChunk<uint16_t, 1> {
  using Raw = uint16_t;
  static constexpr int EL = 1;
  static __device__ __forceinline__ Raw zero() { return 0; }
  static __device__ __forceinline__ void add(float *a, Raw r) { a[0] += bf16_lo(r); }
  static __device__ __forceinline__ void fma(float *a, float w, Raw r) {
    a[0] = __builtin_fmaf(w, bf16_lo(r), a[0]);
  }
};

// FP8 E4M3 (the OCP "fn" encoding) codes, decoded by the hardware
// conversion, which yields the exact value of each code: bytes 0-1 of a
// 32-bit word with word_sel false, bytes 2-3 with true.
template <>
struct RowChunk<uint8_t, 4> {
  using Raw = uint4;
  static constexpr int EL = 16;
  static __device__ __forceinline__ Raw zero() { return make_uint4(0u, 0u, 0u, 0u); }
  static __device__ __forceinline__ void add(float *a, Raw r) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
      a[4 * i] += lo[0];
      a[4 * i + 1] += lo[1];
      a[4 * i + 2] += hi[0];
      a[4 * i + 3] += hi[1];
    }
  }
  static __device__ __forceinline__ void fma(float *a, float wt, Raw r) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
      a[4 * i] = __builtin_fmaf(wt, lo[0], a[4 * i]);
      a[4 * i + 1] = __builtin_fmaf(wt, lo[1], a[4 * i + 1]);
      a[4 * i + 2] = __builtin_fmaf(wt, hi[0], a[4 * i + 2]);
      a[4 * i + 3] = __builtin_fmaf(wt, hi[1], a[4 * i + 3]);
    }
  }
};

template <>
struct RowChunk<uint8_t, 1> {
  using Raw = uint8_t;
  static constexpr int EL = 1;
  static __device__ __forceinline__ Raw zero() { return 0; }
  static __device__ __forceinline__ float val(Raw r) {
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)r, false)[0];
  }
  static __device__ __forceinline__ void add(float *a, Raw r) { a[0] += val(r); }
  static __device__ __forceinline__ void fma(float *a, float w, Raw r) {
    a[0] = __builtin_fmaf(w, val(r), a[0]);
  }
};

// Stores chunk c (EL floats) of a float32 row.
template <int EL>
__device__ __forceinline__ void store_chunk(float *row, int c, const float *a) {
  if constexpr (EL == 1) {
    row[c] = a[0];
  } else if constexpr (EL == 4) {
    reinterpret_cast<float4 *>(row)[c] = make_float4(a[0], a[1], a[2], a[3]);
  } else {
    float4 *p = reinterpret_cast<float4 *>(row) + (EL / 4) * c;
#pragma unroll
    for (int q = 0; q < EL / 4; ++q)
      p[q] = make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
  }
}

// Adds row chunk v, weighted by w when PSW.
template <typename RC, bool PSW>
__device__ __forceinline__ void accumulate(float *acc, float w, typename RC::Raw v) {
  if constexpr (PSW)
    RC::fma(acc, w, v);
  else
    RC::add(acc, v);
}

// Generic path: pools bag [s, e) of `tab` for chunk c of a row of nvec chunks,
// each lane reading the indices (and weights) itself.
template <typename TT, int VW, bool PSW>
__device__ __forceinline__ void pool_chunk(const TT *__restrict__ tab,
                                           const int32_t *__restrict__ idx,
                                           const float *__restrict__ wt, int s, int e, int nvec,
                                           int c, float *acc) {
  using RC = RowChunk<TT, VW>;
  using Raw = typename RC::Raw;
  const Raw *col = reinterpret_cast<const Raw *>(tab) + c;
#pragma unroll
  for (int i = 0; i < RC::EL; ++i) acc[i] = 0.f;
  int l = s;
  for (; l + kUnroll <= e; l += kUnroll) {
    int r[kUnroll];
    float w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      r[u] = idx[l + u];
      w[u] = PSW ? wt[l + u] : 1.f;
    }
    Raw v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = col[(size_t)(uint32_t)r[u] * (size_t)nvec];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) accumulate<RC, PSW>(acc, w[u], v[u]);
  }
  const int rem = e - l;
  if (rem > 0) {
    int r[kUnroll - 1];
    float w[kUnroll - 1];
#pragma unroll
    for (int u = 0; u < kUnroll - 1; ++u) {
      r[u] = (u < rem) ? idx[l + u] : 0;
      w[u] = (PSW && u < rem) ? wt[l + u] : 1.f;
    }
    Raw v[kUnroll - 1];
#pragma unroll
    for (int u = 0; u < kUnroll - 1; ++u)
      v[u] = (u < rem) ? col[(size_t)(uint32_t)r[u] * (size_t)nvec] : RC::zero();
#pragma unroll
    for (int u = 0; u < kUnroll - 1; ++u)
      if (u < rem) accumulate<RC, PSW>(acc, w[u], v[u]);
  }
}

// Shuffle path (G lanes per group, G a power of two <= 64, nvec % G == 0):
// pools bag [s, e) for 16-byte chunk c.  Every lane of the group must call
// this together (the index and weight broadcasts read the other lanes); gbase
// is the wave lane of the group's first lane.
template <typename TT, int G, bool PSW>
__device__ __forceinline__ void pool_group(const TT *__restrict__ tab,
                                           const int32_t *__restrict__ idx,
                                           const float *__restrict__ wt, int s, int e, int nvec,
                                           int c_lane, int c, int gbase, float *acc) {
  using RC = RowChunk<TT, 4>;
  using Raw = typename RC::Raw;
  // (weighted bf16 rows over 4-lane groups keep 8 rows in flight: 12 would
  // not fit the registers beside the prefetched indices and weights)
  constexpr int R = (PSW && G == 4 && sizeof(TT) == 2) ? 8 : kRound<TT>;
  constexpr int T = (R + G - 1) / G;  // index registers per lane
  const Raw *col = reinterpret_cast<const Raw *>(tab) + c;
#pragma unroll
  for (int i = 0; i < RC::EL; ++i) acc[i] = 0.f;
  // Indices (and weights) of the round starting at l0: lane c_lane loads
  // positions c_lane, c_lane + G, ... of the round.
  int mine[T];
  float mine_w[T];
  auto load_round = [&](int l0) {
    const int n = min(R, e - l0);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int l = c_lane + G * t;
      mine[t] = (l < n) ? idx[l0 + l] : 0;
      mine_w[t] = (PSW && l < n) ? wt[l0 + l] : 0.f;
    }
  };
  if (s < e) load_round(s);
  for (int l0 = s; l0 < e; l0 += R) {
    const int n = min(R, e - l0);
    Raw v[R];
    float w[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int src = (gbase + (u % G)) << 2;
      const int r = __builtin_amdgcn_ds_bpermute(src, mine[u / G]);
      w[u] = PSW ? __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(mine_w[u / G])))
                 : 1.f;
      v[u] = (u < n) ? col[(size_t)(uint32_t)r * (size_t)nvec] : RC::zero();
    }
    // The next round's indices go out behind this round's rows, so their
    // latency overlaps the rows' instead of adding to it.
    if (l0 + R < e) load_round(l0 + R);
#pragma unroll
    for (int u = 0; u < R; ++u)
      if (u < n) accumulate<RC, PSW>(acc, w[u], v[u]);
  }
}

// Pools bag (b, k) into `row` (nvec chunks) and optionally `eo`, dividing by
// the bag size for mean pooling.  All G lanes of the group call it together.
template <typename TT, int VW, int GS, bool CSR, bool PSW>
__device__ __forceinline__ void pool_bag(const TableSet &ts, int k, int b, int B, int nvec,
                                         int G, int c0, float *row, float *eo) {
  constexpr int EL = RowChunk<TT, VW>::EL;
  int bs, be;
  bag_bounds<CSR>(ts, k, b, B, bs, be);
  const TT *tab = static_cast<const TT *>(ts.table[k]);
  const float *wt = PSW ? ts.wt[k] : nullptr;
  for (int c = c0; c < nvec; c += G) {
    float acc[EL];
    if constexpr (GS > 0) {
      const int gbase = (threadIdx.x & 63) & ~(GS - 1);
      pool_group<TT, GS, PSW>(tab, ts.idx[k], wt, bs, be, nvec, c0, c, gbase, acc);
    } else {
      pool_chunk<TT, VW, PSW>(tab, ts.idx[k], wt, bs, be, nvec, c, acc);
    }
    if (ts.mean && be > bs) {
      const float n = (float)(be - bs);
#pragma unroll
      for (int i = 0; i < EL; ++i) acc[i] = acc[i] / n;
    }
    if (ts.scaled) {
      const float sc = ts.scale[k];
#pragma unroll
      for (int i = 0; i < EL; ++i) acc[i] *= sc;
    }
    store_chunk<EL>(row, c, acc);
    if (eo) store_chunk<EL>(eo, c, acc);
  }
}

enum { MODE_FUSED = 0, MODE_LOAD = 1 };


// The dots of the S samples staged in X go to out0 + s * ld + p for the
// nvalid first samples (out0 may point to global memory or to LDS).

// One quad per dot, p -> (i, j) in closed form (any D; used by the scalar path).
template <int VW>
__device__ __forceinline__ void dots_per_pair(const float *X, const InteractParams &ip, int FR,
                                              float *out0, int64_t ld, int nvalid) {
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
    if (r == 0 && s < nvalid) out0[(int64_t)s * ld + p] = acc;
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
__device__ __forceinline__ void dots_blocked(const float *X, const InteractParams &ip, int FR,
                                             float *out0, int64_t ld, int nvalid) {
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
    if (tl < 4 && s < nvalid && i < F) {
      float *o = out0 + (int64_t)s * ld + i * (i - 1) / 2;
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int j = 4 * J + y;
        if (j < i) o[j] = z[y];
      }
    }
  }
}

// Shuffle-path group size for a row of nvec float4 chunks (0: generic path).
// Rows narrower than 4 chunks keep the generic path: with 1 or 2 lanes per
// group the index registers of a round would not fit beside the row loads.
inline int shuffle_group(int nvec) {
  if (nvec < 4) return 0;
  if (nvec <= 64 && (nvec & (nvec - 1)) == 0) return nvec;
  if (nvec % 64 == 0) return 64;
  return 0;
}


inline int lanes_per_row(int D, int el) {
  const int nvec = D / el;
  return nvec < kWave ? nvec : kWave;
}

// Elements per row chunk: 4 (float32) or 8 (bfloat16) on the vector path, 1
// on the scalar path.
inline int chunk_elems(int dtype, bool vec) {
  return vec ? (dtype == kFP8 ? 16 : dtype == kBF16 ? 8 : 4) : 1;
}

}  // namespace dlrm
