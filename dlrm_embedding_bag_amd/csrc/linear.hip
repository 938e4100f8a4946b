// linear.hip -- fused linear + bias + activation for gfx950:
//   C[m, n] = act(bias[n] + sum_k A[m, k] W[n, k])
// ([FASTPATHS] matmul2d.rs, Activation epilogue; the linear_bias_relu /
// linear_bias_sigmoid frontends), where [FASTPATHS] = page "luminal_python:
// vanilla-PyTorch DLRMv1 fast paths + batched FFI + input cache".
//
// The MLP layers are the one dense contraction of the path, so they run on
// the f32 matrix cores: v_mfma_f32_16x16x4f32 (16x16 output block, k = 4 per
// instruction, full f32 precision).  Both A and W are k-contiguous; each lane
// reads a float4 of 4 consecutive k and feeds its components to 4 successive
// MFMAs, which permutes the order of the k sum but not its terms.  W is fed
// as the matrix core's first operand, so a lane's 4 accumulators are 4
// consecutive output columns of one row: the epilogue adds a float4 of bias,
// applies the activation and stores a float4.
//
// Tiles: BM x BN per workgroup of GM x GN waves (128 x 128 on 2 x 4 waves,
// 128 x 64 on 4 x 2, 64 x 64 or 64 x 32 on 2 x 2), BK = 32 staged through
// two LDS buffers (row stride BK + 4 floats: the 16 rows a ds_read_b128
// touches start on different banks): k-slabs are loaded into registers two slabs
// ahead and stored to the other LDS buffer while the current one is
// multiplied, one barrier per slab.  Full slabs load without bounds tests
// (rows past the matrix are clamped and their outputs masked at the store);
// only the last, partial slab tests k.  Tiles are assigned to XCDs in
// contiguous m-major runs so the workgroups that share rows of A share an L2.
// The 64-row tiles, chosen when larger ones would leave CUs idle, run on two
// wave groups that split each slab's k and add their partial tiles through
// LDS in group order (measured at M = 256: 512 -> 256 10.5 -> 9.2 us).
//
// Layers with N <= 8 (the final 256 -> 1 head) are a matrix-vector product
// bound by reading A; they take a wave-per-4-rows kernel with DPP row sums
// (for N = 1 with aligned rows, with each row's loads issued together).
// Layers with K <= 16 (the 13 -> 512 first layer) are bound by writing C;
// they take a VALU kernel with the weights in registers (thin_k_kernel).
//
// Split A ([FASTPATHS] matmul2d.rs, a_split and the *_split_a frontends: the
// top MLP reads cat(dense, interactions) from two pointers without building
// the concat): columns [0, k_lo) of A come from one matrix and [k_lo, K) from
// another.  Both kernels take the A source as a struct; the unsplit
// instantiations never look at its second half.
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace dlrm {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 32;      // k per LDS slab
constexpr int kKSplit = 2;   // wave groups splitting k in the 64-row tiles

__device__ __forceinline__ float apply_act(float x, int act) {
  if (act == 1) return x > 0.0f ? x : 0.0f;
  if (act == 2) return 1.0f / (1.0f + expf(-x));
  return x;
}

// float4 of columns k..k+3 of row `row` (already clamped into the matrix) of
// a matrix with stride ld, for a slab known to lie inside K: no bounds tests.
// Where A's columns live: [0, k_lo) in lo (row stride ld_lo), [k_lo, K) in
// hi (row stride ld_hi) when split.
struct ASrc {
  const float *lo;
  int64_t ld_lo;
  const float *hi;
  int64_t ld_hi;
  int k_lo;
  // The reducing instantiations (NRED > 1) read A as the NRED partial sums
  // of the layer before, red_stride floats apart from lo on: A[m][k] =
  // red_act(red_bias[k] + ((P_0[m][k] + P_1[m][k]) + ...)), red_bias may be
  // null.
  int64_t red_stride = 0;
  const float *red_bias = nullptr;
  int red_act = 0;
};

// Four floats at a 4-byte-aligned address: global memory takes a 16-byte
// load at dword alignment, so rows of a K that is not a multiple of 4 (the
// 415-wide top layer) still load as one global_load_dwordx4 per lane.
typedef float float4_a4 __attribute__((ext_vector_type(4), aligned(4)));

template <bool VEC>
__device__ __forceinline__ float4 load_full(const float *__restrict__ base, int64_t ld, int row,
                                            int k) {
  const float *p = base + (int64_t)row * ld + k;
  if (VEC) return *reinterpret_cast<const float4 *>(p);
  const float4_a4 v = *reinterpret_cast<const float4_a4 *>(p);
  return make_float4(v.x, v.y, v.z, v.w);
}

// Same for the last, partial slab: columns at or past K read as zero.  The
// addresses are clamped so every load stays inside the row.
__device__ __forceinline__ float4 load_tail(const float *__restrict__ base, int64_t ld, int row,
                                            int k, int K) {
  const float *p = base + (int64_t)row * ld;
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int kk = k + e;
    const float x = p[kk < K ? kk : K - 1];
    v[e] = kk < K ? x : 0.0f;
  }
  return make_float4(v[0], v[1], v[2], v[3]);
}

// Column k (and k+1..k+3) of row `row` of A, inside K.  Split: with VEC the
// split point is a multiple of 4, so a float4 lies in one half; without, each
// element picks its half.
template <bool SPLIT, bool VEC>
__device__ __forceinline__ float4 load_a_full(const ASrc &a, int row, int k) {
  if constexpr (!SPLIT) {
    return load_full<VEC>(a.lo, a.ld_lo, row, k);
  } else if constexpr (VEC) {
    const bool lo = k < a.k_lo;
    return load_full<true>(lo ? a.lo : a.hi, lo ? a.ld_lo : a.ld_hi, row, lo ? k : k - a.k_lo);
  } else {
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kk = k + e;
      v[e] = kk < a.k_lo ? a.lo[(int64_t)row * a.ld_lo + kk]
                         : a.hi[(int64_t)row * a.ld_hi + (kk - a.k_lo)];
    }
    return make_float4(v[0], v[1], v[2], v[3]);
  }
}

// Branch-free activation (both forms computed, one selected): inside the k
// loop a branch would make the compiler's wait-count pass drain the
// outstanding prefetch loads where the paths join.
__device__ __forceinline__ float act_select(float x, int act) {
  const float r = (act == 1 && !(x > 0.0f)) ? 0.0f : x;
  const float sg = 1.0f / (1.0f + expf(-x));
  return act == 2 ? sg : r;
}

// Columns k..k+3 of row `row` of a reduced source, inside its K: the NRED
// partials' float4s (16-byte aligned) are all loaded before any is added,
// then added in partial order; the bias (one dword-aligned 16-byte load
// from a valid address whether or not there is a bias) and the activation
// follow.
// Split in two for callers that issue several of them before any add:
// red_raw loads, red_combine adds and activates.
template <int NRED>
__device__ __forceinline__ void red_raw(const ASrc &a, int row, int k, float4 (&t)[NRED],
                                        float4 &b) {
  const float *p = a.lo + (int64_t)row * a.ld_lo + k;
#pragma unroll
  for (int s = 0; s < NRED; ++s)
    t[s] = *reinterpret_cast<const float4 *>(p + (int64_t)s * a.red_stride);
  const float4_a4 bb = *reinterpret_cast<const float4_a4 *>(a.red_bias ? a.red_bias + k : p);
  b = make_float4(bb.x, bb.y, bb.z, bb.w);
}

template <int NRED>
__device__ __forceinline__ float4 red_combine(const ASrc &a, const float4 (&t)[NRED],
                                              const float4 &b) {
  float v[4] = {t[0].x, t[0].y, t[0].z, t[0].w};
#pragma unroll
  for (int s = 1; s < NRED; ++s) {
    v[0] += t[s].x;
    v[1] += t[s].y;
    v[2] += t[s].z;
    v[3] += t[s].w;
  }
  const bool hb = a.red_bias != nullptr;
  return make_float4(act_select(v[0] + (hb ? b.x : 0.0f), a.red_act),
                     act_select(v[1] + (hb ? b.y : 0.0f), a.red_act),
                     act_select(v[2] + (hb ? b.z : 0.0f), a.red_act),
                     act_select(v[3] + (hb ? b.w : 0.0f), a.red_act));
}

template <int NRED>
__device__ __forceinline__ float4 load_red_full(const ASrc &a, int row, int k) {
  float4 t[NRED], b;
  red_raw<NRED>(a, row, k, t, b);
  return red_combine<NRED>(a, t, b);
}

// The same for the last, partial slab: columns at or past K read as zero
// (clamped addresses, every load inside the row).
template <int NRED>
__device__ __forceinline__ float4 load_red_tail(const ASrc &a, int row, int k, int K) {
  const float *p = a.lo + (int64_t)row * a.ld_lo;
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int kk = min(k + e, K - 1);
    float t[NRED];
#pragma unroll
    for (int s = 0; s < NRED; ++s) t[s] = p[(int64_t)s * a.red_stride + kk];
    const float bl = *(a.red_bias ? a.red_bias + kk : p + kk);
    const float b = a.red_bias ? bl : 0.0f;
    float x = t[0];
#pragma unroll
    for (int s = 1; s < NRED; ++s) x += t[s];
    x = act_select(x + b, a.red_act);
    v[e] = k + e < K ? x : 0.0f;
  }
  return make_float4(v[0], v[1], v[2], v[3]);
}

template <bool SPLIT>
__device__ __forceinline__ float4 load_a_tail(const ASrc &a, int row, int k, int K) {
  if constexpr (!SPLIT) {
    return load_tail(a.lo, a.ld_lo, row, k, K);
  } else {
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kk = min(k + e, K - 1);
      const float x = kk < a.k_lo ? a.lo[(int64_t)row * a.ld_lo + kk]
                                  : a.hi[(int64_t)row * a.ld_hi + (kk - a.k_lo)];
      v[e] = k + e < K ? x : 0.0f;
    }
    return make_float4(v[0], v[1], v[2], v[3]);
  }
}

// A one-output layer applied to this layer's activations in the epilogue
// (the sigmoid head of the top MLP): out[m] = act(bias + sum_n h[m][n] w[n])
// with h = this layer's act(A W^T + bias) row, which is never stored.
struct HeadArgs {
  const float *w;     // (N,) weights of the head
  const float *bias;  // (1,) or nullptr
  int act;
  float *out;         // out[m * ldo]
  int64_t ldo;
};

// k split across workgroups: workgroup (tile, s) multiplies k in
// [s kc, s kc + kc) and stores its raw partial sums (the launcher passes no
// bias and no activation) to C + s c_stride.  kc = 0: one workgroup per tile.
struct KSplitArgs {
  int kc;
  int tiles;
  int64_t c_stride;
};

template <int BM, int BN, int GM, int GN, int KS, bool VA, bool VW, bool VC, bool SPLIT,
          bool HEAD = false, int NRED = 1>
__global__ __launch_bounds__(64 * GM * GN * KS) void gemm_kernel(int M, int N, int Kfull,
                                                                 const ASrc Afull,
                                                                 const float *__restrict__ Wfull,
                                                                 const float *__restrict__ bias,
                                                                 int act, float *__restrict__ Cs,
                                                                 int64_t ldc, int tiles_n,
                                                                 int xcd_chunk,
                                                                 const HeadArgs head,
                                                                 const KSplitArgs ks) {
  static_assert(NRED == 1 || (VA && !SPLIT && !HEAD), "a reduced A is aligned and unsplit");
  // KS wave groups split k: a staged slab holds KS x kBK columns and group g
  // multiplies columns [g kBK, (g + 1) kBK) of it; the groups' partial tiles
  // are added in group order through LDS at the end.
  constexpr int NT = 64 * GM * GN * KS;    // threads
  constexpr int SK = kBK * KS;             // k per staged slab
  constexpr int STR = SK + 4;              // LDS row stride: 4 mod 32 banks, so the 16 rows
                                           // a ds_read_b128 touches start on different banks
  constexpr int WM = BM / GM, WN = BN / GN;  // wave tile (GM x GN waves per group)
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int A_V4 = BM * SK / 4 / NT;   // float4 loads per thread per slab
  constexpr int W_V4 = BN * SK / 4 / NT;
  static_assert(A_V4 >= 1 && W_V4 >= 1 && TM >= 1 && TN >= 1, "tile too small");
  static_assert(A_V4 * NT * 4 == BM * SK && W_V4 * NT * 4 == BN * SK, "tile split");
  constexpr int A_ELEMS = BM * STR, W_ELEMS = BN * STR;
  static_assert(KS == 1 || (KS - 1) * GM * GN * TM * TN * 4 * 64 <= 2 * (A_ELEMS + W_ELEMS),
                "the partial tiles of groups 1.. must fit the slab buffers");

  // Two LDS buffers: slab s+1 is stored while slab s is multiplied.
  __shared__ float lds[2 * (A_ELEMS + W_ELEMS)];

  // XCD-aware tile order: workgroup ids are dealt to the 8 XCDs round robin;
  // give XCD x the contiguous m-major tile range [x*chunk, (x+1)*chunk).
  int bid = blockIdx.x;
  if (xcd_chunk > 0) bid = (bid & 7) * xcd_chunk + (bid >> 3);
  // With a k split, the workgroup's k range: A's columns and W's columns
  // from k0 on, K of them (every range holds at least one column).
  int K = Kfull;
  ASrc A = Afull;
  const float *W = Wfull;
  float *C = Cs;
  if (ks.kc > 0) {
    const int s = bid / ks.tiles;
    bid -= s * ks.tiles;
    const int k0 = s * ks.kc;
    K = min(ks.kc, Kfull - k0);
    A.lo += k0;
    if (A.red_bias) A.red_bias += k0;
    W += k0;
    C += s * ks.c_stride;
  }
  const int64_t ldw = Kfull;
  const int tm_blk = bid / tiles_n;
  const int tn_blk = bid - tm_blk * tiles_n;
  const int m0 = tm_blk * BM, n0 = tn_blk * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kg = wave / (GM * GN);       // k group
  const int wg = wave - kg * (GM * GN);  // wave within the group
  const int wm = wg / GN, wn = wg - (wg / GN) * GN;
  const int l16 = lane & 15, lq = lane >> 4;

  // Rows each thread stages; rows past the matrix are clamped to its last row
  // (their products land in outputs that are never stored).
  int arow[A_V4], wrow[W_V4], acol[A_V4], wcol[W_V4];
#pragma unroll
  for (int i = 0; i < A_V4; ++i) {
    const int v = tid + NT * i;
    arow[i] = min(m0 + v / (SK / 4), M - 1);
    acol[i] = 4 * (v % (SK / 4));
  }
#pragma unroll
  for (int i = 0; i < W_V4; ++i) {
    const int v = tid + NT * i;
    wrow[i] = min(n0 + v / (SK / 4), N - 1);
    wcol[i] = 4 * (v % (SK / 4));
  }

  floatx4 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nfull = K / SK;                    // slabs inside K
  const int nslab = (K + SK - 1) / SK;
  auto fetch = [&](int sl, float4 (&ra)[A_V4], float4 (&rw)[W_V4]) {
    const int kb = sl * SK;
    if (sl < nfull) {
#pragma unroll
      for (int i = 0; i < A_V4; ++i) {
        if constexpr (NRED > 1)
          ra[i] = load_red_full<NRED>(A, arow[i], kb + acol[i]);
        else
          ra[i] = load_a_full<SPLIT, VA>(A, arow[i], kb + acol[i]);
      }
#pragma unroll
      for (int i = 0; i < W_V4; ++i) rw[i] = load_full<VW>(W, ldw, wrow[i], kb + wcol[i]);
    } else {
#pragma unroll
      for (int i = 0; i < A_V4; ++i) {
        if constexpr (NRED > 1)
          ra[i] = load_red_tail<NRED>(A, arow[i], kb + acol[i], K);
        else
          ra[i] = load_a_tail<SPLIT>(A, arow[i], kb + acol[i], K);
      }
#pragma unroll
      for (int i = 0; i < W_V4; ++i) rw[i] = load_tail(W, ldw, wrow[i], kb + wcol[i], K);
    }
  };
  auto stash = [&](int buf, const float4 (&ra)[A_V4], const float4 (&rw)[W_V4]) {
    float *As = lds + buf * (A_ELEMS + W_ELEMS);
    float *Ws = As + A_ELEMS;
#pragma unroll
    for (int i = 0; i < A_V4; ++i) {
      const int v = tid + NT * i;
      *reinterpret_cast<float4 *>(&As[(v / (SK / 4)) * STR + acol[i]]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < W_V4; ++i) {
      const int v = tid + NT * i;
      *reinterpret_cast<float4 *>(&Ws[(v / (SK / 4)) * STR + wcol[i]]) = rw[i];
    }
  };
  // Fragments of one k-quad block (16 k) of the group's part of the slab.
  const int kgo = kg * kBK;
  auto frags = [&](const float *As, const float *Ws, int kq, float4 (&af)[TM],
                   float4 (&wf)[TN]) {
#pragma unroll
    for (int a = 0; a < TM; ++a)
      af[a] = *reinterpret_cast<const float4 *>(
          &As[(wm * WM + a * 16 + l16) * STR + kgo + kq + 4 * lq]);
#pragma unroll
    for (int b = 0; b < TN; ++b)
      wf[b] = *reinterpret_cast<const float4 *>(
          &Ws[(wn * WN + b * 16 + l16) * STR + kgo + kq + 4 * lq]);
  };
  // 4 MFMA steps over the 4 k of each lane's float4, component-major so
  // consecutive MFMAs never share an accumulator.
  auto mfmas = [&](const float4 (&af)[TM], const float4 (&wf)[TN]) {
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[b].x, af[a].x, acc[a][b], 0, 0, 0);
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[b].y, af[a].y, acc[a][b], 0, 0, 0);
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[b].z, af[a].z, acc[a][b], 0, 0, 0);
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[b].w, af[a].w, acc[a][b], 0, 0, 0);
  };
  // All MFMAs of the slab in LDS buffer `buf`; the next k-quad's fragments are
  // read while this one's MFMAs run.
  auto compute = [&](int buf) {
    const float *As = lds + buf * (A_ELEMS + W_ELEMS);
    const float *Ws = As + A_ELEMS;
    float4 af0[TM], wf0[TN], af1[TM], wf1[TN];
    frags(As, Ws, 0, af0, wf0);
#pragma unroll
    for (int kq = 0; kq < kBK; kq += 32) {
      frags(As, Ws, kq + 16, af1, wf1);
      mfmas(af0, wf0);
      if (kq + 32 < kBK) frags(As, Ws, kq + 32, af0, wf0);
      mfmas(af1, wf1);
    }
    // Scheduling hint: LLVM's instruction-group-level-parallelism strategy 1
    // interleaves the MFMAs with the LDS fragment reads of the next k-quad.
    // Same instructions, same results; measured per launch at 8192 x 512 x
    // 415: 41.1 -> 38.8 us, 8192 x 256 x 512: 25.7 -> 23.8, 16384 x 512 x
    // 512: 83.8 -> 79.9 (strategies 0 and 2 gained less).
    __builtin_amdgcn_iglp_opt(1);
  };

  // Slab s is loaded into register set s & 1 two slabs ahead of its use and
  // stored to LDS buffer s & 1 one slab ahead: each global load has two slabs
  // of MFMA work to arrive.
  float4 ra0[A_V4], rw0[W_V4], ra1[A_V4], rw1[W_V4];
  if constexpr (NRED > 1) {
    // The first slab of a reduced A: every partial and W load issued before
    // the first add (a scheduling barrier keeps the adds from being moved
    // between them), so the slab arrives in one memory round trip; nothing
    // else is in flight yet to hide more.
    if (nfull > 0) {
      float4 t[A_V4][NRED], b[A_V4];
#pragma unroll
      for (int i = 0; i < A_V4; ++i) red_raw<NRED>(A, arow[i], acol[i], t[i], b[i]);
#pragma unroll
      for (int i = 0; i < W_V4; ++i) rw0[i] = load_full<VW>(W, ldw, wrow[i], wcol[i]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < A_V4; ++i) ra0[i] = red_combine<NRED>(A, t[i], b[i]);
    } else {
      fetch(0, ra0, rw0);
    }
  } else {
    fetch(0, ra0, rw0);
  }
  stash(0, ra0, rw0);
  if (nslab > 1) fetch(1, ra1, rw1);
  __syncthreads();
  int sl = 0;
  // Steady state: both slabs fetched in an iteration are full, so every
  // fetch is issued unconditionally.  (With a conditional fetch the
  // compiler's wait-count pass merges the paths with and without the new
  // loads and makes each stash wait for the loads just issued, which turns
  // the two-slab prefetch into one.)
  for (; sl + 3 < nfull; sl += 2) {
    fetch(sl + 2, ra0, rw0);
    compute(0);
    stash(1, ra1, rw1);
    __syncthreads();
    fetch(sl + 3, ra1, rw1);
    compute(1);
    stash(0, ra0, rw0);
    __syncthreads();
  }
  // The last slabs (fewer than two full ones ahead, or a partial one).
  for (; sl < nslab; sl += 2) {
    // even slab: buffer 0; register set 0 is free
    if (sl + 2 < nslab) fetch(sl + 2, ra0, rw0);
    compute(0);
    if (sl + 1 < nslab) stash(1, ra1, rw1);
    __syncthreads();
    if (sl + 1 >= nslab) break;
    // odd slab: buffer 1; register set 1 is free
    if (sl + 3 < nslab) fetch(sl + 3, ra1, rw1);
    compute(1);
    if (sl + 2 < nslab) stash(0, ra0, rw0);
    __syncthreads();
  }

  if constexpr (KS > 1) {
    // Groups 1.. park their partial tiles in the (now idle) slab buffers;
    // group 0 adds them in group order and stores.  The loop ended on a
    // barrier, so every wave is done reading the buffers.
    constexpr int PER = TM * TN * 4;  // floats per lane of one wave's tile
    if (kg > 0) {
      float *red = lds + ((size_t)((kg - 1) * GM * GN + wg) * PER) * 64 + lane;
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
          for (int v = 0; v < 4; ++v) red[((a * TN + b) * 4 + v) * 64] = acc[a][b][v];
    }
    __syncthreads();
    if (kg > 0 && !HEAD) return;  // (with a head every wave meets its barrier)
    if (kg == 0) {
#pragma unroll
      for (int g = 1; g < KS; ++g) {
        const float *red = lds + ((size_t)((g - 1) * GM * GN + wg) * PER) * 64 + lane;
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[a][b][v] += red[((a * TN + b) * 4 + v) * 64];
      }
    }
  }

  if constexpr (HEAD) {
    // The tile owns whole rows (BN >= N): each wave of group 0 folds its
    // columns into one partial dot per row, act(acc + bias[n]) * w[n] summed
    // over its columns in (b, v) order; the 4 lanes of a row (lq) are then
    // added by two butterfly steps, and the waves' partials in wave order
    // through LDS.  The order is fixed, so the result is deterministic.
    __shared__ float head_part[GM * GN * BM];
    if (kg == 0) {
      float part[TM];
#pragma unroll
      for (int a = 0; a < TM; ++a) part[a] = 0.0f;
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const int n = n0 + wn * WN + b * 16 + 4 * lq;
        float bv[4], hw[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const bool in = n + v < N;
          bv[v] = (bias && in) ? bias[n + v] : 0.0f;
          hw[v] = in ? head.w[n + v] : 0.0f;
        }
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (n + v < N) part[a] = __builtin_fmaf(apply_act(acc[a][b][v] + bv[v], act), hw[v],
                                                    part[a]);
      }
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        part[a] += __shfl_xor(part[a], 16);
        part[a] += __shfl_xor(part[a], 32);
      }
      if (lq == 0) {
#pragma unroll
        for (int a = 0; a < TM; ++a) head_part[wn * GM * BM + wm * WM + a * 16 + l16] = part[a];
      }
    }
    __syncthreads();
    if (tid < BM) {
      const int m = m0 + tid;
      if (m < M) {
        float t = 0.0f;
#pragma unroll
        for (int w = 0; w < GN; ++w) t += head_part[w * GM * BM + tid];
        if (head.bias) t += head.bias[0];
        head.out[(int64_t)m * head.ldo] = apply_act(t, head.act);
      }
    }
    return;
  }

  // Epilogue: lane holds C[m][n .. n+3] for m = .. + l16, n = .. + 4*lq.
#pragma unroll
  for (int b = 0; b < TN; ++b) {
    const int n = n0 + wn * WN + b * 16 + 4 * lq;
    float bv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) bv[v] = (bias && n + v < N) ? bias[n + v] : 0.0f;
#pragma unroll
    for (int a = 0; a < TM; ++a) {
      const int m = m0 + wm * WM + a * 16 + l16;
      if (m >= M) continue;
      float o[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) o[v] = apply_act(acc[a][b][v] + bv[v], act);
      float *cp = C + (int64_t)m * ldc + n;
      if (VC && n + 3 < N) {
        *reinterpret_cast<float4 *>(cp) = make_float4(o[0], o[1], o[2], o[3]);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (n + v < N) cp[v] = o[v];
      }
    }
  }
}

// N <= 8: each wave computes 4 rows at a time, 16 lanes per row.  With
// NRED > 1, A is reduced from the partial sums of the layer before (vector
// path only).
template <bool VEC, bool SPLIT, int NRED = 1>
__global__ __launch_bounds__(256) void gemv_kernel(int M, int N, int K, const ASrc A,
                                                   const float *__restrict__ W,
                                                   const float *__restrict__ bias, int act,
                                                   float *__restrict__ C, int64_t ldc) {
  static_assert(NRED == 1 || (VEC && !SPLIT), "a reduced A is aligned and unsplit");
  const int lane = threadIdx.x & 63;
  const int row_in_wave = lane >> 4;
  const int c = lane & 15;
  const int m = (blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * 4 + row_in_wave;
  // All 16 lanes of a row stay active through the DPP sums, so rows past M
  // compute on row M-1 and skip the store.
  const int mr = m < M ? m : M - 1;
  const float *a = A.lo + (int64_t)mr * A.ld_lo;
  const float *ah = SPLIT ? A.hi + (int64_t)mr * A.ld_hi - A.k_lo : nullptr;  // column k at ah[k]
  for (int n = 0; n < N; ++n) {
    const float *w = W + (int64_t)n * K;
    float acc = 0.0f;
    if (NRED > 1) {
      for (int k = 4 * c; k < K; k += 64)
        acc = vdot_acc(load_red_full<NRED>(A, mr, k), *reinterpret_cast<const float4 *>(w + k),
                       acc);
    } else if (VEC) {
      for (int k = 4 * c; k < K; k += 64) {
        const float *src = (SPLIT && k >= A.k_lo) ? ah : a;
        const float4 x = *reinterpret_cast<const float4 *>(src + k);
        const float4 y = *reinterpret_cast<const float4 *>(w + k);
        acc = vdot_acc(x, y, acc);
      }
    } else {
      for (int k = c; k < K; k += 16)
        acc = __builtin_fmaf((SPLIT && k >= A.k_lo) ? ah[k] : a[k], w[k], acc);
    }
    acc = row16_sum(acc);
    if (c == 0 && m < M) {
      const float bv = bias ? bias[n] : 0.0f;
      C[(int64_t)m * ldc + n] = apply_act(acc + bv, act);
    }
  }
}

// N == 1 (the sigmoid head) with 16-byte aligned A and W and K % 4 == 0:
// RW rows per wave, 64 / RW lanes per row, lane c taking columns
// 4c + 256 j / RW (chunks j < NCH) in j order, then a DPP sum over the row's
// lanes (a reduced A adds its partials in order, then the bias and the
// activation, as gemv_kernel).  Every load of the lane (all partials of all
// its chunks, the bias and W) is issued before any arithmetic, which a
// scheduling barrier keeps from being interleaved with it: one memory round
// trip per row rather than one per chunk.  Chunks past K load a clamped
// column and add nothing.
template <int NRED, int NCH, int RW>
__global__ __launch_bounds__(256) void head_row_kernel(int M, int K, const ASrc A,
                                                       const float *__restrict__ W,
                                                       const float *__restrict__ bias, int act,
                                                       float *__restrict__ C, int64_t ldc) {
  static_assert(RW == 1 || RW == 4, "one or four rows per wave");
  constexpr int LPR = 64 / RW;  // lanes per row
  constexpr int CW = 4 * LPR;   // columns per chunk
  const int lane = threadIdx.x & 63;
  const int c = lane % LPR;
  const int m = (blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * RW + lane / LPR;
  // All lanes of a row stay active through the DPP sums, so rows past M
  // compute on row M-1 and skip the store.
  const int mr = m < M ? m : M - 1;
  const float *row = A.lo + (int64_t)mr * A.ld_lo;
  float4 t[NCH][NRED], rb[NCH], w[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int k = min(4 * c + CW * j, K - 4);
#pragma unroll
    for (int s = 0; s < NRED; ++s)
      t[j][s] = *reinterpret_cast<const float4 *>(row + (int64_t)s * A.red_stride + k);
    if constexpr (NRED > 1) {
      // (a dword-aligned load from a valid address whether or not there is
      // a bias)
      const float4_a4 b = *reinterpret_cast<const float4_a4 *>(A.red_bias ? A.red_bias + k
                                                                           : row + k);
      rb[j] = make_float4(b.x, b.y, b.z, b.w);
    }
    w[j] = *reinterpret_cast<const float4 *>(W + k);
  }
  __builtin_amdgcn_sched_barrier(0);
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    float4 x = t[j][0];
    if constexpr (NRED > 1) {
#pragma unroll
      for (int s = 1; s < NRED; ++s) {
        x.x += t[j][s].x;
        x.y += t[j][s].y;
        x.z += t[j][s].z;
        x.w += t[j][s].w;
      }
      const bool hb = A.red_bias != nullptr;
      x = make_float4(act_select(x.x + (hb ? rb[j].x : 0.0f), A.red_act),
                      act_select(x.y + (hb ? rb[j].y : 0.0f), A.red_act),
                      act_select(x.z + (hb ? rb[j].z : 0.0f), A.red_act),
                      act_select(x.w + (hb ? rb[j].w : 0.0f), A.red_act));
    }
    const float d = vdot_acc(x, w[j], acc);
    acc = 4 * c + CW * j < K ? d : acc;
  }
  acc = row16_sum(acc);
  if constexpr (LPR == 64) {
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
  }
  if (c == 0 && m < M) C[(int64_t)m * ldc] = apply_act(acc + (bias ? bias[0] : 0.0f), act);
}

// Up to kHeadWaveRowMaxM rows, a wave per row (more workgroups, each with
// fewer bytes to fetch); above, four rows per wave.
constexpr int kHeadWaveRowMaxM = 4096;

// Launches head_row_kernel for K up to 1,024 (a wave per row) or 512 (four
// rows per wave) while a lane's loads fit in registers (NRED x chunks at
// most 32); false otherwise (the caller then takes gemv_kernel).
template <int NRED>
bool launch_head_row(int M, int K, const ASrc &A, const float *W, const float *bias, int act,
                     float *C, int64_t ldc, hipStream_t stream) {
#define DLRM_HEAD_ROW(NCH_, RW_)                                                             \
  launch_kernel((head_row_kernel<NRED, NCH_, RW_>), dim3((unsigned)((M + 4 * RW_ - 1) /       \
                                                                    (4 * RW_))),             \
                dim3(256), 0, stream, M, K, A, W, bias, act, C, ldc)
  if (M <= kHeadWaveRowMaxM) {
    if (K <= 256) {
      DLRM_HEAD_ROW(1, 1);
    } else if (K <= 512) {
      DLRM_HEAD_ROW(2, 1);
    } else {
      if constexpr (NRED > 4) return false;
      if (K > 1024) return false;
      DLRM_HEAD_ROW(4, 1);
    }
  } else {
    if (K <= 64) {
      DLRM_HEAD_ROW(1, 4);
    } else if (K <= 128) {
      DLRM_HEAD_ROW(2, 4);
    } else if (K <= 256) {
      DLRM_HEAD_ROW(4, 4);
    } else {
      if constexpr (NRED > 4) return false;
      if (K > 512) return false;
      DLRM_HEAD_ROW(8, 4);
    }
  }
#undef DLRM_HEAD_ROW
  return true;
}

// K <= 16 (the 13 -> 512 first bottom layer): the layer is bound by writing
// C, M N floats against (M + N) K read, and a matrix-core tile would spend
// its time on one partial k-slab.  Measured on MI355X at 8192 x 512 x 13:
// 9.7 us against 11.4 us for the 128 x 128 MFMA tile.  Each wave owns 256
// consecutive output columns (4 per lane) of RB consecutive rows: the lane's
// 4 x K weights and bias stay in registers, the RB rows of A are wave-uniform
// (scalar loads, all issued before the arithmetic), and each row costs a lane
// 4 K FMAs and one float4 store.  The k sum runs in order, then the bias is
// added.
constexpr int kThinMaxK = 16;
// Rows per wave: 8 rows of 13 k would spill the scalar registers, and so
// would 4 with a split A (each k then picks its source row at run time).
template <int K, bool SPLIT>
constexpr int thin_rows() {
  return SPLIT ? (K > 13 ? 1 : 2) : 4;
}
template <int K, bool SPLIT, int NB>
__global__ __launch_bounds__(256) void thin_k_kernel(int M, int N, const ASrc A,
                                                     const float *__restrict__ W,
                                                     const float *__restrict__ bias, int act,
                                                     float *__restrict__ C, int64_t ldc,
                                                     int col_groups, int xcd_run) {
  // A wave computes NB batches of RB rows with the same weights in registers
  // (a compile-time count, so the next batch's row loads can be issued
  // early).
  constexpr int RB = thin_rows<K, SPLIT>();
  // XCD-aware order: workgroup i runs on XCD i % 8 and takes the i / 8-th of
  // that XCD's contiguous run of workgroups, so each XCD writes a contiguous
  // band of rows, the band the next layer's m-major tiles on that XCD read.
  const int wg = (int)(blockIdx.x & 7) * xcd_run + (int)(blockIdx.x >> 3);
  const int wave = __builtin_amdgcn_readfirstlane(wg * (int)(blockDim.x >> 6) +
                                                  (int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int cg = wave % col_groups;
  const int mw = (wave / col_groups) * RB * NB;
  if (mw >= M) return;
  const int n = cg * 256 + 4 * lane;
  const bool live = n < N;  // N % 4 == 0: a live lane owns 4 real columns
  float w[4][K];
  float bv[4];
  const int nl = live ? n : 0;  // dead lanes read column 0 and store nothing
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int k = 0; k < K; ++k) w[j][k] = W[(int64_t)(nl + j) * K + k];
    bv[j] = bias ? bias[nl + j] : 0.0f;
  }
#pragma unroll
  for (int bt = 0; bt < NB; ++bt) {
    const int m0 = mw + bt * RB;
    if (m0 >= M) break;
    const int rows = min(RB, M - m0);
    float av[RB][K];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int64_t m = m0 + min(r, rows - 1);  // rows past M repeat the last one
#pragma unroll
      for (int k = 0; k < K; ++k)
        av[r][k] = (SPLIT && k >= A.k_lo) ? A.hi[m * A.ld_hi + (k - A.k_lo)]
                                          : A.lo[m * A.ld_lo + k];
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      if (r >= rows) break;
      float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < K; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_fmaf(av[r][k], w[j][k], acc[j]);
      if (live) {
        float4 o;
        o.x = apply_act(acc[0] + bv[0], act);
        o.y = apply_act(acc[1] + bv[1], act);
        o.z = apply_act(acc[2] + bv[2], act);
        o.w = apply_act(acc[3] + bv[3], act);
        *reinterpret_cast<float4 *>(C + (int64_t)(m0 + r) * ldc + n) = o;
      }
    }
  }
}

template <int BM, int BN, int GM, int GN, bool SPLIT, int KS = 1>
hipError_t launch_gemm_cfg(int M, int N, int K, const ASrc &A, int nred, const float *W,
                           const float *bias, int act, float *C, int64_t ldc, bool va, bool vw,
                           bool vc, int kc, int64_t c_stride, hipStream_t stream) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  const int64_t splits = kc > 0 ? (K + kc - 1) / kc : 1;
  const int64_t wgs = tiles * splits;
  const int xcd_chunk = (wgs % 8 == 0) ? (int)(wgs / 8) : 0;
  const KSplitArgs ks{kc, (int)tiles, c_stride};
  dim3 grid((unsigned)wgs), block(64 * GM * GN * KS);
#define DLRM_GEMM_LAUNCH(A_, W_, C_, R_)                                                    \
  launch_kernel((gemm_kernel<BM, BN, GM, GN, KS, A_, W_, C_, SPLIT, false, R_>), grid, block, \
                0, stream, M, N, K, A, W, bias, act, C, ldc, tiles_n, xcd_chunk, HeadArgs{}, ks)
  if (nred > 1) {
    // reduced sources exist for aligned A and W, and for the tiles a K of at
    // least 128 selects (the launcher checked both)
    if constexpr (!SPLIT && (KS > 1 || BM == 128)) {
      if (vc) {
        if (nred == 2) DLRM_GEMM_LAUNCH(true, true, true, 2);
        else if (nred == 4) DLRM_GEMM_LAUNCH(true, true, true, 4);
        else DLRM_GEMM_LAUNCH(true, true, true, 8);
      } else {
        if (nred == 2) DLRM_GEMM_LAUNCH(true, true, false, 2);
        else if (nred == 4) DLRM_GEMM_LAUNCH(true, true, false, 4);
        else DLRM_GEMM_LAUNCH(true, true, false, 8);
      }
    }
  } else if (va && vw && vc)
    DLRM_GEMM_LAUNCH(true, true, true, 1);
  else if (va && !vw && vc)
    DLRM_GEMM_LAUNCH(true, false, true, 1);
  else if (!va && vw && vc)
    DLRM_GEMM_LAUNCH(false, true, true, 1);
  else if (!va && !vw && vc)
    DLRM_GEMM_LAUNCH(false, false, true, 1);
  else if (va && vw)
    DLRM_GEMM_LAUNCH(true, true, false, 1);
  else
    DLRM_GEMM_LAUNCH(false, false, false, 1);
#undef DLRM_GEMM_LAUNCH
  return hipGetLastError();
}

// The tile launch_linear takes for an M x N x K layer (N > 8, K > 16): the
// largest tile that still gives every CU a workgroup.  128 x 128 tiles on 8
// waves (two per SIMD) when there are enough of them for every CU, else
// 128 x 64 on 8 waves of 32 x 32, else 64 x 64, else 64 x 32 on 4 waves.
// (At 8192 x 256 x 512, 128 x 64 on 8 waves: 24.5 us, 64 x 64 on 4 waves:
// 26.6 us, the same sums bit for bit.)  The 64-row tiles leave one wave per
// SIMD: with K of at least two staged slabs, kKSplit wave groups split each
// tile's k (kKSplit times the waves, 1/kKSplit of the MFMA chain and of the
// slab round trips).
enum class GemmCfg { T128x128, T128x64, T64x64, T64x64KS, T64x32, T64x32KS };

// Across-workgroup k splits: at most kMaxSplit partials, enough to give about
// kSplitFill workgroups (one per CU).
constexpr int kMaxSplit = 8;
constexpr int kSplitFill = 256;

// k columns per partial when K is cut into s partials of whole slabs of sk.
int split_width(int K, int s, int sk) {
  const int per = (K + s - 1) / s;
  return (per + sk - 1) / sk * sk;
}

int64_t gemm_tiles(int M, int N, int bm, int bn) {
  return (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn);
}

GemmCfg gemm_cfg(int M, int N, int K) {
  if (gemm_tiles(M, N, 128, 128) >= 256) return GemmCfg::T128x128;
  if (gemm_tiles(M, N, 128, 64) >= 256) return GemmCfg::T128x64;
  const bool ksplit = kKSplit > 1 && K >= 2 * kBK * kKSplit;
  if (gemm_tiles(M, N, 64, 64) >= 256) return ksplit ? GemmCfg::T64x64KS : GemmCfg::T64x64;
  return ksplit ? GemmCfg::T64x32KS : GemmCfg::T64x32;
}

int64_t cfg_tiles(GemmCfg c, int M, int N) {
  switch (c) {
    case GemmCfg::T128x128: return gemm_tiles(M, N, 128, 128);
    case GemmCfg::T128x64: return gemm_tiles(M, N, 128, 64);
    case GemmCfg::T64x64:
    case GemmCfg::T64x64KS: return gemm_tiles(M, N, 64, 64);
    default: return gemm_tiles(M, N, 64, 32);
  }
}

// k per staged slab of the tile: the unit a k split is cut in.
int cfg_slab_k(GemmCfg c) {
  return (c == GemmCfg::T64x64KS || c == GemmCfg::T64x32KS) ? kBK * kKSplit : kBK;
}

hipError_t launch_gemm(GemmCfg cfg, int M, int N, int K, const ASrc &A, int nred,
                       const float *W, const float *bias, int act, float *C, int64_t ldc,
                       bool va, bool vw, bool vc, int kc, int64_t c_stride,
                       hipStream_t stream) {
  constexpr int KS = kKSplit;
  switch (cfg) {
    case GemmCfg::T128x128:
      return launch_gemm_cfg<128, 128, 2, 4, false>(M, N, K, A, nred, W, bias, act, C, ldc, va,
                                                    vw, vc, kc, c_stride, stream);
    case GemmCfg::T128x64:
      return launch_gemm_cfg<128, 64, 4, 2, false>(M, N, K, A, nred, W, bias, act, C, ldc, va,
                                                   vw, vc, kc, c_stride, stream);
    case GemmCfg::T64x64KS:
      return launch_gemm_cfg<64, 64, 2, 2, false, KS>(M, N, K, A, nred, W, bias, act, C, ldc,
                                                      va, vw, vc, kc, c_stride, stream);
    case GemmCfg::T64x64:
      return launch_gemm_cfg<64, 64, 2, 2, false>(M, N, K, A, nred, W, bias, act, C, ldc, va,
                                                  vw, vc, kc, c_stride, stream);
    case GemmCfg::T64x32KS:
      return launch_gemm_cfg<64, 32, 2, 2, false, KS>(M, N, K, A, nred, W, bias, act, C, ldc,
                                                      va, vw, vc, kc, c_stride, stream);
    default:
      return launch_gemm_cfg<64, 32, 2, 2, false>(M, N, K, A, nred, W, bias, act, C, ldc, va,
                                                  vw, vc, kc, c_stride, stream);
  }
}

template <bool SPLIT>
hipError_t launch_linear_src(int M, int N, int K, const ASrc &A, bool va, const float *W,
                             const float *bias, int act, float *C, int64_t ldc,
                             hipStream_t stream) {
  const bool vw = aligned16(W) && K % 4 == 0;
  const bool vc = aligned16(C) && ldc % 4 == 0;
  if (!SPLIT && N == 1 && va && vw && K >= 4 &&
      launch_head_row<1>(M, K, A, W, bias, act, C, ldc, stream))
    return hipGetLastError();
  if (N <= 8) {
    const int rows_per_block = 16;
    dim3 grid((unsigned)((M + rows_per_block - 1) / rows_per_block)), block(256);
    if (va && vw && K % 4 == 0)
      launch_kernel((gemv_kernel<true, SPLIT>), grid, block, 0, stream, M, N, K, A, W, bias,
                    act, C, ldc);
    else
      launch_kernel((gemv_kernel<false, SPLIT>), grid, block, 0, stream, M, N, K, A, W,
                    bias, act, C, ldc);
    return hipGetLastError();
  }
  const int col_groups = (N + 255) / 256;
  // (wave ids are int: at most M x col_groups waves, each a multiple of 8
  // workgroups of 4)
  if (K >= 1 && K <= kThinMaxK && N % 4 == 0 && vc && (int64_t)M * col_groups < (1LL << 30)) {
    auto run = [&](auto kc) -> hipError_t {
      constexpr int KK = decltype(kc)::value;
      constexpr int rb = thin_rows<KK, SPLIT>();
      // Two row batches per wave halve the weight loads but also the waves:
      // taken while 2048 waves remain (measured at 13 -> 512: M = 8192
      // 10.0 -> 9.3 us, M = 16384 15.3 -> 12.7; at M = 2048 5.4 -> 6.3, so
      // one batch there; four batches were slower everywhere).
      const int64_t waves2 = (int64_t)((M + 2 * rb - 1) / (2 * rb)) * col_groups;
      const int batches = waves2 >= 2048 ? 2 : 1;
      const int64_t waves = (int64_t)((M + batches * rb - 1) / (batches * rb)) * col_groups;
      const int64_t xcd_run = ((waves + 3) / 4 + 7) / 8;  // workgroups per XCD
      if (batches == 2)
        launch_kernel((thin_k_kernel<KK, SPLIT, 2>), dim3((unsigned)(xcd_run * 8)), dim3(256), 0,
                      stream, M, N, A, W, bias, act, C, ldc, col_groups, (int)xcd_run);
      else
        launch_kernel((thin_k_kernel<KK, SPLIT, 1>), dim3((unsigned)(xcd_run * 8)), dim3(256), 0,
                      stream, M, N, A, W, bias, act, C, ldc, col_groups, (int)xcd_run);
      return hipGetLastError();
    };
    switch (K) {
      case 1: return run(std::integral_constant<int, 1>{});
      case 2: return run(std::integral_constant<int, 2>{});
      case 3: return run(std::integral_constant<int, 3>{});
      case 4: return run(std::integral_constant<int, 4>{});
      case 5: return run(std::integral_constant<int, 5>{});
      case 6: return run(std::integral_constant<int, 6>{});
      case 7: return run(std::integral_constant<int, 7>{});
      case 8: return run(std::integral_constant<int, 8>{});
      case 9: return run(std::integral_constant<int, 9>{});
      case 10: return run(std::integral_constant<int, 10>{});
      case 11: return run(std::integral_constant<int, 11>{});
      case 12: return run(std::integral_constant<int, 12>{});
      case 13: return run(std::integral_constant<int, 13>{});
      case 14: return run(std::integral_constant<int, 14>{});
      case 15: return run(std::integral_constant<int, 15>{});
      case 16: return run(std::integral_constant<int, 16>{});
      default: break;
    }
  }
  if constexpr (SPLIT) {
    // the two-part A source keeps the tile rules of the plain one
    const GemmCfg cfg = gemm_cfg(M, N, K);
    constexpr int KS = kKSplit;
    switch (cfg) {
      case GemmCfg::T128x128:
        return launch_gemm_cfg<128, 128, 2, 4, true>(M, N, K, A, 1, W, bias, act, C, ldc, va,
                                                     vw, vc, 0, 0, stream);
      case GemmCfg::T128x64:
        return launch_gemm_cfg<128, 64, 4, 2, true>(M, N, K, A, 1, W, bias, act, C, ldc, va, vw,
                                                    vc, 0, 0, stream);
      case GemmCfg::T64x64KS:
        return launch_gemm_cfg<64, 64, 2, 2, true, KS>(M, N, K, A, 1, W, bias, act, C, ldc, va,
                                                       vw, vc, 0, 0, stream);
      case GemmCfg::T64x64:
        return launch_gemm_cfg<64, 64, 2, 2, true>(M, N, K, A, 1, W, bias, act, C, ldc, va, vw,
                                                   vc, 0, 0, stream);
      case GemmCfg::T64x32KS:
        return launch_gemm_cfg<64, 32, 2, 2, true, KS>(M, N, K, A, 1, W, bias, act, C, ldc, va,
                                                       vw, vc, 0, 0, stream);
      default:
        return launch_gemm_cfg<64, 32, 2, 2, true>(M, N, K, A, 1, W, bias, act, C, ldc, va, vw,
                                                   vc, 0, 0, stream);
    }
  } else {
    return launch_gemm(gemm_cfg(M, N, K), M, N, K, A, 1, W, bias, act, C, ldc, va, vw, vc, 0, 0,
                       stream);
  }
}

}  // namespace

hipError_t launch_linear(int M, int N, int K, const float *A, int64_t lda, const float *W,
                         const float *bias, int act, float *C, int64_t ldc, hipStream_t stream) {
  const ASrc src{A, lda, nullptr, 0, K};
  const bool va = aligned16(A) && lda % 4 == 0;
  return launch_linear_src<false>(M, N, K, src, va, W, bias, act, C, ldc, stream);
}

// The fewest k partials (a power of two, at most kMaxSplit) that give the
// layer's tiles about one workgroup per CU, each partial a whole number of
// staged slabs and none empty; 1 when the tiles already fill the chip or the
// layer does not take a GEMM tile.
int linear_split_count(int M, int N, int K) {
  if (M < 1 || N <= 8 || K <= kThinMaxK) return 1;
  const GemmCfg cfg = gemm_cfg(M, N, K);
  const int64_t tiles = cfg_tiles(cfg, M, N);
  const int sk = cfg_slab_k(cfg);
  int s = 1;
  while (s < kMaxSplit && tiles * s < kSplitFill) s *= 2;
  while (s > 1) {
    const int kc = split_width(K, s, sk);
    if ((K + kc - 1) / kc == s) break;
    s /= 2;
  }
  return s;
}

bool linear_reduce_supported(int M, int N, int K, const float *W, int nred) {
  if (nred != 2 && nred != 4 && nred != 8) return false;
  if (!aligned16(W) || K % 4 != 0) return false;
  if (N <= 8) return true;  // the vector matrix-vector kernel
  if (K < 2 * kBK * kKSplit) return false;  // tiles with reduced-source instantiations
  // (64 x 64 tiles reading 8 partials would spill registers)
  return !(nred == 8 && gemm_cfg(M, N, K) == GemmCfg::T64x64KS);
}

hipError_t launch_linear_call(const LinearCall &c, hipStream_t stream) {
  const int M = c.M, N = c.N, K = c.K;
  if (c.a_nred <= 1 && c.nsplit <= 1)
    return launch_linear(M, N, K, c.A, c.lda, c.W, c.bias, c.act, c.C, c.ldc, stream);
  ASrc src{c.A, c.lda, nullptr, 0, K};
  const bool red = c.a_nred > 1;
  if (red) {
    if (!linear_reduce_supported(M, N, K, c.W, c.a_nred) || !aligned16(c.A) || c.lda % 4 != 0 ||
        c.a_stride % 4 != 0)
      return hipErrorInvalidValue;
    src.red_stride = c.a_stride;
    src.red_bias = c.a_bias;
    src.red_act = c.a_act;
  }
  const bool va = aligned16(c.A) && c.lda % 4 == 0;
  const bool vw = aligned16(c.W) && K % 4 == 0;
  const bool vc = aligned16(c.C) && c.ldc % 4 == 0;
  if (N <= 8) {
    if (c.nsplit > 1) return hipErrorInvalidValue;
    if (N == 1 && K >= 4) {
      bool ok = false;
      if (c.a_nred == 2)
        ok = launch_head_row<2>(M, K, src, c.W, c.bias, c.act, c.C, c.ldc, stream);
      else if (c.a_nred == 4)
        ok = launch_head_row<4>(M, K, src, c.W, c.bias, c.act, c.C, c.ldc, stream);
      else
        ok = launch_head_row<8>(M, K, src, c.W, c.bias, c.act, c.C, c.ldc, stream);
      if (ok) return hipGetLastError();
    }
    const int rows_per_block = 16;
    dim3 grid((unsigned)((M + rows_per_block - 1) / rows_per_block)), block(256);
    if (c.a_nred == 2)
      launch_kernel((gemv_kernel<true, false, 2>), grid, block, 0, stream, M, N, K, src, c.W,
                    c.bias, c.act, c.C, c.ldc);
    else if (c.a_nred == 4)
      launch_kernel((gemv_kernel<true, false, 4>), grid, block, 0, stream, M, N, K, src, c.W,
                    c.bias, c.act, c.C, c.ldc);
    else
      launch_kernel((gemv_kernel<true, false, 8>), grid, block, 0, stream, M, N, K, src, c.W,
                    c.bias, c.act, c.C, c.ldc);
    return hipGetLastError();
  }
  if (K <= kThinMaxK) return hipErrorInvalidValue;
  const GemmCfg cfg = gemm_cfg(M, N, K);
  int kc = 0;
  if (c.nsplit > 1) {
    kc = split_width(K, c.nsplit, cfg_slab_k(cfg));
    if ((K + kc - 1) / kc != c.nsplit || !vc) return hipErrorInvalidValue;
  }
  return launch_gemm(cfg, M, N, K, src, red ? c.a_nred : 1, c.W, c.nsplit > 1 ? nullptr : c.bias,
                     c.nsplit > 1 ? 0 : c.act, c.C, c.ldc, va, vw, vc, kc,
                     c.nsplit > 1 ? c.c_stride : 0, stream);
}

hipError_t launch_linear_split(int M, int N, int K_lo, const float *A_lo, int64_t lda_lo,
                               int K_hi, const float *A_hi, int64_t lda_hi, const float *W,
                               const float *bias, int act, float *C, int64_t ldc,
                               hipStream_t stream) {
  const ASrc src{A_lo, lda_lo, A_hi, lda_hi, K_lo};
  const bool va = aligned16(A_lo) && lda_lo % 4 == 0 && aligned16(A_hi) && lda_hi % 4 == 0 &&
                  K_lo % 4 == 0;
  return launch_linear_src<true>(M, N, K_lo + K_hi, src, va, W, bias, act, C, ldc, stream);
}

// The head tile: 32 whole rows (up to 256 columns) per workgroup on 4 waves
// of 32 x 64, split over KS wave groups along k.
constexpr int kHeadBM = 32, kHeadBN = 256, kHeadKS = 2;

bool linear_head_supported(int N, int K) { return N >= 1 && N <= kHeadBN && K >= 1; }

// One workgroup per 32 rows, one workgroup per CU (157 KB of LDS): the fused
// launch pays off when its grid is about one band per CU, 224..256 bands
// (measured at 512 -> 256 -> 1: M = 8192 24.0 us against 27.3 us for the
// two launches; M = 2048 23.2 against 12.8 us; past 256 bands a second,
// partial wave of bands costs more than the launch it saves).
bool linear_head_preferred(int M) {
  const int64_t bands = (int64_t)(M + kHeadBM - 1) / kHeadBM;
  return bands >= 224 && bands <= 256;
}

hipError_t launch_linear_head(int M, int N, int K, const float *A, int64_t lda, const float *W,
                              const float *bias, int act, const float *head_w,
                              const float *head_bias, int head_act, float *out, int64_t ldo,
                              hipStream_t stream) {
  if (!linear_head_supported(N, K)) return hipErrorInvalidValue;
  const ASrc src{A, lda, nullptr, 0, K};
  const bool va = aligned16(A) && lda % 4 == 0;
  const bool vw = aligned16(W) && K % 4 == 0;
  const HeadArgs head{head_w, head_bias, head_act, out, ldo};
  const int tiles = (M + kHeadBM - 1) / kHeadBM;
  const int xcd_chunk = (tiles % 8 == 0) ? tiles / 8 : 0;
  dim3 grid((unsigned)tiles), block(64 * 4 * kHeadKS);
#define DLRM_HEAD_LAUNCH(A_, W_)                                                              \
  launch_kernel((gemm_kernel<kHeadBM, kHeadBN, 1, 4, kHeadKS, A_, W_, false, false, true>), grid, \
                block, 0, stream, M, N, K, src, W, bias, act, nullptr, (int64_t)0, 1, xcd_chunk,  \
                head, KSplitArgs{0, 0, 0})
  if (va && vw)
    DLRM_HEAD_LAUNCH(true, true);
  else if (va)
    DLRM_HEAD_LAUNCH(true, false);
  else if (vw)
    DLRM_HEAD_LAUNCH(false, true);
  else
    DLRM_HEAD_LAUNCH(false, false);
#undef DLRM_HEAD_LAUNCH
  return hipGetLastError();
}

}  // namespace dlrm
