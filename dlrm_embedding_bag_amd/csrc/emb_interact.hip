// emb_interact.hip -- the gather and interaction kernels for gfx950:
// emb_bag_kernel (pooled bags to HBM) and interact_kernel (the interaction
// over a pooled tensor, or fused with the gather so the pooled vectors stay
// in LDS), with their host launchers.  The building blocks and their design
// notes are in gather_interact.hpp.
//
// [FASTPATHS] = page "luminal_python: vanilla-PyTorch DLRMv1 fast paths +
//               batched FFI + input cache" (compare main...vanilla-pytorch).
#include <type_traits>

#include "gather_interact.hpp"

namespace dlrm {

namespace {

// ---------------------------------------------------------------------------
// emb_bag_pool: one group of G lanes per bag (b, k); a workgroup pools a block
// of consecutive samples of one table.
//
// The (table, sample block) tasks, in table-major order, are dealt to the
// XCDs in contiguous runs: the dispatcher sends workgroup i to XCD i % 8, and
// XCD x takes tasks [x * per_xcd, (x + 1) * per_xcd).  Each XCD's L2 then
// holds the hot rows of about K / 8 tables rather than of all K, which is
// what repeated (Zipf) indices reuse.  Measured on MI355X at B = 2048,
// K = 32, D = 64, 20 Zipf indices per bag: 35.3 us cold, 27.2 warm, against
// 38.9 and 33.5 for a bag-major grid; bit-identical output.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;

template <typename TT, int VW, int GS, bool CSR, bool PSW>
__global__ __launch_bounds__(256) void emb_bag_kernel(TableSet ts, int B, int K, int D,
                                                      int G, int64_t per_xcd,
                                                      float *__restrict__ out) {
  const int groups = blockDim.x / G;
  const int g = threadIdx.x / G;
  const int c0 = threadIdx.x - g * G;
  if (g >= groups) return;
  const int64_t blocks_per_table = (B + groups - 1) / groups;
  const int64_t task = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (task >= (int64_t)K * blocks_per_table) return;
  const int k = (int)(task / blocks_per_table);
  const int b = (int)(task - k * blocks_per_table) * groups + g;
  if (b >= B) return;
  pool_bag<TT, VW, GS, CSR, PSW>(ts, k, b, B, D / RowChunk<TT, VW>::EL, G, c0,
                                 out + ((int64_t)b * K + k) * D, nullptr);
}

// Partials 1 .. nred - 1 (nred <= NR) added to x in order.  All NR - 1 loads
// are issued before the first add (indices past nred - 1 repeat the last
// partial and are not added), so the partials arrive in one memory round
// trip rather than one each.
template <typename V, int VW, int NR>
__device__ __forceinline__ void add_partials(const float *p, int64_t stride, int nred, float *x) {
  V t[NR - 1];
#pragma unroll
  for (int r = 1; r < NR; ++r)
    t[r - 1] = *reinterpret_cast<const V *>(p + (int64_t)min(r, nred - 1) * stride);
#pragma unroll
  for (int r = 1; r < NR; ++r)
    if (r < nred) {
#pragma unroll
      for (int e = 0; e < VW; ++e) x[e] += reinterpret_cast<const float *>(&t[r - 1])[e];
    }
}

// Feature 0 from the bottom MLP's partial sums: partial 0 (already loaded as
// v) plus partials 1.. in order, then the bias and the activation.
template <typename V, int VW>
__device__ __forceinline__ V dense_reduce(const InteractParams &ip, V v, int b, int c) {
  float x[VW];
  const float *p = ip.dense + (int64_t)b * ip.ld_dense + c * VW;
#pragma unroll
  for (int e = 0; e < VW; ++e) x[e] = reinterpret_cast<const float *>(&v)[e];
  if (ip.dense_nred <= 4) {
    add_partials<V, VW, 4>(p, ip.dense_stride, ip.dense_nred, x);
  } else {
    for (int r0 = 0; r0 < ip.dense_nred - 1; r0 += 15)
      add_partials<V, VW, 16>(p + (int64_t)r0 * ip.dense_stride, ip.dense_stride,
                              min(16, ip.dense_nred - r0), x);
  }
#pragma unroll
  for (int e = 0; e < VW; ++e) {
    float y = x[e] + (ip.dense_bias ? ip.dense_bias[c * VW + e] : 0.0f);
    if (ip.dense_act == 1) y = y > 0.0f ? y : 0.0f;
    else if (ip.dense_act == 2) y = 1.0f / (1.0f + expf(-y));
    reinterpret_cast<float *>(&v)[e] = y;
  }
  return v;
}

// ---------------------------------------------------------------------------
// Interaction (and fused gather + interaction): one workgroup per S samples.
// MODE_FUSED pools the bags into the LDS tile; MODE_LOAD reads a (B, K, D)
// pooled tensor.
// ---------------------------------------------------------------------------
template <typename TT, int VW, int MODE, bool CSR, int GS, bool PSW>
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
  // With partial sums of the bottom MLP's last layer, they are added in
  // order, then that layer's bias and activation.  Taken by the last threads
  // of the workgroup: their lane groups pool the fewest bags (none, when
  // there are more groups than bags), so the dense loads' round trip is not
  // added to a group that pools the most (measured cold, K = 26, D = 64, 20
  // Zipf indices per bag: the forward at B = 8192 222.0 -> 214.0 us, at
  // B = 4096 140.5 -> 134.2; nc32 unchanged).
  for (int t = nthreads - 1 - (int)threadIdx.x; t < S * nvec; t += nthreads) {
    const int s = t / nvec;
    const int c = t - s * nvec;
    const int b = b0 + s;
    if (b >= B) continue;
    V v = reinterpret_cast<const V *>(ip.dense + (int64_t)b * ip.ld_dense)[c];
    if (ip.dense_nred > 0) v = dense_reduce<V, VW>(ip, v, b, c);
    reinterpret_cast<V *>(X + (size_t)(s * FR) * DP)[c] = v;
    if (ip.copy_dense) {
      float *o = ip.out + (int64_t)b * ip.ld_out;
      if (VW == 1 || ip.out_vec)
        reinterpret_cast<V *>(o)[c] = v;
      else
        store_unaligned(o + c * VW, v);
    }
  }

  // Phase 1b: pooled rows -> features 1..K.  The gather runs at raised wave
  // priority, so a CU issues the row loads of waves still gathering ahead of
  // other waves' dot arithmetic and its L1 miss queue stays full (measured:
  // nc32 41.5 -> 41.1 us, B = 512 17.4 -> 16.9; no change in load mode).
  if constexpr (MODE == MODE_FUSED) __builtin_amdgcn_s_setprio(1);
  const int G = ip.G;
  const int groups = nthreads / G;
  const int g = threadIdx.x / G;
  const int c0 = threadIdx.x - g * G;
  if constexpr (MODE == MODE_FUSED) {
    if (g < groups) {
      for (int t = g; t < S * K; t += groups) {
        const int s = t / K;
        const int k = t - s * K;
        const int b = b0 + s;
        if (b >= B) continue;
        float *row = X + (size_t)(s * FR + 1 + k) * DP;
        float *eo = ip.emb_out ? ip.emb_out + ((int64_t)b * K + k) * D : nullptr;
        pool_bag<TT, VW, GS, CSR, PSW>(ts, k, b, B, D / RowChunk<TT, VW>::EL, G, c0, row, eo);
      }
    }
  } else {
    // The workgroup's pooled rows are one contiguous (nvalid * K, D) block of
    // emb_in.  Each lane issues U = 4 chunk loads before it stores any
    // of them to LDS, so the block arrives in one memory round trip rather
    // than one per row.
    constexpr int U = 4;
    const int rows = min(S, B - b0) * K;
    const int n = rows * nvec;
    const V *src = reinterpret_cast<const V *>(ip.emb_in + (int64_t)b0 * K * D);
    for (int e0 = threadIdx.x; e0 < n; e0 += U * nthreads) {
      V v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + u * nthreads;
        v[u] = src[e < n ? e : 0];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + u * nthreads;
        if (e < n) {
          const int r = e / nvec;
          const int c = e - r * nvec;
          const int s = r / K;
          const int k = r - s * K;
          reinterpret_cast<V *>(X + (size_t)(s * FR + 1 + k) * DP)[c] = v[u];
        }
      }
    }
  }
  __syncthreads();

  // Phase 2: the strict-lower-triangle dots, at normal priority.
  if constexpr (MODE == MODE_FUSED) __builtin_amdgcn_s_setprio(0);
  float *out0 = ip.out + (int64_t)b0 * ip.ld_out + ip.dot_off;
  const int nvalid = min(S, B - b0);
  if constexpr (VW == 4)
    dots_blocked(X, ip, FR, out0, ip.ld_out, nvalid);
  else
    dots_per_pair<VW>(X, ip, FR, out0, ip.ld_out, nvalid);
}

}  // namespace

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
template <typename T>
struct TypeTag {
  using type = T;
};
template <int V>
using IntC = std::integral_constant<int, V>;
template <bool V>
using BoolC = std::integral_constant<bool, V>;

// Calls fn(TypeTag<TT>, IntC<VW>, BoolC<CSR>, IntC<GS>, BoolC<PSW>) with the
// compile-time form of the runtime gather configuration.
template <typename TT, int VW, bool CSR, bool PSW, typename Fn>
static void dispatch_gs(int gs, Fn &&fn) {
  const auto t = TypeTag<TT>{};
  if constexpr (VW == 1) {
    fn(t, IntC<1>{}, BoolC<CSR>{}, IntC<0>{}, BoolC<PSW>{});
  } else {
    switch (gs) {
      case 4: fn(t, IntC<4>{}, BoolC<CSR>{}, IntC<4>{}, BoolC<PSW>{}); break;
      case 8: fn(t, IntC<4>{}, BoolC<CSR>{}, IntC<8>{}, BoolC<PSW>{}); break;
      case 16: fn(t, IntC<4>{}, BoolC<CSR>{}, IntC<16>{}, BoolC<PSW>{}); break;
      case 32: fn(t, IntC<4>{}, BoolC<CSR>{}, IntC<32>{}, BoolC<PSW>{}); break;
      case 64: fn(t, IntC<4>{}, BoolC<CSR>{}, IntC<64>{}, BoolC<PSW>{}); break;
      default: fn(t, IntC<4>{}, BoolC<CSR>{}, IntC<0>{}, BoolC<PSW>{}); break;
    }
  }
}

template <typename TT, int VW, typename Fn>
static void dispatch_flags(bool csr, bool psw, int gs, Fn &&fn) {
  if (csr) {
    if (psw)
      dispatch_gs<TT, VW, true, true>(gs, fn);
    else
      dispatch_gs<TT, VW, true, false>(gs, fn);
  } else {
    if (psw)
      dispatch_gs<TT, VW, false, true>(gs, fn);
    else
      dispatch_gs<TT, VW, false, false>(gs, fn);
  }
}

template <typename Fn>
static void dispatch_gather(const GatherConfig &gc, int D, Fn &&fn) {
  const int gs = gc.vec ? shuffle_group(D / chunk_elems(gc.dtype, true)) : 0;
  if (gc.dtype == kFP8) {
    if (gc.vec)
      dispatch_flags<uint8_t, 4>(gc.csr, gc.psw, gs, fn);
    else
      dispatch_flags<uint8_t, 1>(gc.csr, gc.psw, gs, fn);
  } else if (gc.dtype == kBF16) {
    if (gc.vec)
      dispatch_flags<uint16_t, 4>(gc.csr, gc.psw, gs, fn);
    else
      dispatch_flags<uint16_t, 1>(gc.csr, gc.psw, gs, fn);
  } else {
    if (gc.vec)
      dispatch_flags<float, 4>(gc.csr, gc.psw, gs, fn);
    else
      dispatch_flags<float, 1>(gc.csr, gc.psw, gs, fn);
  }
}

hipError_t launch_emb_bag(const TableSet &ts, const GatherConfig &gc, int B, int K, int D,
                          float *out, hipStream_t stream) {
  const int G = lanes_per_row(D, chunk_elems(gc.dtype, gc.vec));
  const int threads = 256;
  const int groups = threads / G;
  const int64_t tasks = (int64_t)K * ((B + groups - 1) / groups);
  const int64_t per_xcd = (tasks + kXcds - 1) / kXcds;
  if (per_xcd * kXcds > INT32_MAX) return hipErrorInvalidValue;
  dim3 grid((unsigned)(per_xcd * kXcds)), block(threads);
  dispatch_gather(gc, D, [&](auto tt, auto vw, auto csr, auto gs, auto psw) {
    using TT = typename decltype(tt)::type;
    launch_kernel((emb_bag_kernel<TT, decltype(vw)::value, decltype(gs)::value,
                                  decltype(csr)::value, decltype(psw)::value>),
                  grid, block, 0, stream, ts, B, K, D, G, per_xcd, out);
  });
  return hipGetLastError();
}

// Workgroup size of the interaction kernels: 128 threads (2 waves), with the
// lane groups looping over the sample's bags.  Measured on MI355X (nc32
// shape, cold): 45.7 us at up to 512 threads per workgroup, 42.6 at 256,
// 41.2 at 128, 48.3 at 64; CSR bags of 0..40 rows 55.7 -> 48.4 us, since a
// group's several bags even out their sizes.  Small workgroups let many
// resident workgroups interleave their gather and dot phases on a CU.  A
// grid that leaves the chip idle takes larger ones (below): measured cold at
// K = 32, D = 64, 20 Zipf indices per bag, B = 2: 20.4 -> 10.7 us, B = 256:
// 21.8 -> 12.8, B = 1024: 28.6 -> 25.4 (K = 26: 19.5 -> 10.2, 20.2 -> 11.7,
// 26.4 -> 22.9), B >= 2048 unchanged; fill thresholds of 2048 and 8192
// waves were each slower somewhere.
constexpr int kMaxThreadsFull = 128;  // workgroup size while the grid fills the chip
constexpr int64_t kWaveFill = 4096;    // waves that count as a full chip (16 per CU)

bool plan_interact(int B, int K, int D, bool vec4, int el, InteractParams &ip, int &threads) {
  const int F = K + 1;
  ip.B = B;
  ip.K = K;
  ip.D = D;
  ip.P = F * (F - 1) / 2;
  ip.DP = D + (vec4 ? 4 : 1);
  ip.FR = vec4 ? ((F + 3) & ~3) : F;
  ip.G = lanes_per_row(D, el);
  const size_t per_sample = (size_t)ip.FR * ip.DP * sizeof(float);
  if (per_sample > kLdsBudget) return false;
  const int lanes_per_sample = K * ip.G;
  int S = 1;
  while (S * lanes_per_sample < kMinThreads &&
         (size_t)(2 * S) * per_sample <= kLdsBudget / 2 &&
         S < B)
    S *= 2;
  ip.S = S;
  // Workgroup size: kMaxThreadsFull when the grid fills the chip, so that
  // many resident workgroups interleave their gather and dot phases; when it
  // does not (fewer than kWaveFill waves at the next size up), doubled
  // up to all of a sample's lane groups at once, so that its bags are pooled
  // side by side instead of in turn by a few groups.
  const int want = S * lanes_per_sample;
  const int64_t nwg = (B + S - 1) / S;
  int cap = kMaxThreadsFull;
  while (cap < want && 2 * cap <= 1024 && nwg * (2 * cap / kWave) <= kWaveFill) cap *= 2;
  threads = ((min(want, cap) + kWave - 1) / kWave) * kWave;
  if (threads < kMinThreads) threads = kMinThreads;
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

hipError_t launch_interact(const TableSet *ts, const GatherConfig &gc, const InteractParams &ip,
                           int threads, hipStream_t stream) {
  dim3 grid((unsigned)((ip.B + ip.S - 1) / ip.S)), block(threads);
  const size_t lds = (size_t)ip.lds_bytes;
  if (ts) {
    dispatch_gather(gc, ip.D, [&](auto tt, auto vw, auto csr, auto gs, auto psw) {
      using TT = typename decltype(tt)::type;
      launch_kernel((interact_kernel<TT, decltype(vw)::value, MODE_FUSED,
                                     decltype(csr)::value, decltype(gs)::value,
                                     decltype(psw)::value>),
                    grid, block, lds, stream, *ts, ip);
    });
  } else {
    TableSet empty{};
    if (gc.vec)
      launch_kernel((interact_kernel<float, 4, MODE_LOAD, false, 0, false>), grid, block,
                    lds, stream, empty, ip);
    else
      launch_kernel((interact_kernel<float, 1, MODE_LOAD, false, 0, false>), grid, block,
                    lds, stream, empty, ip);
  }
  return hipGetLastError();
}

}  // namespace dlrm
