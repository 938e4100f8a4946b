// forward_small.hip -- the whole DLRMv1 forward in one launch, for models
// whose MLPs are small enough to stream their weights through every
// workgroup (gfx950).
//
// [FASTPATHS] = page "luminal_python: vanilla-PyTorch DLRMv1 fast paths +
//               batched FFI + input cache" (compare main...vanilla-pytorch).
//
// The pages measure their DLRMv1 on a small cell (3 dense features, D = 16,
// two indices per bag, 4096-row tables) where every forward is a handful of
// tiny kernels and the time goes to launching them (the commit message's
// per-iteration breakdown, RESULTS.md).  Here one workgroup carries S samples
// through every step with all intermediates in LDS:
//   bottom MLP  dense_in -> ... -> feature 0 of the interaction tile
//   gather      the K bags of each sample into features 1..K of the tile
//   interaction dense copy and strict-lower-triangle dots into R (LDS)
//   top MLP     R -> ... -> out (HBM)
// Each MLP output is a dot product owned by one 16-lane DPP row: its lanes
// split the inputs and reduce with DPP.  When they fit beside the samples,
// all weights and biases are copied into LDS at the start with the LDS-DMA
// load (global_load_lds: memory to LDS without registers), so the copy is in
// flight together with the gather's loads and no layer waits on L2; otherwise
// the layers read their weight rows from memory (L2-resident: the whole MLP is
// at most kSmallWeightFloats floats).
// The gather and the interaction are the building blocks of the fused
// gather + interaction kernel (gather_interact.hpp).
#include <type_traits>

#include "gather_interact.hpp"

namespace dlrm {

namespace {

constexpr int kSmallThreads = 256;

__device__ __forceinline__ float small_act(float x, int act) {
  if (act == 1) return x > 0.0f ? x : 0.0f;
  if (act == 2) return 1.0f / (1.0f + expf(-x));
  return x;
}

// out[s * ld_out + n] = act(bias[n] + sum_k in[s * ld_in + k] W[n * K + k])
// for s < S, stored only for s < nstore.  A 16-lane DPP row owns one (s, n).
// W and bias point to LDS or to memory; bias is read only when has_bias.
__device__ __forceinline__ void small_layer(const float *in, int ld_in, const float *W,
                                            const float *bias, bool has_bias, int K, int N,
                                            int act, float *out, int64_t ld_out, int S,
                                            int nstore) {
  const int teams = blockDim.x >> 4;
  const int team = threadIdx.x >> 4;
  const int tl = threadIdx.x & 15;
  for (int t = team; t < S * N; t += teams) {
    const int s = t / N;
    const int n = t - s * N;
    const float *w = W + (int64_t)n * K;
    const float *x = in + s * ld_in;
    float acc = 0.0f;
    for (int k = tl; k < K; k += 16) acc = __builtin_fmaf(x[k], w[k], acc);
    acc = row16_sum(acc);
    if (tl == 0 && s < nstore)
      out[(int64_t)s * ld_out + n] = small_act(acc + (has_bias ? bias[n] : 0.0f), act);
  }
}

// Copies n floats from memory to LDS with LDS-DMA loads: lane i of a wave
// moves one dword to dst + c + i.  Nothing waits here; the caller waits for
// the vector-memory counter and synchronizes before the data is read.
__device__ __forceinline__ void dma_to_lds(float *dst, const float *src, int n) {
  const int lane = threadIdx.x & 63;
  const int waves = blockDim.x >> 6;
  for (int c = (threadIdx.x >> 6) * 64; c < n; c += waves * 64)
    if (c + lane < n) __builtin_amdgcn_global_load_lds(src + c + lane, dst + c, 4, 0, 0);
}

// Layer slot l of the model on S samples, its weights read from their LDS
// copies when STAGED, else from memory.
template <bool STAGED>
__device__ __forceinline__ void run_layer(const SmallForwardParams &p, int l, const float *lds,
                                          const float *in, int ld_in, float *out, int64_t ld_out,
                                          int S, int nstore) {
  const SmallLayer &L = p.layer[l];
  if constexpr (STAGED)
    small_layer(in, ld_in, lds + p.w_off[l], lds + p.bias_off[l], L.bias != nullptr, L.K, L.N,
                L.act, out, ld_out, S, nstore);
  else
    small_layer(in, ld_in, L.W, L.bias, L.bias != nullptr, L.K, L.N, L.act, out, ld_out, S,
                nstore);
}

template <int VW, bool CSR, int GS, bool STAGED>
__global__ __launch_bounds__(kSmallThreads) void forward_small_kernel(TableSet ts,
                                                                      SmallForwardParams p) {
  extern __shared__ float4 lds_raw[];
  float *lds = reinterpret_cast<float *>(lds_raw);
  const InteractParams &ip = p.ip;
  const int B = ip.B, K = ip.K, D = ip.D, S = ip.S, DP = ip.DP, FR = ip.FR;
  const int b0 = blockIdx.x * S;
  const int nvalid = min(S, B - b0);
  const int nthreads = blockDim.x;
  float *X = lds;                 // S x FR x DP interaction tile
  float *R = lds + p.r_off;       // S x ldR: [dense | dots]
  float *buf[2] = {lds + p.a_off, lds + p.b_off};  // S x ld_buf each

  // Stage the MLP weights in LDS (in flight during the loads below).
  if constexpr (STAGED) {
#pragma unroll
    for (int l = 0; l < 2 * kMaxSmallLayers; ++l) {
      const SmallLayer &L = p.layer[l];
      if (L.W == nullptr) continue;
      dma_to_lds(lds + p.w_off[l], L.W, L.K * L.N);
      if (L.bias) dma_to_lds(lds + p.bias_off[l], L.bias, L.N);
    }
  }

  // Dense input rows (zeros past the batch).
  for (int t = threadIdx.x; t < S * p.in0; t += nthreads) {
    const int s = t / p.in0;
    const int c = t - s * p.in0;
    buf[0][s * p.ld_buf + c] = (s < nvalid) ? p.dense_in[(int64_t)(b0 + s) * p.in0 + c] : 0.0f;
  }

  // Bottom MLP; its last layer writes feature 0 of each sample's tile.
  auto bottom_mlp = [&]() {
    const float *in = buf[0];
    int ld_in = p.ld_buf;
#pragma unroll
    for (int l = 0; l < kMaxSmallLayers; ++l) {
      if (l >= p.nb) break;
      const bool last = l + 1 == p.nb;
      float *o = last ? X : buf[(l + 1) & 1];
      run_layer<STAGED>(p, l, lds, in, ld_in, o, last ? FR * DP : p.ld_buf, S, S);
      __syncthreads();
      in = o;
      ld_in = last ? FR * DP : p.ld_buf;
    }
  };
  // Order of the first steps (measured on the pages' cells): with weights
  // read from memory, the bottom MLP runs before the gather; with weights
  // staged in LDS, the gather's loads go out together with the copy and the
  // bottom MLP follows.
  if constexpr (!STAGED) {
    __syncthreads();
    bottom_mlp();
  }

  // Gather: the K bags of each sample into features 1..K.
  {
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
        float *row = X + (size_t)(s * FR + 1 + k) * DP;
        pool_bag<float, VW, GS, CSR, false>(ts, k, b, B, D / VW, G, c0, row, nullptr);
      }
    }
  }
  // The LDS-DMA copies (and every other load) have landed; all lanes agree.
  if constexpr (STAGED) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if constexpr (STAGED) bottom_mlp();

  // Interaction: R = [dense | dots] for every staged sample.
  for (int t = threadIdx.x; t < S * D; t += nthreads) {
    const int s = t / D;
    const int c = t - s * D;
    R[s * p.ldR + c] = X[(size_t)(s * FR) * DP + c];
  }
  if constexpr (VW == 4)
    dots_blocked(X, ip, FR, R + D, p.ldR, S);
  else
    dots_per_pair<VW>(X, ip, FR, R + D, p.ldR, S);
  __syncthreads();

  // Top MLP; its last layer writes the output rows of the valid samples.
  {
    const float *in = R;
    int ld_in = p.ldR;
#pragma unroll
    for (int l = 0; l < kMaxSmallLayers; ++l) {
      if (l >= p.nt) break;
      const bool last = l + 1 == p.nt;
      if (last) {
        run_layer<STAGED>(p, kMaxSmallLayers + l, lds, in, ld_in, p.out + (int64_t)b0 * p.n_out,
                  p.n_out, S, nvalid);
      } else {
        float *o = buf[l & 1];
        run_layer<STAGED>(p, kMaxSmallLayers + l, lds, in, ld_in, o, p.ld_buf, S, S);
        __syncthreads();
        in = o;
        ld_in = p.ld_buf;
      }
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static int round4i(int x) { return (x + 3) & ~3; }

bool plan_forward_small(int B, int K, int D, bool vec4, int in0, int nb, const SmallLayer *bottom,
                        int nt, const SmallLayer *top, SmallForwardParams &p, int &threads) {
  if (nb < 1 || nb > kMaxSmallLayers || nt < 1 || nt > kMaxSmallLayers || B < 1) return false;
  int64_t weights = 0;
  int widest = in0;  // widest LDS-held activation outside the tile and R
  for (int l = 0; l < nb; ++l) {
    if (bottom[l].K > kSmallMaxWidth || bottom[l].N > kSmallMaxWidth) return false;
    weights += (int64_t)bottom[l].K * bottom[l].N;
    if (l + 1 < nb) widest = widest > bottom[l].N ? widest : bottom[l].N;
  }
  for (int l = 0; l < nt; ++l) {
    if (top[l].K > kSmallMaxWidth || top[l].N > kSmallMaxWidth) return false;
    weights += (int64_t)top[l].K * top[l].N;
    if (l + 1 < nt) widest = widest > top[l].N ? widest : top[l].N;
  }
  if (weights > kSmallWeightFloats) return false;
  if (in0 > kSmallMaxWidth) return false;
  InteractParams &ip = p.ip;
  int unused = 0;
  if (!plan_interact(B, K, D, vec4, vec4 ? 4 : 1, ip, unused)) return false;
  const int F = K + 1;
  p.ldR = round4i(D + F * (F - 1) / 2);
  p.ld_buf = round4i(widest);
  const size_t tile = (size_t)ip.FR * ip.DP;
  const size_t per_sample = (tile + (size_t)p.ldR + 2 * (size_t)p.ld_buf) * sizeof(float);
  if (per_sample > kLdsBudget) return false;
  // LDS copy of every layer's weights and bias, each segment 16-byte aligned.
  size_t wfloats = 0;
  for (int l = 0; l < kMaxSmallLayers; ++l) {
    const SmallLayer *L[2] = {l < nb ? &bottom[l] : nullptr, l < nt ? &top[l] : nullptr};
    for (int h = 0; h < 2; ++h) {
      const int slot = h * kMaxSmallLayers + l;
      p.w_off[slot] = p.bias_off[slot] = 0;
      if (!L[h]) continue;
      p.w_off[slot] = (int)wfloats;
      wfloats += ((size_t)L[h]->K * L[h]->N + 3) & ~size_t(3);
      p.bias_off[slot] = (int)wfloats;
      if (L[h]->bias) wfloats += ((size_t)L[h]->N + 3) & ~size_t(3);
    }
  }
  // Samples per workgroup: enough workgroups to cover the chip twice when
  // the batch allows, as many as LDS takes otherwise; fewer if that lets the
  // weights be staged in LDS.
  // LDS floats of S samples' regions, rounded up to 16 bytes; the weights follow.
  auto samples_floats = [&](int s) {
    return ((size_t)s * (tile + p.ldR + 2 * (size_t)p.ld_buf) + 3) & ~size_t(3);
  };
  auto staged_fits = [&](int s) {
    return (samples_floats(s) + wfloats) * sizeof(float) <= kLdsBudget;
  };
  int S = 1;
  while (2 * S <= 16 && (size_t)(2 * S) * per_sample <= kLdsBudget && 2 * S * 512 <= B) S *= 2;
  // Staging pays when a workgroup serves several samples (measured on the
  // pages' cells, nc=32: 2 us faster at 4 samples per workgroup (b=2048),
  // 1 us slower at 2 (b=1024)).
  p.w_lds = S >= 4 && staged_fits(S);
  ip.S = S;
  threads = kSmallThreads;
  const int nbr = ip.FR / 4;
  const int work = S * nbr * (nbr + 1) / 2;
  const int quads = threads / 4;
  ip.Q = (work * 4 <= quads) ? 4 : (work * 2 <= quads) ? 2 : 1;
  p.r_off = (int)(S * tile);
  p.a_off = p.r_off + S * p.ldR;
  p.b_off = p.a_off + S * p.ld_buf;
  const int w_base = (int)samples_floats(S);
  for (int slot = 0; slot < 2 * kMaxSmallLayers; ++slot) {
    p.w_off[slot] += w_base;
    p.bias_off[slot] += w_base;
  }
  ip.lds_bytes = (int)(p.w_lds ? (size_t)(w_base + wfloats) * sizeof(float)
                               : (size_t)S * per_sample);
  p.in0 = in0;
  p.nb = nb;
  p.nt = nt;
  for (int l = 0; l < kMaxSmallLayers; ++l) {
    p.layer[l] = l < nb ? bottom[l] : SmallLayer{};
    p.layer[kMaxSmallLayers + l] = l < nt ? top[l] : SmallLayer{};
  }
  return true;
}

hipError_t launch_forward_small(const TableSet &ts, bool csr, bool vec4,
                                const SmallForwardParams &p, int threads, hipStream_t stream) {
  dim3 grid((unsigned)((p.ip.B + p.ip.S - 1) / p.ip.S)), block(threads);
  const size_t lds = (size_t)p.ip.lds_bytes;
  const int gs = vec4 ? shuffle_group(p.ip.D / 4) : 0;
  auto go = [&](auto vw, auto gsv, auto staged) {
    constexpr int VW = decltype(vw)::value, GSV = decltype(gsv)::value;
    constexpr bool ST = decltype(staged)::value;
    if (csr)
      launch_kernel((forward_small_kernel<VW, true, GSV, ST>), grid, block, lds, stream, ts,
                    p);
    else
      launch_kernel((forward_small_kernel<VW, false, GSV, ST>), grid, block, lds, stream, ts,
                    p);
  };
  auto with_stage = [&](auto vw, auto gsv) {
    if (p.w_lds)
      go(vw, gsv, std::true_type{});
    else
      go(vw, gsv, std::false_type{});
  };
  using I1 = std::integral_constant<int, 1>;
  using I4 = std::integral_constant<int, 4>;
  if (!vec4) {
    with_stage(I1{}, std::integral_constant<int, 0>{});
    return hipGetLastError();
  }
  switch (gs) {
    case 4: with_stage(I4{}, std::integral_constant<int, 4>{}); break;
    case 8: with_stage(I4{}, std::integral_constant<int, 8>{}); break;
    case 16: with_stage(I4{}, std::integral_constant<int, 16>{}); break;
    case 32: with_stage(I4{}, std::integral_constant<int, 32>{}); break;
    case 64: with_stage(I4{}, std::integral_constant<int, 64>{}); break;
    default: with_stage(I4{}, std::integral_constant<int, 0>{}); break;
  }
  return hipGetLastError();
}

}  // namespace dlrm
