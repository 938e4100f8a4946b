// probe.hip -- a streaming-read kernel for gfx950: measurement support, not a
// step of the method.  It reads a device buffer once with the access shape of
// the gather's row loads (16-byte loads, 16 consecutive lanes covering 256
// contiguous bytes, several loads in flight per lane) and stores nothing but
// a never-taken conditional write, so its duration measures the rate at
// which HBM delivers reads, the practical peak the gather's bytes are held
// against, and a dispatch of known read bytes calibrates the memory-traffic
// counters.
#include "../../include/dlrm_embedding_bag.h"
#include "common.hpp"

namespace dlrm {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeInFlight = 8;  // 16-byte loads in flight per lane

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(
    const uint4 *__restrict__ p, int64_t n16, uint32_t key, float *__restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeInFlight - 1) * stride < n16; i += kProbeInFlight * stride) {
    uint4 v[kProbeInFlight];
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // The loads feed a value the host cannot predict; the store happens only
  // when it equals the caller's key, which a caller picks not to occur.
  if (acc == key) sink[0] = __uint_as_float(acc);
}

}  // namespace

}  // namespace dlrm

extern "C" {

int dlrm_stream_read(const void *buf, size_t bytes, float *sink, void *stream) {
  if (bytes == 0) return DLRM_OK;
  if (!buf || !sink) return DLRM_ERR_NULL;
  if ((bytes & 15u) != 0 || !dlrm::aligned16(buf)) return DLRM_ERR_SHAPE;
  const int64_t n16 = (int64_t)(bytes / 16);
  // 8 workgroups per CU of the 256-CU chip, fewer for a small buffer
  const int64_t per_sweep = (int64_t)dlrm::kProbeThreads * dlrm::kProbeInFlight;
  int64_t wgs = (n16 + per_sweep - 1) / per_sweep;
  if (wgs > 2048) wgs = 2048;
  dlrm::launch_kernel(dlrm::stream_read_kernel, dim3((unsigned)wgs), dim3(dlrm::kProbeThreads),
                      0, (hipStream_t)stream, reinterpret_cast<const uint4 *>(buf), n16,
                      0x9e3779b9u, sink);
  return hipGetLastError() == hipSuccess ? DLRM_OK : DLRM_ERR_HIP;
}

}  // extern "C"
