// common.hpp -- internal helpers shared by the HIP kernels of libdlrm_mi355x.
//
// Target: gfx950 (CDNA4): 64-lane wavefronts, 160 KiB LDS per CU, 256 CUs in
// 8 XCDs, HBM3E.  Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace dlrm {

constexpr int kMaxTables = 64;
constexpr int kWave = 64;
constexpr size_t kLdsBudget = 64 * 1024;  // dynamic LDS per workgroup we allow

// Table storage types (values of dlrm_dtype).
enum { kF32 = 0, kBF16 = 1, kFP8 = 2 };

// Per-table device pointers and bag geometry, passed to the kernels by value
// in the kernel-argument segment (2.8 KiB), so a call needs no host-to-device
// copy of a pointer table.
struct TableSet {
  const void *table[kMaxTables];   // float32, bfloat16 or fp8 rows, per the kernel's type
  const int32_t *idx[kMaxTables];
  const int32_t *off[kMaxTables];  // CSR bag starts; unused in uniform mode
  const float *wt[kMaxTables];     // per-sample weights (n_idx,); used by weighted kernels
  int32_t bag[kMaxTables];         // L_k, uniform mode
  int32_t nidx[kMaxTables];        // number of indices of table k
  float scale[kMaxTables];         // per-table factor on the pooled value
  int32_t mean;                    // divide every non-empty bag's sum by its size
  int32_t scaled;                  // apply scale[]
};

template <int VW>
struct Vec;
template <>
struct Vec<1> {
  using T = float;
};
template <>
struct Vec<4> {
  using T = float4;
};

__device__ __forceinline__ float4 operator_add(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ float operator_add(float a, float b) { return a + b; }

template <typename T>
__device__ __forceinline__ T vzero();
template <>
__device__ __forceinline__ float vzero<float>() {
  return 0.0f;
}
template <>
__device__ __forceinline__ float4 vzero<float4>() {
  return make_float4(0.f, 0.f, 0.f, 0.f);
}

// Dot-product accumulation of one vector chunk.
__device__ __forceinline__ float vdot_acc(float4 a, float4 b, float acc) {
  acc = __builtin_fmaf(a.x, b.x, acc);
  acc = __builtin_fmaf(a.y, b.y, acc);
  acc = __builtin_fmaf(a.z, b.z, acc);
  acc = __builtin_fmaf(a.w, b.w, acc);
  return acc;
}
__device__ __forceinline__ float vdot_acc(float a, float b, float acc) {
  return __builtin_fmaf(a, b, acc);
}

// Sum over the 4 lanes of a quad with two DPP quad permutations; every lane
// of the quad ends with the total.  All 4 lanes must be active.
__device__ __forceinline__ float quad_sum(float v) {
  // quad_perm [1,0,3,2]: swap neighbours
  int s1 = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false);
  v += __int_as_float(s1);
  // quad_perm [2,3,0,1]: swap pairs
  int s2 = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false);
  v += __int_as_float(s2);
  return v;
}

// Sum over the 16 lanes of a DPP row; every lane of the row ends with the
// total.  All 16 lanes must be active.
__device__ __forceinline__ float row16_sum(float v) {
  v = quad_sum(v);
  // row_half_mirror: lane i <- lane 7-i within each half row (other quad)
  int s3 = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false);
  v += __int_as_float(s3);
  // row_mirror: lane i <- lane 15-i (other half row)
  int s4 = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false);
  v += __int_as_float(s4);
  return v;
}

// Strict-lower-triangle pair p -> (i, j), i > j, in row-major order.
// Row i starts at i(i-1)/2, so i is the largest integer with i(i-1)/2 <= p,
// i.e. i = floor((1 + sqrt(8p + 1)) / 2) = (1 + isqrt(8p + 1)) / 2.  The
// integer square root starts from the float estimate and is made exact by
// one correction in each direction (the estimate is within one for every
// argument below 2^48).
__device__ __forceinline__ void pair_from_index(uint32_t p, int &i, int &j) {
  const uint64_t q = 8ull * p + 1ull;
  uint64_t r = (uint64_t)__builtin_sqrtf((float)q);
  r -= (r * r > q) ? 1 : 0;
  r += ((r + 1) * (r + 1) <= q) ? 1 : 0;
  i = (int)((r + 1) >> 1);
  j = (int)(p - (uint32_t)i * (uint32_t)(i - 1) / 2u);
}

// Events that the calling thread's kernel launches record at the kernel's own
// start and end (both null when timing is off); set through
// dlrm_set_kernel_timing_events, stored per thread in abi.hip.
struct LaunchTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
LaunchTiming &launch_timing();

// Every kernel of the library is launched here.  With timing on, the launch
// goes through hipExtLaunchKernel, whose events take the dispatch's own begin
// and end timestamps, so their elapsed time is the kernel's execution alone;
// argument conversion to the kernel's parameter types is the same either way.
template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds,
                          hipStream_t stream, Args &&...args) {
  const LaunchTiming &t = launch_timing();
  if (t.start)
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, stream, t.start, t.stop, 0u,
                          std::forward<Args>(args)...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, std::forward<Args>(args)...);
}

__host__ __device__ inline bool aligned16(const void *p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

}  // namespace dlrm
