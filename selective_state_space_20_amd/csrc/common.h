// common.h -- device helpers shared by the gfx950 scan kernels (HIP, CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sss {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kFltMax = 3.402823466e+38f;

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float fast_rcp(float v) { return __builtin_amdgcn_rcpf(v); }

// silu(z) = z / (1 + e^-z) with v_exp / v_rcp.
__device__ __forceinline__ float silu(float z) { return z * fast_rcp(1.0f + fast_exp2(-z * kLog2e)); }

// Workgroup id -> logical id such that consecutive logical ids share an XCD (workgroups
// are dealt round-robin over the 8 XCDs of an MI355X; neighbouring channel tiles then
// share that XCD's L2).  Identity when the grid is not a multiple of 8.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t id, uint32_t n) {
  if ((n & 7u) != 0u) return id;
  return (id & 7u) * (n >> 3) + (id >> 3);
}

}  // namespace sss
