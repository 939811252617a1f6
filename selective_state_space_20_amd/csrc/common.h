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

// Delta front-end bits of a kernel's option mask: kFront -- the step size is delta + bias[d];
// kSoftplus (with kFront) -- softplus of that.
constexpr int kFront = 2, kSoftplus = 4;

// softplus(v) = max(v, 0) + log1p(e^-|v|); log1p through the log(u) * e / (u - 1) form so
// that small e keeps its relative precision.
__device__ __forceinline__ float softplus_f(float v) {
  const float e = fast_exp2(-fabsf(v) * kLog2e);
  const float u = 1.0f + e;
  const float l = u == 1.0f ? e : __builtin_amdgcn_logf(u) * kLn2 * e * fast_rcp(u - 1.0f);
  return fmaxf(v, 0.0f) + l;
}

// The step size the recurrence uses: the stored delta, or delta + bias (then softplus).
template <int FL>
__device__ __forceinline__ float step_size(float raw, float bias) {
  if constexpr ((FL & kFront) == 0) return raw;
  const float v = raw + bias;
  if constexpr ((FL & kSoftplus) != 0) return softplus_f(v);
  return v;
}

// Workgroup id -> logical id such that consecutive logical ids share an XCD (workgroups
// are dealt round-robin over the 8 XCDs of an MI355X; neighbouring channel tiles then
// share that XCD's L2).  Identity when the grid is not a multiple of 8.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t id, uint32_t n) {
  if ((n & 7u) != 0u) return id;
  return (id & 7u) * (n >> 3) + (id >> 3);
}

}  // namespace sss
