// front.h -- the delta front end shared by the forward scan and its gradients (HIP, gfx950):
// both form every step size from the raw delta with the same instructions, so that the
// gradients call recomputes exactly the states the forward call formed.
#pragma once
#include "common.h"

namespace sss {

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

// The slope of softplus at v, sigmoid(v) = 1 / (1 + e^-v): 1 / (1 + e) for v >= 0 and e / (1 + e)
// below, e = e^-|v| (accurate in both tails; e and 1 + e are the ones softplus_f forms).
__device__ __forceinline__ float softplus_slope(float v) {
  const float e = fast_exp2(-fabsf(v) * kLog2e);
  return (v >= 0.0f ? 1.0f : e) * fast_rcp(1.0f + e);
}

// The step size the recurrence uses: the stored delta, or delta + bias (then softplus).
template <int FL>
__device__ __forceinline__ float step_size(float raw, float bias) {
  if constexpr ((FL & kFront) == 0) return raw;
  const float v = raw + bias;
  if constexpr ((FL & kSoftplus) != 0) return softplus_f(v);
  return v;
}

}  // namespace sss
