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

// The slope of softplus at v from the step size sp = softplus(v): sigmoid(v) = 1 - e^-sp.  Below sp = 1/16
// the series sp (1 - sp/2 (1 - sp/3 (1 - sp/4))) (truncation below 2e-7 relative, no
// cancellation), above it 1 - e^-sp (cancellation below 1e-6 relative).
__device__ __forceinline__ float softplus_slope_of_step(float sp) {
  const float ser = sp * (1.0f - 0.5f * sp * (1.0f - (1.0f / 3.0f) * sp * (1.0f - 0.25f * sp)));
  return sp < 0.0625f ? ser : 1.0f - fast_exp2(-sp * kLog2e);
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
