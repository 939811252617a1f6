// common.h -- device helpers shared by the gfx950 scan kernels (HIP, CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sss {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFltMax = 3.402823466e+38f;

// ---------------------------------------------------------------- DPP (wave64, gfx9 encodings)
// dpp_ctrl values: row_shr:n = 0x110 + n, wave_shr:1 = 0x138, row_bcast:15 = 0x142,
// row_bcast:31 = 0x143.  With bound_ctrl off, a lane whose source is outside the pattern
// (or whose row is masked off) keeps `old`.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_or(float old, float src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, src), CTRL, ROW_MASK,
                                                               0xF, false));
}

// One Hillis-Steele level of an inclusive scan of affine pairs (a, b) ~ h -> a*h + b:
// this lane's pair is composed after the pair held DIST lanes earlier (identity (1, 0)
// where that lane is outside the group).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void scan_level(float& a, float& b) {
  float ap = dpp_or<CTRL, ROW_MASK>(1.0f, a);
  float bp = dpp_or<CTRL, ROW_MASK>(0.0f, b);
  b = __builtin_fmaf(a, bp, b);
  a = a * ap;
}

// Inclusive scan over all 64 lanes of the wave (lane order = time order).
__device__ __forceinline__ void wave_scan_pairs(float& a, float& b) {
  scan_level<0x111, 0xF>(a, b);  // row_shr:1
  scan_level<0x112, 0xF>(a, b);  // row_shr:2
  scan_level<0x114, 0xF>(a, b);  // row_shr:4
  scan_level<0x118, 0xF>(a, b);  // row_shr:8
  scan_level<0x142, 0xA>(a, b);  // row_bcast:15 into rows 1, 3
  scan_level<0x143, 0xC>(a, b);  // row_bcast:31 into rows 2, 3
}

// Same scan with the lane shift fused into the arithmetic (v_fmac/v_mul with a DPP source):
// a lane whose source is outside the pattern, or whose row is masked off, is not written,
// which leaves it composed with the identity.  Per level: b = a * b[src] + b, then
// a = a[src] * a.  The s_nop 1 before each DPP instruction provides the two wait states a
// DPP read of a VGPR written by the previous VALU instruction needs on gfx9.
__device__ __forceinline__ void wave_scan_pairs_fused(float& a, float& b) {
  asm volatile(
      "s_nop 1\n\tv_fmac_f32_dpp %1, %1, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_fmac_f32_dpp %1, %1, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_fmac_f32_dpp %1, %1, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_fmac_f32_dpp %1, %1, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\tv_fmac_f32_dpp %1, %1, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "s_nop 1\n\tv_fmac_f32_dpp %1, %1, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
      "s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf"
      : "+v"(a), "+v"(b));
}

// Lane j receives v from lane j-1; lane 0 receives `first`.
__device__ __forceinline__ float wave_shift_in(float v, float first) {
  float r;
  asm volatile("s_nop 1\n\tv_mov_b32_dpp %0, %1 wave_shr:1 row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(v), "0"(first));
  return r;
}

// Wave-wide inclusive sum (lane order), then the total from lane 63.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_or<0x111, 0xF>(0.0f, v);
  v += dpp_or<0x112, 0xF>(0.0f, v);
  v += dpp_or<0x114, 0xF>(0.0f, v);
  v += dpp_or<0x118, 0xF>(0.0f, v);
  v += dpp_or<0x142, 0xA>(0.0f, v);
  v += dpp_or<0x143, 0xC>(0.0f, v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// vec with lane `lane` replaced by the (wave-uniform) value val.
__device__ __forceinline__ float set_lane(float vec, float val, int lane) {
  return (int)(threadIdx.x & 63) == lane ? val : vec;
}

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

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
