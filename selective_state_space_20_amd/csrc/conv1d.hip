// conv1d.hip -- gfx950 kernel for the causal depthwise convolution in front of the scan.
//
// The Mamba block runs x through a short causal depthwise convolution (and silu) before
// the selective scan ("Toan Canh Tien Hoa Kien Truc AI ...", section "5.3. Toi uu hoa
// Kernel Fusion cho Mamba SSM", which names the causal_conv1d kernel):
//   out[b,t,d] = bias[d] + sum_{k<W} w[d,k] * x[b, t-(W-1)+k, d]   (x = 0 before t = 0),
//   then optionally silu.
// It is pure streaming (2 + 2 bytes per element in bf16, W fmas), so it is laid out like
// the elementwise scan: one lane per channel, 64 adjacent channels per wave (every load and
// store is one 128/256-byte row piece through a buffer descriptor with a wave-uniform step
// offset), two batches of steps in flight, and the last W-1 inputs of the channel kept in
// registers as a sliding window.  Time is cut into segments for parallelism; a segment
// starts by reading the W-1 inputs before it.  On a chip where the scan itself is bound by
// transcendental issue, a separate streaming pass costs about what fusing it into both
// scan passes would add there, and keeps the scan kernels unchanged.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace sss {

struct ConvSeg {
  int64_t batch, L, D, seg_len;
  int ngroups;  // ceil(D / 64)
};

constexpr int kConvU = 16;  // steps per load batch

__device__ __forceinline__ __amdgpu_buffer_rsrc_t conv_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  const uint32_t q = (u >> 16) | 0x40u;  // quiet NaN keeps its sign
  return (u & 0x7FFFFFFFu) > 0x7F800000u ? q : r;
}

template <int W, bool BF16, bool SILU>
__global__ __launch_bounds__(64) void conv1d_kernel(const void* __restrict__ x, const float* __restrict__ w,
                                                    const float* __restrict__ bias, void* __restrict__ out,
                                                    ConvSeg g) {
  const int lane = threadIdx.x;
  uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = (int)(lid % (uint32_t)g.ngroups);
  lid /= (uint32_t)g.ngroups;
  const int64_t b = (int64_t)(lid % (uint32_t)g.batch);
  const int s = (int)(lid / (uint32_t)g.batch);
  const int64_t d0 = (int64_t)grp * 64;
  const int64_t dc = min(d0 + lane, g.D - 1);  // lanes past D-1 mirror channel D-1
  const int loff = (int)(dc - d0);
  const int64_t tbeg = (int64_t)s * g.seg_len;
  const int len = (int)(min(tbeg + g.seg_len, g.L) - tbeg);

  constexpr int ES = BF16 ? 2 : 4;
  float wk[W];
#pragma unroll
  for (int k = 0; k < W; ++k) wk[k] = w[dc * W + k];
  const float bv = bias != nullptr ? bias[dc] : 0.0f;

  const int64_t row0 = (b * g.L + tbeg) * g.D + d0;
  const __amdgpu_buffer_rsrc_t rx = conv_rsrc((const char*)x + row0 * ES);
  const __amdgpu_buffer_rsrc_t ro = conv_rsrc((char*)out + row0 * ES);
  const int vo = loff * ES;
  const int rs = (int)(g.D * ES);
  constexpr int kNT = 2;  // non-temporal
  auto ld = [&](int soff) -> float {
    if (BF16) return __builtin_bit_cast(float, (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rx, vo, soff, kNT) << 16);
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, vo, soff, kNT));
  };

  // window[k] = x at step t-(W-1)+k for the step being produced; the W-1 inputs before the
  // segment come from the previous segment (zero before t = 0)
  float win[W];
#pragma unroll
  for (int k = 0; k < W - 1; ++k) {
    const int64_t tg = tbeg - (W - 1) + k;
    float v = 0.0f;
    if (tg >= 0) {
      const int64_t e = ((b * g.L + tg) * g.D + dc);
      v = BF16 ? __builtin_bit_cast(float, (uint32_t) static_cast<const uint16_t*>(x)[e] << 16)
               : static_cast<const float*>(x)[e];
    }
    win[k] = v;
  }

  float q[2][kConvU];
#define CONV_LOAD(SLOT, T0)                                                                \
  do {                                                                                     \
    _Pragma("unroll") for (int i_ = 0; i_ < kConvU; ++i_) q[SLOT][i_] = ld(min((T0) + i_, len - 1) * rs); \
  } while (0)
#define CONV_STEP(SLOT, I, T)                                                              \
  do {                                                                                     \
    win[W - 1] = q[SLOT][I];                                                               \
    float v_ = bv;                                                                         \
    _Pragma("unroll") for (int k = 0; k < W; ++k) v_ = __builtin_fmaf(wk[k], win[k], v_);  \
    if (SILU) v_ = silu(v_);                                                               \
    if (BF16) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)bf16_rne(v_), ro, vo, (T) * rs, kNT); \
    else __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v_), ro, vo, (T) * rs, kNT); \
    _Pragma("unroll") for (int k = 0; k < W - 1; ++k) win[k] = win[k + 1];                 \
  } while (0)

  CONV_LOAD(0, 0);
  int t0 = 0;
  for (; t0 + 2 * kConvU <= len; t0 += 2 * kConvU) {
    CONV_LOAD(1, t0 + kConvU);
#pragma unroll
    for (int i = 0; i < kConvU; ++i) CONV_STEP(0, i, t0 + i);
    CONV_LOAD(0, t0 + 2 * kConvU);
#pragma unroll
    for (int i = 0; i < kConvU; ++i) CONV_STEP(1, i, t0 + kConvU + i);
  }
  if (t0 < len) {  // ragged tail: slot 0 holds steps t0 .. t0+kConvU-1
    CONV_LOAD(1, t0 + kConvU);
    for (int i = 0; i < kConvU && t0 + i < len; ++i) CONV_STEP(0, i, t0 + i);
    for (int i = 0; i < kConvU && t0 + kConvU + i < len; ++i) CONV_STEP(1, i, t0 + kConvU + i);
  }
#undef CONV_LOAD
#undef CONV_STEP
}

ConvPlan plan_conv1d(int64_t batch, int64_t seqlen, int64_t dim, int num_cus) {
  ConvPlan pl{};
  const int64_t waves = batch * ((dim + 63) / 64);
  // streaming only 2-4 bytes per lane and step: many short-lived waves keep enough loads in
  // flight (measured on the 1 x 65536 x 5120 bf16 layer: 13 segments 2.8 TB/s, 128 4.4 TB/s,
  // 512 4.9 TB/s, 1024 4.7 TB/s) -- aim at about 160 waves of work per CU
  const int64_t target = (int64_t)std::max(num_cus, 1) * 160;
  int64_t S = waves >= target ? 1 : (target + waves - 1) / waves;
  S = std::min<int64_t>(S, std::max<int64_t>(1, seqlen / (4 * kConvU)));  // segments of >= 64 steps
  const int forced = env_int("SSS_FORCE_SEGMENTS", 0);
  if (forced > 0) S = std::min<int64_t>(forced, seqlen);
  // buffer offsets inside a segment stay below 2^30 bytes (dim <= 2^24 is checked)
  const int64_t max_len = std::max<int64_t>(1, ((int64_t)1 << 30) / (dim * 4));
  int64_t seg_len = std::min((seqlen + S - 1) / S, max_len);
  pl.segments = (int)((seqlen + seg_len - 1) / seg_len);
  pl.seg_len = seg_len;
  return pl;
}

template <int W, bool BF16>
static hipError_t run_conv(const ConvArgs& a, const ConvPlan& pl, hipStream_t stream) {
  ConvSeg g{};
  g.batch = a.batch;
  g.L = a.seqlen;
  g.D = a.dim;
  g.seg_len = pl.seg_len;
  g.ngroups = (int)((a.dim + 63) / 64);
  const dim3 grid((unsigned)((int64_t)g.ngroups * a.batch * pl.segments)), block(64);
  if (a.silu)
    hipLaunchKernelGGL((conv1d_kernel<W, BF16, true>), grid, block, 0, stream, a.x, a.w, a.bias, a.out, g);
  else
    hipLaunchKernelGGL((conv1d_kernel<W, BF16, false>), grid, block, 0, stream, a.x, a.w, a.bias, a.out, g);
  return hipGetLastError();
}

template <bool BF16>
static hipError_t dispatch_conv(const ConvArgs& a, const ConvPlan& pl, hipStream_t stream) {
  switch (a.width) {
    case 1: return run_conv<1, BF16>(a, pl, stream);
    case 2: return run_conv<2, BF16>(a, pl, stream);
    case 3: return run_conv<3, BF16>(a, pl, stream);
    case 4: return run_conv<4, BF16>(a, pl, stream);
    case 5: return run_conv<5, BF16>(a, pl, stream);
    case 6: return run_conv<6, BF16>(a, pl, stream);
    case 7: return run_conv<7, BF16>(a, pl, stream);
    case 8: return run_conv<8, BF16>(a, pl, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_conv1d(const ConvArgs& a, const ConvPlan& pl, hipStream_t stream) {
  return a.bf16 ? dispatch_conv<true>(a, pl, stream) : dispatch_conv<false>(a, pl, stream);
}

}  // namespace sss
