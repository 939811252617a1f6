// conv1d.hip -- gfx950 kernel for the causal depthwise convolution in front of the scan.
//
// The Mamba block runs x through a short causal depthwise convolution (and silu) before
// the selective scan ("Toan Canh Tien Hoa Kien Truc AI ...", section "5.3. Toi uu hoa
// Kernel Fusion cho Mamba SSM", which names the causal_conv1d kernel):
//   out[b,t,d] = bias[d] + sum_{k<W} w[d,k] * x[b, t-(W-1)+k, d]   (x = 0 before t = 0),
//   then optionally silu.
// It is pure streaming (2 + 2 bytes per element in bf16, W fmas).  Each lane owns a few
// adjacent channels -- 8 bytes of a row, 4 channels in bf16 and 2 in fp32, when dim splits
// evenly, else one -- so that every load and store of a wave is one 512-byte row piece
// through a buffer descriptor with a wave-uniform step offset (128-byte pieces, one bf16
// channel per lane, streamed at 2.9 TB/s here against 5.0 TB/s for 512-byte pieces); two
// batches of steps are in flight, and the last W-1 inputs of each channel stay in
// registers as a sliding window.  bf16 results are rounded by the hardware conversion.
// Time is cut into segments for parallelism; a segment starts by reading the W-1 inputs
// before it.  On a chip where the scan itself is bound by transcendental issue, a separate
// streaming pass costs about what fusing it into both scan passes would add there, and
// keeps the scan kernels unchanged.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace sss {

struct ConvSeg {
  int64_t batch, L, D, seg_len;
  int ngroups;  // ceil(D / (64 * channels per lane))
};

constexpr int kConvU = 8;  // steps per load batch

__device__ __forceinline__ __amdgpu_buffer_rsrc_t conv_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}

typedef __bf16 conv_bf2 __attribute__((ext_vector_type(2)));
typedef float conv_f2 __attribute__((ext_vector_type(2)));

// two fp32 -> two bf16 in one dword (low half = a), rounded to nearest even by the
// hardware conversion (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  const conv_f2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, conv_bf2));
}

typedef uint32_t conv_u2 __attribute__((ext_vector_type(2)));

// The CPL adjacent channels of one lane, as raw dwords: CPL elements of ES bytes each
// (CPL * ES is 2, 4 or 8 bytes; below 4 the element sits in the low half of dword 0).
template <bool BF16, int CPL>
struct ConvRaw {
  static constexpr int ES = BF16 ? 2 : 4;
  static constexpr int VB = CPL * ES;  // bytes per lane and step
  static constexpr int ND = VB >= 4 ? VB / 4 : 1;
  uint32_t w[ND];

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int vo, int so) {
    if constexpr (VB == 8) {
      const conv_u2 v = __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, 2);
      w[0] = v.x;
      w[1] = v.y;
    } else if constexpr (VB == 4) {
      w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 2);
    } else {
      w[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, vo, so, 2);
    }
  }
  // element c (0 <= c < CPL) widened to fp32
  __device__ __forceinline__ float get(int c) const {
    if constexpr (BF16) {
      const uint32_t d = w[c >> 1];
      return __builtin_bit_cast(float, (c & 1) ? (d & 0xFFFF0000u) : (d << 16));
    } else {
      return __builtin_bit_cast(float, w[c]);
    }
  }
};

template <bool BF16, int CPL>
__device__ __forceinline__ void conv_store(const float* v, __amdgpu_buffer_rsrc_t r, int vo, int so) {
  constexpr int VB = CPL * (BF16 ? 2 : 4);
  uint32_t o[VB >= 4 ? VB / 4 : 1];
  if constexpr (BF16) {
    if constexpr (CPL == 1) {
      o[0] = bf16_pair(v[0], 0.0f) & 0xFFFFu;
    } else {
#pragma unroll
      for (int c = 0; c < CPL; c += 2) o[c >> 1] = bf16_pair(v[c], v[c + 1]);
    }
  } else {
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[c] = __builtin_bit_cast(uint32_t, v[c]);
  }
  if constexpr (VB == 8) {
    const conv_u2 q = {o[0], o[1]};
    __builtin_amdgcn_raw_buffer_store_b64(q, r, vo, so, 2);
  } else if constexpr (VB == 4) {
    __builtin_amdgcn_raw_buffer_store_b32(o[0], r, vo, so, 2);
  } else {
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)o[0], r, vo, so, 2);
  }
}

// One wave = 64 lanes x CPL adjacent channels of one batch row and one time segment.  With
// CPL > 1 (dim a multiple of CPL) every lane moves 8 bytes per tensor and step, so each
// wave-wide load or store is one contiguous 512-byte row piece.
template <int W, bool BF16, bool SILU, int CPL>
__global__ __launch_bounds__(64) void conv1d_kernel(const void* __restrict__ x, const float* __restrict__ w,
                                                    const float* __restrict__ bias, void* __restrict__ out,
                                                    ConvSeg g) {
  const int lane = threadIdx.x;
  uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = (int)(lid % (uint32_t)g.ngroups);
  lid /= (uint32_t)g.ngroups;
  const int64_t b = (int64_t)(lid % (uint32_t)g.batch);
  const int s = (int)(lid / (uint32_t)g.batch);
  const int64_t d0 = (int64_t)grp * 64 * CPL;
  // lanes past the row's end mirror the last CPL channels (equal values, duplicate stores)
  const int64_t dc = min(d0 + (int64_t)lane * CPL, g.D - CPL);
  const int loff = (int)(dc - d0);
  const int64_t tbeg = (int64_t)s * g.seg_len;
  const int len = (int)(min(tbeg + g.seg_len, g.L) - tbeg);

  constexpr int ES = BF16 ? 2 : 4;
  float wk[CPL][W], bv[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
#pragma unroll
    for (int k = 0; k < W; ++k) wk[c][k] = w[(dc + c) * W + k];
    bv[c] = bias != nullptr ? bias[dc + c] : 0.0f;
  }

  const int64_t row0 = (b * g.L + tbeg) * g.D + d0;
  const __amdgpu_buffer_rsrc_t rx = conv_rsrc((const char*)x + row0 * ES);
  const __amdgpu_buffer_rsrc_t ro = conv_rsrc((char*)out + row0 * ES);
  const int vo = loff * ES;
  const int rs = (int)(g.D * ES);

  // win[c][k] = x at step t-(W-1)+k of channel dc+c for the step being produced; the W-1
  // inputs before the segment come from the previous segment (zero before t = 0)
  float win[CPL][W];
#pragma unroll
  for (int k = 0; k < W - 1; ++k) {
    const int64_t tg = tbeg - (W - 1) + k;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float v = 0.0f;
      if (tg >= 0) {
        const int64_t e = (b * g.L + tg) * g.D + dc + c;
        v = BF16 ? __builtin_bit_cast(float, (uint32_t) static_cast<const uint16_t*>(x)[e] << 16)
                 : static_cast<const float*>(x)[e];
      }
      win[c][k] = v;
    }
  }

  ConvRaw<BF16, CPL> q[2][kConvU];
#define CONV_LOAD(SLOT, T0)                                                                \
  do {                                                                                     \
    _Pragma("unroll") for (int i_ = 0; i_ < kConvU; ++i_) q[SLOT][i_].load(rx, vo, min((T0) + i_, len - 1) * rs); \
  } while (0)
#define CONV_STEP(SLOT, I, T)                                                              \
  do {                                                                                     \
    float o_[CPL];                                                                         \
    _Pragma("unroll") for (int c = 0; c < CPL; ++c) {                                      \
      win[c][W - 1] = q[SLOT][I].get(c);                                                   \
      float v_ = bv[c];                                                                    \
      _Pragma("unroll") for (int k = 0; k < W; ++k) v_ = __builtin_fmaf(wk[c][k], win[c][k], v_); \
      o_[c] = SILU ? silu(v_) : v_;                                                        \
      _Pragma("unroll") for (int k = 0; k < W - 1; ++k) win[c][k] = win[c][k + 1];         \
    }                                                                                      \
    conv_store<BF16, CPL>(o_, ro, vo, (T) * rs);                                           \
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

// channels per lane: 8 bytes per lane and step where the row splits evenly, else one
int conv_channels_per_lane(int64_t dim, bool bf16) {
  const int cpl = bf16 ? 4 : 2;
  return dim % cpl == 0 ? cpl : 1;
}

ConvPlan plan_conv1d(int64_t batch, int64_t seqlen, int64_t dim, bool bf16, int num_cus) {
  ConvPlan pl{};
  const int cpl = conv_channels_per_lane(dim, bf16);
  const int64_t waves = batch * ((dim + 64 * cpl - 1) / (64 * cpl));
  // pure streaming: many short-lived waves keep every CU's loads in flight to the end
  // (measured on the 1 x 65536 x 5120 bf16 layer, 4 channels per lane: 10 waves per CU
  // 0.290 ms, 20 0.279, 40 0.275, 80 0.270, 160 0.269, 320 0.270)
  const int64_t target = (int64_t)std::max(num_cus, 1) * env_int("SSS_CONV_WAVES_PER_CU", 80);
  int64_t S = waves >= target ? 1 : (target + waves - 1) / waves;
  S = std::min<int64_t>(S, std::max<int64_t>(1, seqlen / (4 * kConvU)));  // segments of >= 32 steps
  const int forced = env_int("SSS_FORCE_SEGMENTS", 0);
  if (forced > 0) S = std::min<int64_t>(forced, seqlen);
  // buffer offsets inside a segment stay below 2^30 bytes (dim <= 2^24 is checked)
  const int64_t max_len = std::max<int64_t>(1, ((int64_t)1 << 30) / (dim * 4));
  int64_t seg_len = std::min((seqlen + S - 1) / S, max_len);
  pl.segments = (int)((seqlen + seg_len - 1) / seg_len);
  pl.seg_len = seg_len;
  pl.cpl = cpl;
  return pl;
}

template <int W, bool BF16, int CPL>
static hipError_t run_conv_cpl(const ConvArgs& a, const ConvPlan& pl, hipStream_t stream) {
  ConvSeg g{};
  g.batch = a.batch;
  g.L = a.seqlen;
  g.D = a.dim;
  g.seg_len = pl.seg_len;
  g.ngroups = (int)((a.dim + 64 * CPL - 1) / (64 * CPL));
  const dim3 grid((unsigned)((int64_t)g.ngroups * a.batch * pl.segments)), block(64);
  if (a.silu)
    hipLaunchKernelGGL((conv1d_kernel<W, BF16, true, CPL>), grid, block, 0, stream, a.x, a.w, a.bias, a.out, g);
  else
    hipLaunchKernelGGL((conv1d_kernel<W, BF16, false, CPL>), grid, block, 0, stream, a.x, a.w, a.bias, a.out, g);
  return hipGetLastError();
}

template <int W, bool BF16>
static hipError_t run_conv(const ConvArgs& a, const ConvPlan& pl, hipStream_t stream) {
  constexpr int kWide = BF16 ? 4 : 2;
  if (pl.cpl == kWide) return run_conv_cpl<W, BF16, kWide>(a, pl, stream);
  if (pl.cpl == 1) return run_conv_cpl<W, BF16, 1>(a, pl, stream);
  return hipErrorInvalidValue;
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
