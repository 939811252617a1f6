// elementwise_scan.hip -- gfx950 kernels for the per-channel elementwise scan of
// "15. Selective (Data-Dependent) SSM Scan" (Reference solution):
//   h = A_t*h + B_t*x_t,  y_t = C_t*h  (read-out from the updated state), h_{-1} = h0.
//
// The operation is pure streaming (20 bytes per step, 3 flops), so the design is about HBM:
// one lane per channel walks its steps in order, neighbouring lanes are neighbouring
// channels (every load and store of a wave is one contiguous 256-byte row segment), and
// each lane keeps two batches of U steps of loads in flight (software double buffering)
// so that enough bytes are outstanding to cover HBM latency.  When there are too few
// channels to fill the GPU, time is split into S segments: pass 1 folds each segment into
// its affine pair (prod A, state from zero), a carry kernel composes the pairs in order
// from h0 ("Scan bien recurrence ..." of "Selective Scan trong Mamba toi uu chuoi dai the
// nao?": the pair compose rule), and pass 2 replays every segment from its entering state.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace sss {

struct EwParams {
  const float* x;
  const float* A;
  const float* B;
  const float* C;
  const float* h0;
  float* y;
  float* h_last;
  float* seg_a;  // [S][batch*dim]: product of A over each segment
  float* seg_b;  // [S][batch*dim]: end state from zero; after the carry, the entering state
  int64_t batch, L, D, seg_len;
  int S, ngroups;  // ngroups = ceil(D / 64) channel groups per batch
};

#ifndef EW_STEPS_PER_BATCH
#define EW_STEPS_PER_BATCH 16
#endif
constexpr int kU = EW_STEPS_PER_BATCH;  // steps per load batch (two batches in flight)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t ew_rsrc(const float* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, 0x7FFFFFFF, 0x00020000);
}

// One wave = 64 consecutive channels d0..d0+63 of one batch over one time segment; lane l
// owns channel d0+l (lanes past D-1 mirror channel D-1 and store equal values).  All loads
// and stores are buffer operations on descriptors based at the wave's first row of the
// segment with a wave-uniform step offset, so a step of one array is one 256-byte row piece.
// PASS 1 (segments 0..S-2): seg_a/seg_b = (prod A, end state from zero) of the segment.
// PASS 2 (all segments): entering state from seg_b (S > 1) or h0, then y (and h_last).
template <int PASS>
__global__ __launch_bounds__(64, 1) void ew_scan_kernel(EwParams p) {
  const int lane = threadIdx.x;
  uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = (int)(lid % (uint32_t)p.ngroups);
  lid /= (uint32_t)p.ngroups;
  const int64_t b = (int64_t)(lid % (uint32_t)p.batch);
  const int s = (int)(lid / (uint32_t)p.batch);
  const int64_t d0 = (int64_t)grp * 64;
  const int64_t dc = min(d0 + lane, p.D - 1);
  const int loff = (int)(dc - d0);
  const int64_t ch = b * p.D + dc;
  const int64_t nch = p.batch * p.D;
  const int64_t tbeg = (int64_t)s * p.seg_len;
  const int len = (int)(min(tbeg + p.seg_len, p.L) - tbeg);  // < 2^28 (plan)

  float h = 0.0f, aprod = 1.0f;
  if (PASS == 2) h = p.S > 1 ? p.seg_b[(int64_t)s * nch + ch] : (p.h0 ? p.h0[ch] : 0.0f);

  const int64_t row0 = (b * p.L + tbeg) * p.D + d0;
  const __amdgpu_buffer_rsrc_t rx = ew_rsrc(p.x + row0), ra = ew_rsrc(p.A + row0), rb = ew_rsrc(p.B + row0);
  const __amdgpu_buffer_rsrc_t rc = ew_rsrc(PASS == 2 ? p.C + row0 : p.x + row0);
  const __amdgpu_buffer_rsrc_t ry = ew_rsrc(PASS == 2 ? p.y + row0 : p.x + row0);
  const int vo = loff * 4;
  const int rs = (int)(p.D * 4);  // bytes between steps
  constexpr int kNT = 2;          // non-temporal: every value is used once

  float qa[2][kU], qb[2][kU], qx[2][kU], qc[2][kU];
#define EW_LOAD(SLOT, T0)                                                                        \
  do {                                                                                           \
    _Pragma("unroll") for (int i_ = 0; i_ < kU; ++i_) {                                          \
      const int so_ = min((T0) + i_, len - 1) * rs; /* clamped: tail values are not used */     \
      qa[SLOT][i_] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, vo, so_, kNT)); \
      qb[SLOT][i_] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, vo, so_, kNT)); \
      qx[SLOT][i_] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, vo, so_, kNT)); \
      if (PASS == 2)                                                                             \
        qc[SLOT][i_] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rc, vo, so_, kNT)); \
    }                                                                                            \
  } while (0)
#define EW_STEP(SLOT, I, T)                                                                      \
  do {                                                                                           \
    h = __builtin_fmaf(qa[SLOT][I], h, qb[SLOT][I] * qx[SLOT][I]);                               \
    if (PASS == 1) aprod *= qa[SLOT][I];                                                         \
    else __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, qc[SLOT][I] * h), ry, vo, (T) * rs, kNT); \
  } while (0)

  EW_LOAD(0, 0);
  int t0 = 0;
  for (; t0 + 2 * kU <= len; t0 += 2 * kU) {
    EW_LOAD(1, t0 + kU);
#pragma unroll
    for (int i = 0; i < kU; ++i) EW_STEP(0, i, t0 + i);
    EW_LOAD(0, t0 + 2 * kU);
#pragma unroll
    for (int i = 0; i < kU; ++i) EW_STEP(1, i, t0 + kU + i);
  }
  if (t0 < len) {  // ragged tail (< 2 kU steps): slot 0 holds steps t0 .. t0+kU-1
    EW_LOAD(1, t0 + kU);
    for (int i = 0; i < kU && t0 + i < len; ++i) EW_STEP(0, i, t0 + i);
    for (int i = 0; i < kU && t0 + kU + i < len; ++i) EW_STEP(1, i, t0 + kU + i);
  }
#undef EW_LOAD
#undef EW_STEP

  if (PASS == 1) {
    p.seg_a[(int64_t)s * nch + ch] = aprod;
    p.seg_b[(int64_t)s * nch + ch] = h;
  } else if (p.h_last != nullptr && s == p.S - 1) {
    p.h_last[ch] = h;
  }
}

// In place over the segment pairs, one thread per channel: seg_b[s] := state entering
// segment s (h0 for s = 0, then A-product * state + end state of the previous segment).
__global__ __launch_bounds__(256) void ew_carry_kernel(EwParams p) {
  const int64_t nch = p.batch * p.D;
  const int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (ch >= nch) return;
  float h = p.h0 ? p.h0[ch] : 0.0f;
  for (int s = 0; s < p.S; ++s) {
    const int64_t o = (int64_t)s * nch + ch;
    const float a = s + 1 < p.S ? p.seg_a[o] : 0.0f;
    const float bb = s + 1 < p.S ? p.seg_b[o] : 0.0f;
    p.seg_b[o] = h;
    h = __builtin_fmaf(a, h, bb);
  }
}

static size_t align_up_ew(size_t v, size_t a) { return (v + a - 1) / a * a; }

EwPlan plan_elementwise(int64_t batch, int64_t seqlen, int64_t dim, int num_cus) {
  EwPlan pl{};
  const int64_t waves = batch * ((dim + 63) / 64);
  // Streaming: one wave per CU with two batches of loads in flight already covers HBM
  // latency; only when there are fewer channel groups than CUs is time split, and then
  // into enough segments for about one wave per SIMD.
  const int64_t cus = std::max(num_cus, 1);
  int64_t S = 1;
  if (waves < cus) S = (4 * cus + waves - 1) / waves;
  const int64_t max_seg = std::max<int64_t>(1, seqlen / (2 * kU));  // segments of >= 2 batches
  S = std::min<int64_t>(S, max_seg);
  S = std::min<int64_t>(S, 1024);
  const int forced = env_int("SSS_FORCE_SEGMENTS", 0);
  if (forced > 0) S = std::min<int64_t>(forced, seqlen);
  if (S < 1) S = 1;
  // buffer offsets inside a segment stay below 2^30 bytes (dim is capped by the caller)
  const int64_t max_len = std::max<int64_t>(1, ((int64_t)1 << 30) / (dim * 4));
  int64_t seg_len = std::min((seqlen + S - 1) / S, max_len);
  S = (seqlen + seg_len - 1) / seg_len;
  pl.segments = (int)S;
  pl.seg_len = seg_len;
  pl.ws_total = S > 1 ? align_up_ew((size_t)S * batch * dim * 4, 256) * 2 : 0;
  return pl;
}

hipError_t launch_elementwise(const EwArgs& a, const EwPlan& pl, hipStream_t stream) {
  EwParams p{};
  p.x = a.x;
  p.A = a.A;
  p.B = a.B;
  p.C = a.C;
  p.h0 = a.h0;
  p.y = a.y;
  p.h_last = a.h_last;
  p.batch = a.batch;
  p.L = a.seqlen;
  p.D = a.dim;
  p.seg_len = pl.seg_len;
  p.S = pl.segments;
  p.ngroups = (int)((a.dim + 63) / 64);
  const int64_t per_seg = (int64_t)p.ngroups * a.batch;
  if (pl.segments > 1) {
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    p.seg_a = reinterpret_cast<float*>(ws);
    p.seg_b = reinterpret_cast<float*>(ws + pl.ws_total / 2);
    hipLaunchKernelGGL(ew_scan_kernel<1>, dim3((unsigned)(per_seg * (pl.segments - 1))), dim3(64), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nch = a.batch * a.dim;
    hipLaunchKernelGGL(ew_carry_kernel, dim3((unsigned)((nch + 255) / 256)), dim3(256), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(ew_scan_kernel<2>, dim3((unsigned)(per_seg * pl.segments)), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sss
