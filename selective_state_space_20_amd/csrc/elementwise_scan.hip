// elementwise_scan.hip -- gfx950 kernels for the per-channel elementwise scan of
// "15. Selective (Data-Dependent) SSM Scan" (Reference solution):
//   h = A_t*h + B_t*x_t,  y_t = C_t*h  (read-out from the updated state), h_{-1} = h0.
//
// The operation is pure streaming (20 bytes per step, 3 flops), so the design is about HBM:
// each lane walks its channels' steps in order, neighbouring lanes own neighbouring
// channels (two per lane where dim is even: every load and store of a wave is one
// contiguous 512-byte row segment), and each lane keeps two batches of U steps of loads in
// flight (software double buffering) so that enough bytes are outstanding to cover HBM
// latency.  When there are too few
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

// Steps per load batch (two batches in flight): 16 steps of 4 bytes per lane and array, or
// fewer steps of wider pieces, keep the queue at 128 VGPRs.
template <int CPL>
constexpr int ew_steps_per_batch() { return 16 / CPL; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t ew_rsrc(const float* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, 0x7FFFFFFF, 0x00020000);
}

typedef uint32_t ew_u2 __attribute__((ext_vector_type(2)));
typedef uint32_t ew_u4 __attribute__((ext_vector_type(4)));
constexpr int kEwNT = 2;  // non-temporal: every value is used once

// bits -> float through a by-value argument: __builtin_bit_cast applied directly to an
// element of an ext_vector (q.y, q.z, ...) has been compiled as a cast of element 0
__device__ __forceinline__ float ew_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t ew_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

// CPL adjacent fp32 channels of one lane: one 4-, 8- or 16-byte buffer access
template <int CPL>
__device__ __forceinline__ void ew_load(float (&v)[CPL], __amdgpu_buffer_rsrc_t r, int vo, int so) {
  if constexpr (CPL == 4) {
    const ew_u4 q = __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, kEwNT);
    v[0] = ew_f32(q.x);
    v[1] = ew_f32(q.y);
    v[2] = ew_f32(q.z);
    v[3] = ew_f32(q.w);
  } else if constexpr (CPL == 2) {
    const ew_u2 q = __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, kEwNT);
    v[0] = ew_f32(q.x);
    v[1] = ew_f32(q.y);
  } else {
    v[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, vo, so, kEwNT));
  }
}

template <int CPL>
__device__ __forceinline__ void ew_store(const float (&v)[CPL], __amdgpu_buffer_rsrc_t r, int vo, int so) {
  if constexpr (CPL == 4) {
    const ew_u4 q = {ew_u32(v[0]), ew_u32(v[1]),
                     ew_u32(v[2]), ew_u32(v[3])};
    __builtin_amdgcn_raw_buffer_store_b128(q, r, vo, so, kEwNT);
  } else if constexpr (CPL == 2) {
    const ew_u2 q = {ew_u32(v[0]), ew_u32(v[1])};
    __builtin_amdgcn_raw_buffer_store_b64(q, r, vo, so, kEwNT);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(ew_u32(v[0]), r, vo, so, kEwNT);
  }
}

// One wave = 64 lanes x CPL consecutive channels of one batch over one time segment; lane l
// owns channels d0+l*CPL .. +CPL-1 (lanes past the row's end mirror its last CPL channels
// and store equal values; CPL > 1 only where dim is a multiple of CPL).  All loads and
// stores are buffer operations on descriptors based at the wave's first row of the segment
// with a wave-uniform step offset, so a step of one array is one 256*CPL-byte row piece.
// PASS 1 (segments 0..S-2): seg_a/seg_b = (prod A, end state from zero) of the segment.
// PASS 2 (all segments): entering state from seg_b (S > 1) or h0, then y (and h_last).
template <int PASS, int CPL>
__global__ __launch_bounds__(64, 1) void ew_scan_kernel(EwParams p) {
  constexpr int kU = ew_steps_per_batch<CPL>();
  const int lane = threadIdx.x;
  uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = (int)(lid % (uint32_t)p.ngroups);
  lid /= (uint32_t)p.ngroups;
  const int64_t b = (int64_t)(lid % (uint32_t)p.batch);
  const int s = (int)(lid / (uint32_t)p.batch);
  const int64_t d0 = (int64_t)grp * 64 * CPL;
  const int64_t dc = min(d0 + (int64_t)lane * CPL, p.D - CPL);
  const int loff = (int)(dc - d0);
  const int64_t ch = b * p.D + dc;
  const int64_t nch = p.batch * p.D;
  const int64_t tbeg = (int64_t)s * p.seg_len;
  const int len = (int)(min(tbeg + p.seg_len, p.L) - tbeg);  // < 2^28 (plan)

  float h[CPL], aprod[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    h[c] = 0.0f;
    aprod[c] = 1.0f;
    if (PASS == 2) h[c] = p.S > 1 ? p.seg_b[(int64_t)s * nch + ch + c] : (p.h0 ? p.h0[ch + c] : 0.0f);
  }

  const int64_t row0 = (b * p.L + tbeg) * p.D + d0;
  const __amdgpu_buffer_rsrc_t rx = ew_rsrc(p.x + row0), ra = ew_rsrc(p.A + row0), rb = ew_rsrc(p.B + row0);
  const __amdgpu_buffer_rsrc_t rc = ew_rsrc(PASS == 2 ? p.C + row0 : p.x + row0);
  const __amdgpu_buffer_rsrc_t ry = ew_rsrc(PASS == 2 ? p.y + row0 : p.x + row0);
  const int vo = loff * 4;
  const int rs = (int)(p.D * 4);  // bytes between steps

  float qa[2][kU][CPL], qb[2][kU][CPL], qx[2][kU][CPL], qc[2][kU][CPL];
#define EW_LOAD(SLOT, T0)                                                                        \
  do {                                                                                           \
    _Pragma("unroll") for (int i_ = 0; i_ < kU; ++i_) {                                          \
      const int so_ = min((T0) + i_, len - 1) * rs; /* clamped: tail values are not used */     \
      ew_load<CPL>(qa[SLOT][i_], ra, vo, so_);                                                   \
      ew_load<CPL>(qb[SLOT][i_], rb, vo, so_);                                                   \
      ew_load<CPL>(qx[SLOT][i_], rx, vo, so_);                                                   \
      if (PASS == 2) ew_load<CPL>(qc[SLOT][i_], rc, vo, so_);                                    \
    }                                                                                            \
  } while (0)
#define EW_STEP(SLOT, I, T)                                                                      \
  do {                                                                                           \
    float o_[CPL];                                                                               \
    _Pragma("unroll") for (int c = 0; c < CPL; ++c) {                                            \
      h[c] = __builtin_fmaf(qa[SLOT][I][c], h[c], qb[SLOT][I][c] * qx[SLOT][I][c]);              \
      if (PASS == 1) aprod[c] *= qa[SLOT][I][c];                                                 \
      else o_[c] = qc[SLOT][I][c] * h[c];                                                        \
    }                                                                                            \
    if (PASS == 2) ew_store<CPL>(o_, ry, vo, (T) * rs);                                          \
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
#pragma unroll
    for (int i = 0; i < kU; ++i)
      if (t0 + i < len) EW_STEP(0, i, t0 + i);
#pragma unroll
    for (int i = 0; i < kU; ++i)
      if (t0 + kU + i < len) EW_STEP(1, i, t0 + kU + i);
  }
#undef EW_LOAD
#undef EW_STEP

#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    if (PASS == 1) {
      p.seg_a[(int64_t)s * nch + ch + c] = aprod[c];
      p.seg_b[(int64_t)s * nch + ch + c] = h[c];
    } else if (p.h_last != nullptr && s == p.S - 1) {
      p.h_last[ch + c] = h[c];
    }
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
  // two adjacent channels per lane (512-byte row pieces per wave) where dim is even:
  // 8 x 32768 x 4096 runs in 3.65 ms against 4.09 ms with one channel (256-byte pieces)
  int cpl = env_int("SSS_EW_CPL", 2);
  if (cpl != 1 && cpl != 2 && cpl != 4) cpl = 1;
  if (dim % cpl != 0) cpl = 1;
  pl.cpl = cpl;
  const int kU = 16 / cpl;
  const int64_t waves = batch * ((dim + 64 * cpl - 1) / (64 * cpl));
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

template <int CPL>
static hipError_t run_elementwise(EwParams& p, const EwArgs& a, const EwPlan& pl, hipStream_t stream) {
  const int64_t per_seg = (int64_t)p.ngroups * a.batch;
  if (pl.segments > 1) {
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    p.seg_a = reinterpret_cast<float*>(ws);
    p.seg_b = reinterpret_cast<float*>(ws + pl.ws_total / 2);
    hipLaunchKernelGGL((ew_scan_kernel<1, CPL>), dim3((unsigned)(per_seg * (pl.segments - 1))), dim3(64), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nch = a.batch * a.dim;
    hipLaunchKernelGGL(ew_carry_kernel, dim3((unsigned)((nch + 255) / 256)), dim3(256), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((ew_scan_kernel<2, CPL>), dim3((unsigned)(per_seg * pl.segments)), dim3(64), 0, stream, p);
  return hipGetLastError();
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
  p.ngroups = (int)((a.dim + 64 * pl.cpl - 1) / (64 * pl.cpl));
  switch (pl.cpl) {
    case 4: return run_elementwise<4>(p, a, pl, stream);
    case 2: return run_elementwise<2>(p, a, pl, stream);
    case 1: return run_elementwise<1>(p, a, pl, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sss
