// selective_scan.hip -- gfx950 kernels for the selective (Mamba) scan.
//
// Computes, per batch b, channel d, state n (see include/sss.h):
//   Abar_t = exp(delta_t*A[d,n]),  h_t = Abar_t*h_{t-1} + delta_t*B_t[n]*x_t,
//   y_t = (sum_n C_t[n]*h_t[n] + D[d]*x_t) * silu(z_t)
// The recurrence is the selective SSM of "Selective Scan trong Mamba toi uu chuoi dai the
// nao?" (sections "Tai sao Mamba can Selective Scan?", "Selection pha vo convolution
// kernel co dinh"); the (B,L,D,N) state never leaves registers (sections "Tai sao chi
// parallel scan van chua du nhanh?" and "Kernel fusion").
//
// Mapping, chosen from measurements on MI355X (row-major (B,L,D) inputs only stream at HBM
// speed when each request covers >= 128 contiguous bytes of a row; exp issues at a quarter
// of the fp32 rate and shares the VALU with everything else):
//   * one wave = 64 consecutive channels of one batch: every load of x/delta/z and every
//     store of y is one contiguous 128-/256-byte row segment;
//   * B_t and C_t are the same for all 64 lanes, so they are read with scalar loads into
//     SGPRs and used directly as VALU operands (no LDS, no per-lane copies);
//   * each lane walks time in order with its N states in registers: per step and state
//     one exp (v_exp_f32 of delta*A*log2e), delta*x*B, the state fma and the C*h fma;
//   * time is split into S segments so that long sequences over few channels still fill
//     the GPU.  Affine steps compose associatively ("Scan bien recurrence thanh phep toan
//     co the song song hoa ra sao?": (a2,b2)(x)(a1,b1) = (a2*a1, a2*b1 + b2)), so
//       pass 1 folds each segment (but the last) into its pair (exp2(A' * sum delta), end
//              state from zero),
//       carry  composes the pairs in order from h0 into the state entering each segment,
//       pass 2 replays every segment from its entering state and writes y (and h_last).
//     With S = 1 only pass 2 runs, from h0.
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <type_traits>

namespace sss {

constexpr int kStepsPerBatch = 2;  // time steps whose x/delta/z loads are issued together
// register budget: at least this many resident waves per SIMD (512 VGPRs / waves each);
// 32 and 64 states need the larger budgets to stay spill-free
constexpr int min_waves_per_simd(int ns) { return ns >= 64 ? 1 : ns >= 32 ? 3 : 4; }
constexpr int kStreamPolicy = 2;    // buffer cache policy of streamed x/delta/z/y: non-temporal

// Raw buffer descriptor (gfx9 dword3) over 2^31-1 bytes from `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}

constexpr int kZoh = 1, kFront = 2, kSoftplus = 4;

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

// e^x - 1 for x = arg * ln 2 given e2 = 2^arg: a short Taylor series where |x| < 1/16 (no
// cancellation), else e2 - 1.
__device__ __forceinline__ float expm1_of_log2(float arg, float e2) {
  const float xn = arg * kLn2;
  const float p = xn * __builtin_fmaf(xn, __builtin_fmaf(xn, __builtin_fmaf(xn, 1.0f / 24.0f, 1.0f / 6.0f), 0.5f), 1.0f);
  return fabsf(xn) < 0.0625f ? p : e2 - 1.0f;
}

struct SelSeg {
  int64_t batch, L, D, seg_len;
  int N, S, ngroups;  // ngroups = ceil(D / 64)
  int gpb;            // channel groups (waves) per workgroup, all on the same segment
  int nblk;           // workgroups per (batch, segment) = ceil(ngroups / gpb)
  int kshift, nsub;   // PASS 3: a checkpoint every 2^kshift steps, nsub per segment
};

// ------------------------------------------------------------------ pass 1 / pass 2
// PASS 1 (segments 0..S-2): seg_state[s][b][n][d] = end state from zero, seg_dsum[s][b][d].
// PASS 2 (segments 0..S-1): y, and h_last from the last segment; entering state from
//         carry[s][b][n][d] (S > 1) or h0 (S == 1).
// PASS 3 (segments 0..S-1, for the backward pass): from the same entering state, the state
//         before every 2^kshift-th step into seg_state[s * nsub + j][b][n][d].
// FL: bit kZoh -- exact zero-order-hold input term, expm1(delta*A)/A * B instead of
//     delta * B; bits kFront / kSoftplus -- the step size is delta + bias[d], then (with
//     kSoftplus) softplus of it.
template <int NS, bool BF16, int PASS, bool HAS_Z, int FL>
__global__ __launch_bounds__(256, min_waves_per_simd(NS)) void sel_seq_kernel(const void* __restrict__ x, const void* __restrict__ delta,
                                                     const float* __restrict__ A, const float* __restrict__ Bm,
                                                     const float* __restrict__ Cm, const float* __restrict__ Dsk,
                                                     const void* __restrict__ z, const float* __restrict__ h0,
                                                     const float* __restrict__ carry, float* __restrict__ y,
                                                     float* __restrict__ h_last, float* __restrict__ seg_state,
                                                     float* __restrict__ seg_dsum, const float* __restrict__ dbias,
                                                     SelSeg g) {
  // Workgroup = gpb waves on adjacent channel groups and the SAME time segment, so that the
  // scalar B_t/C_t rows one wave fetches are scalar-cache hits for the others.
  const int lane = threadIdx.x & 63;
  uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int blk = (int)(lid % (uint32_t)g.nblk);
  lid /= (uint32_t)g.nblk;
  const int64_t b = (int64_t)(lid % (uint32_t)g.batch);
  const int s = (int)(lid / (uint32_t)g.batch);
  // wave index made provably wave-uniform, so that everything derived from it (row bases,
  // buffer descriptors) lives in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int grp = min(blk * g.gpb + wave, g.ngroups - 1);  // surplus waves mirror the last group
  const int64_t d0 = (int64_t)grp * 64;
  // Lanes past the last channel mirror channel D-1: same inputs, same state, same outputs,
  // so every load and store can stay unconditional (duplicate stores write equal values).
  const int64_t dc = min(d0 + lane, g.D - 1);
  const int loff = (int)(dc - d0);
  const int64_t tbeg = (int64_t)s * g.seg_len;
  const int len = (int)(min(tbeg + g.seg_len, g.L) - tbeg);  // < 2^30 (plan)
  const int N = NS;

  constexpr bool zoh = (FL & kZoh) != 0;
  float a2[NS], h[NS];
  float ia[zoh ? NS : 1], az[zoh ? NS : 1];  // exact hold: 1/A[n] and (A[n] == 0)
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    const float an = A[dc * N + n];
    a2[n] = fmaxf(an * kLog2e, -kFltMax);  // -inf clamped so that 0*a2 = 0
    if constexpr (zoh) {
      ia[n] = an != 0.0f ? 1.0f / an : 0.0f;
      az[n] = an != 0.0f ? 0.0f : 1.0f;
    }
    if (PASS == 1) {
      h[n] = 0.0f;
    } else if (g.S > 1) {
      h[n] = carry[(((int64_t)s * g.batch + b) * N + n) * g.D + dc];
    } else {
      h[n] = h0 ? h0[(b * g.D + dc) * N + n] : 0.0f;
    }
  }
  const float Dd = (PASS == 2 && Dsk != nullptr) ? Dsk[dc] : 0.0f;
  const int kmask = (1 << g.kshift) - 1;
  const float dbv = ((FL & kFront) != 0 && dbias != nullptr) ? dbias[dc] : 0.0f;
  constexpr bool has_z = PASS == 2 && HAS_Z;
  float dsum = 0.0f;

  // Buffer descriptors based at this wave's first row of the segment: per-step offsets are
  // wave-uniform (SGPR soffset), the lane offset is a constant VGPR, so no per-load VALU
  // address arithmetic is needed.  The host keeps seg_len * D * 4 below 2^31.
  constexpr int ES = BF16 ? 2 : 4;
  const int64_t row0 = b * g.L + tbeg;
  const int rstride = (int)(g.D * ES);  // bytes between consecutive steps
  const uint32_t vo = (uint32_t)loff * ES;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc((const char*)x + (row0 * g.D + d0) * ES);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc((const char*)delta + (row0 * g.D + d0) * ES);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(has_z ? (const char*)z + (row0 * g.D + d0) * ES : (const char*)x);
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(PASS == 2 ? (const char*)(y + row0 * g.D + d0) : (const char*)x);
  const int ystride = (int)(g.D * 4);
  const float* Br = Bm + row0 * N;
  const float* Cr = Cm + row0 * N;

  constexpr int U = kStepsPerBatch;
  // raw loaded values (bf16 bits or fp32 bits) are widened only when used, so that the
  // loads of the next batch stay in flight while the current batch is computed
  uint32_t xq[2][U], dq[2][U], zq[2][U];
  auto ld = [vo](__amdgpu_buffer_rsrc_t r, int soff) -> uint32_t {
    if (BF16) return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)vo, soff, kStreamPolicy);
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)vo, soff, kStreamPolicy);
  };
  auto wid = [](uint32_t v) -> float { return BF16 ? __builtin_bit_cast(float, v << 16) : __builtin_bit_cast(float, v); };
#define SSS_LOAD_BATCH(SLOT, T0)                                                 \
  do {                                                                           \
    _Pragma("unroll") for (int i_ = 0; i_ < U; ++i_) {                           \
      const int t_ = min((T0) + i_, len - 1); /* clamped, unused */              \
      xq[SLOT][i_] = ld(rx, t_ * rstride);                                       \
      dq[SLOT][i_] = ld(rd, t_ * rstride);                                       \
      if (has_z) zq[SLOT][i_] = ld(rz, t_ * rstride);                            \
    }                                                                            \
  } while (0)

  // one step at segment-relative time T from register slot (SLOT, I); B_t / C_t rows are
  // wave-uniform and come through scalar loads
#define SSS_STEP(SLOT, I, T)                                                     \
  do {                                                                           \
    const float* Bt = Br + (T) * N;                                              \
    const float* Ct = Cr + (T) * N;                                              \
    if (PASS == 3 && ((T) & kmask) == 0) {                                       \
      _Pragma("unroll") for (int n = 0; n < NS; ++n)                             \
        seg_state[((((int64_t)s * g.nsub + ((T) >> g.kshift)) * g.batch + b) * N + n) * g.D + dc] = h[n]; \
    }                                                                            \
    const float xv = wid(xq[SLOT][I]);                                           \
    const float dl = step_size<FL>(wid(dq[SLOT][I]), dbv);                       \
    const float dx = dl * xv;                                                    \
    float y0 = Dd * xv, y1 = 0.0f;                                               \
    _Pragma("unroll") for (int n = 0; n < NS; ++n) {                             \
      const float arg = dl * a2[n];                                              \
      const float ab = fast_exp2(arg);                                           \
      if constexpr (zoh) {                                                       \
        const float cf = __builtin_fmaf(expm1_of_log2(arg, ab), ia[n], dl * az[n]); \
        h[n] = __builtin_fmaf(ab, h[n], cf * (xv * Bt[n]));                      \
      } else {                                                                   \
        h[n] = __builtin_fmaf(ab, h[n], dx * Bt[n]);                             \
      }                                                                          \
      if (PASS == 2) {                                                           \
        if (n & 1) y1 = __builtin_fmaf(Ct[n], h[n], y1);                         \
        else y0 = __builtin_fmaf(Ct[n], h[n], y0);                               \
      }                                                                          \
    }                                                                            \
    if (PASS == 1) {                                                             \
      dsum += dl;                                                                \
    } else if (PASS == 2) {                                                      \
      float out = y0 + y1;                                                       \
      if (has_z) out *= silu(wid(zq[SLOT][I]));                                  \
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, out), ry, (int)(loff * 4), \
                                            (T) * ystride, kStreamPolicy);       \
    }                                                                            \
  } while (0)

  SSS_LOAD_BATCH(0, 0);
  int t0 = 0;
  // full blocks of 2U steps: straight-line code, no per-step branches
  for (; t0 + 2 * U <= len; t0 += 2 * U) {
    SSS_LOAD_BATCH(1, t0 + U);
#pragma unroll
    for (int i = 0; i < U; ++i) SSS_STEP(0, i, t0 + i);
    SSS_LOAD_BATCH(0, t0 + 2 * U);
#pragma unroll
    for (int i = 0; i < U; ++i) SSS_STEP(1, i, t0 + U + i);
  }
  // ragged tail (< 2U steps): slot 0 already holds steps t0 .. t0+U-1
  if (t0 < len) {
    SSS_LOAD_BATCH(1, t0 + U);
    for (int i = 0; i < U && t0 + i < len; ++i) SSS_STEP(0, i, t0 + i);
    for (int i = 0; i < U && t0 + U + i < len; ++i) SSS_STEP(1, i, t0 + U + i);
  }
#undef SSS_LOAD_BATCH
#undef SSS_STEP

  if (PASS == 1) {
    if (lane == 0 || d0 + lane < g.D) seg_dsum[((int64_t)s * g.batch + b) * g.D + dc] = dsum;
#pragma unroll
    for (int n = 0; n < NS; ++n) seg_state[(((int64_t)s * g.batch + b) * N + n) * g.D + dc] = h[n];
  } else if (PASS == 2 && h_last != nullptr && s == g.S - 1) {
#pragma unroll
    for (int n = 0; n < NS; ++n) h_last[(b * g.D + dc) * N + n] = h[n];
  }
}

// ------------------------------------------------------------------ carry between segments
// One thread per (b, n, d), in place over the segment states: slot s holds the end state
// of segment s from zero on entry and the state entering segment s on exit,
//   carry[0] = h0,  carry[s+1] = exp2(A' * dsum_s) * carry[s] + state_s.
// Loads of a batch of segments are issued before the serial fma chain consumes them.
constexpr int kCarryBatch = 8;

static __global__ __launch_bounds__(256) void sel_carry_kernel(const float* __restrict__ A, const float* __restrict__ h0,
                                                        float* slots, const float* __restrict__ seg_dsum, SelSeg g) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_b = (int64_t)g.N * g.D;
  if (idx >= g.batch * per_b) return;
  const int64_t b = idx / per_b;
  const int64_t rem = idx - b * per_b;
  const int64_t n = rem / g.D, d = rem - n * g.D;
  const float a2 = fmaxf(A[d * g.N + n] * kLog2e, -kFltMax);
  float h = h0 ? h0[(b * g.D + d) * g.N + n] : 0.0f;
  const int64_t sstride = g.batch * per_b, dstride = g.batch * g.D;
  float* slot = slots + b * per_b + rem;              // [s][b][n][d]
  const float* dsp = seg_dsum + b * g.D + d;          // [s][b][d]
  for (int s0 = 0; s0 < g.S; s0 += kCarryBatch) {
    float st[kCarryBatch], ds[kCarryBatch];
#pragma unroll
    for (int i = 0; i < kCarryBatch; ++i) {
      const bool live = s0 + i < g.S - 1;            // segment S-1 has no end state
      st[i] = live ? slot[(int64_t)(s0 + i) * sstride] : 0.0f;
      ds[i] = live ? dsp[(int64_t)(s0 + i) * dstride] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kCarryBatch; ++i) {
      if (s0 + i < g.S) slot[(int64_t)(s0 + i) * sstride] = h;
      h = __builtin_fmaf(fast_exp2(a2 * ds[i]), h, st[i]);
    }
  }
}

static SelSeg make_seg(const SelArgs& a, const SelPlan& pl, int ns) {
  SelSeg g{};
  g.batch = a.batch;
  g.L = a.seqlen;
  g.D = a.dim;
  g.seg_len = pl.seg_len;
  g.N = ns;
  g.S = pl.segments;
  g.ngroups = (int)((a.dim + 63) / 64);
  g.gpb = std::min(2, g.ngroups);
  g.nblk = (g.ngroups + g.gpb - 1) / g.gpb;
  return g;
}

// Pass 1 and the carry: the workspace's state slots end up holding the state entering
// every segment (S > 1; nothing to do for a single segment).
template <int NS, bool BF16, int FL>
static hipError_t run_states(const SelArgs& a, const SelPlan& pl, hipStream_t stream) {
  if (pl.segments <= 1) return hipSuccess;
  const SelSeg g = make_seg(a, pl, NS);
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  float* st = reinterpret_cast<float*>(ws + pl.ws_state);
  float* ds = reinterpret_cast<float*>(ws + pl.ws_dsum);
  const int64_t per_seg = (int64_t)g.nblk * g.batch;
  hipLaunchKernelGGL((sel_seq_kernel<NS, BF16, 1, false, FL>), dim3((unsigned)(per_seg * (pl.segments - 1))),
                     dim3(64u * (unsigned)g.gpb), 0, stream, a.x, a.delta, a.A, a.B, a.C, a.Dsk, a.z, a.h0,
                     (const float*)nullptr, a.y, a.h_last, st, ds, a.delta_bias, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nthr = g.batch * (int64_t)NS * g.D;
  hipLaunchKernelGGL(sel_carry_kernel, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, stream, a.A, a.h0, st,
                     (const float*)ds, g);
  return hipGetLastError();
}

template <int NS, bool BF16, int FL>
static hipError_t run_selective(const SelArgs& a, const SelPlan& pl, hipStream_t stream) {
  hipError_t e = run_states<NS, BF16, FL>(a, pl, stream);
  if (e != hipSuccess) return e;
  const SelSeg g = make_seg(a, pl, NS);
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  const float* st = pl.segments > 1 ? reinterpret_cast<const float*>(ws + pl.ws_state) : nullptr;
  const int64_t per_seg = (int64_t)g.nblk * g.batch;
  const dim3 grid((unsigned)(per_seg * pl.segments)), block(64u * (unsigned)g.gpb);
  if (a.z != nullptr)
    hipLaunchKernelGGL((sel_seq_kernel<NS, BF16, 2, true, FL>), grid, block, 0, stream, a.x, a.delta, a.A, a.B, a.C,
                       a.Dsk, a.z, a.h0, st, a.y, a.h_last, (float*)nullptr, (float*)nullptr, a.delta_bias, g);
  else
    hipLaunchKernelGGL((sel_seq_kernel<NS, BF16, 2, false, FL>), grid, block, 0, stream, a.x, a.delta, a.A, a.B,
                       a.C, a.Dsk, a.z, a.h0, st, a.y, a.h_last, (float*)nullptr, (float*)nullptr, a.delta_bias, g);
  return hipGetLastError();
}

// Segment entering states of the plain form (no options), for the backward pass.
template <int NS, bool BF16>
hipError_t run_segment_states(const SelArgs& a, const SelPlan& pl, hipStream_t stream) {
  return run_states<NS, BF16, 0>(a, pl, stream);
}

// Checkpoints for the backward pass (after run_segment_states): the state before every
// 2^kshift-th step of every segment, into ckpt[s * nsub + j][b][n][d].
template <int NS, bool BF16>
hipError_t run_checkpoints(const SelArgs& a, const SelPlan& pl, float* ckpt, int kshift, int nsub,
                           hipStream_t stream) {
  SelSeg g = make_seg(a, pl, NS);
  g.kshift = kshift;
  g.nsub = nsub;
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  const float* st = pl.segments > 1 ? reinterpret_cast<const float*>(ws + pl.ws_state) : nullptr;
  const int64_t per_seg = (int64_t)g.nblk * g.batch;
  hipLaunchKernelGGL((sel_seq_kernel<NS, BF16, 3, false, 0>), dim3((unsigned)(per_seg * pl.segments)),
                     dim3(64u * (unsigned)g.gpb), 0, stream, a.x, a.delta, a.A, a.B, a.C, a.Dsk, a.z, a.h0, st,
                     (float*)nullptr, (float*)nullptr, ckpt, (float*)nullptr, (const float*)nullptr, g);
  return hipGetLastError();
}

// Front end / hold variants: plain, exact hold, delta + bias (+ softplus), and both.
template <int NS, bool BF16>
hipError_t run_flags(const SelArgs& a, const SelPlan& pl, hipStream_t stream) {
  const bool front = a.delta_bias != nullptr || a.softplus;
  const int fl = (a.exact_zoh ? kZoh : 0) | (front ? kFront : 0) | (a.softplus ? kSoftplus : 0);
  switch (fl) {
    case 0: return run_selective<NS, BF16, 0>(a, pl, stream);
    case kZoh: return run_selective<NS, BF16, kZoh>(a, pl, stream);
    case kFront: return run_selective<NS, BF16, kFront>(a, pl, stream);
    case kFront | kSoftplus: return run_selective<NS, BF16, kFront | kSoftplus>(a, pl, stream);
    case kZoh | kFront: return run_selective<NS, BF16, kZoh | kFront>(a, pl, stream);
    case kZoh | kFront | kSoftplus: return run_selective<NS, BF16, kZoh | kFront | kSoftplus>(a, pl, stream);
    default: return hipErrorInvalidValue;
  }
}

// Explicit instances: the file is compiled once per state count (SSS_INST_NS = N) and once
// for the host part (plan and dispatch), so that the builds of the instances run in parallel.
#ifdef SSS_INST_NS
template hipError_t run_flags<SSS_INST_NS, false>(const SelArgs&, const SelPlan&, hipStream_t);
template hipError_t run_flags<SSS_INST_NS, true>(const SelArgs&, const SelPlan&, hipStream_t);
template hipError_t run_segment_states<SSS_INST_NS, false>(const SelArgs&, const SelPlan&, hipStream_t);
template hipError_t run_segment_states<SSS_INST_NS, true>(const SelArgs&, const SelPlan&, hipStream_t);
template hipError_t run_checkpoints<SSS_INST_NS, false>(const SelArgs&, const SelPlan&, float*, int, int, hipStream_t);
template hipError_t run_checkpoints<SSS_INST_NS, true>(const SelArgs&, const SelPlan&, float*, int, int, hipStream_t);
#else
#define SSS_EXTERN_INSTANCES(N)                                                                        \
  extern template hipError_t run_flags<N, false>(const SelArgs&, const SelPlan&, hipStream_t);           \
  extern template hipError_t run_flags<N, true>(const SelArgs&, const SelPlan&, hipStream_t);            \
  extern template hipError_t run_segment_states<N, false>(const SelArgs&, const SelPlan&, hipStream_t);  \
  extern template hipError_t run_segment_states<N, true>(const SelArgs&, const SelPlan&, hipStream_t);            \
  extern template hipError_t run_checkpoints<N, false>(const SelArgs&, const SelPlan&, float*, int, int, hipStream_t); \
  extern template hipError_t run_checkpoints<N, true>(const SelArgs&, const SelPlan&, float*, int, int, hipStream_t);
SSS_EXTERN_INSTANCES(1)
SSS_EXTERN_INSTANCES(2)
SSS_EXTERN_INSTANCES(4)
SSS_EXTERN_INSTANCES(8)
SSS_EXTERN_INSTANCES(16)
SSS_EXTERN_INSTANCES(32)
SSS_EXTERN_INSTANCES(64)
#undef SSS_EXTERN_INSTANCES

// ------------------------------------------------------------------ host side
static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

SelPlan plan_selective(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int num_cus) {
  SelPlan pl{};
  const int64_t groups = batch * ((dim + 63) / 64);
  const int64_t simds = (int64_t)std::max(num_cus, 1) * 4;
  // One wave per (channel group, segment).  Splitting time costs a second pass over the
  // inputs, so it is only worth it when the channel groups alone leave most SIMDs idle;
  // then aim at ~20 waves per SIMD: short segments keep every SIMD busy to the end.
  int64_t S = 1;
  if (groups < 2 * simds) {
    const int64_t target = simds * env_int("SSS_WAVES_PER_SIMD", 20);
    S = std::max<int64_t>(1, (target + groups / 2) / groups);
    S = std::min<int64_t>(S, std::max<int64_t>(1, seqlen / 32));  // segments of >= 32 steps
    S = std::min<int64_t>(S, 4096);
  }
  const int forced = env_int("SSS_FORCE_SEGMENTS", 0);
  if (forced > 0) S = std::min<int64_t>(forced, (seqlen + kStepsPerBatch - 1) / kStepsPerBatch);
  if (S < 1) S = 1;
  // buffer offsets inside one segment (seg_len rows of dim fp32 values) must stay below
  // 2^30 bytes; dim <= 2^24 is checked by the caller, so max_len >= 16 steps (the B/C row
  // pointers advance by dstate floats per step, also kept below 2^30 bytes)
  const int64_t row_bytes = std::max(dim, dstate) * 4;
  const int64_t max_len = std::max<int64_t>(kStepsPerBatch, ((int64_t)1 << 30) / row_bytes / kStepsPerBatch * kStepsPerBatch);
  int64_t seg_len = (seqlen + S - 1) / S;
  seg_len = (seg_len + kStepsPerBatch - 1) / kStepsPerBatch * kStepsPerBatch;
  seg_len = std::min(seg_len, max_len);
  S = (seqlen + seg_len - 1) / seg_len;
  pl.segments = (int)S;
  pl.seg_len = seg_len;
  // workspace: segment states / entering states [S][batch][dstate][dim], segment sums of
  // delta [S][batch][dim]
  pl.ws_state = 0;
  pl.ws_dsum = align_up(S > 1 ? (size_t)S * batch * dstate * dim * 4 : 0, 256);
  pl.ws_total = align_up(pl.ws_dsum + (S > 1 ? (size_t)S * batch * dim * 4 : 0), 256);
  if (S == 1) pl.ws_dsum = pl.ws_total = 0;
  return pl;
}

template <bool BF16>
static hipError_t dispatch_n(const SelArgs& a, const SelPlan& pl, hipStream_t stream) {
  switch (a.dstate) {
    case 1: return run_flags<1, BF16>(a, pl, stream);
    case 2: return run_flags<2, BF16>(a, pl, stream);
    case 4: return run_flags<4, BF16>(a, pl, stream);
    case 8: return run_flags<8, BF16>(a, pl, stream);
    case 16: return run_flags<16, BF16>(a, pl, stream);
    case 32: return run_flags<32, BF16>(a, pl, stream);
    case 64: return run_flags<64, BF16>(a, pl, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_selective(const SelArgs& a, const SelPlan& pl, hipStream_t stream) {
  return a.bf16 ? dispatch_n<true>(a, pl, stream) : dispatch_n<false>(a, pl, stream);
}

template <bool BF16>
static hipError_t dispatch_states(const SelArgs& a, const SelPlan& pl, hipStream_t stream) {
  switch (a.dstate) {
    case 1: return run_segment_states<1, BF16>(a, pl, stream);
    case 2: return run_segment_states<2, BF16>(a, pl, stream);
    case 4: return run_segment_states<4, BF16>(a, pl, stream);
    case 8: return run_segment_states<8, BF16>(a, pl, stream);
    case 16: return run_segment_states<16, BF16>(a, pl, stream);
    case 32: return run_segment_states<32, BF16>(a, pl, stream);
    case 64: return run_segment_states<64, BF16>(a, pl, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_segment_states(const SelArgs& a, const SelPlan& pl, hipStream_t stream) {
  return a.bf16 ? dispatch_states<true>(a, pl, stream) : dispatch_states<false>(a, pl, stream);
}

template <bool BF16>
static hipError_t dispatch_ckpt(const SelArgs& a, const SelPlan& pl, float* ckpt, int kshift, int nsub,
                                hipStream_t stream) {
  switch (a.dstate) {
    case 1: return run_checkpoints<1, BF16>(a, pl, ckpt, kshift, nsub, stream);
    case 2: return run_checkpoints<2, BF16>(a, pl, ckpt, kshift, nsub, stream);
    case 4: return run_checkpoints<4, BF16>(a, pl, ckpt, kshift, nsub, stream);
    case 8: return run_checkpoints<8, BF16>(a, pl, ckpt, kshift, nsub, stream);
    case 16: return run_checkpoints<16, BF16>(a, pl, ckpt, kshift, nsub, stream);
    case 32: return run_checkpoints<32, BF16>(a, pl, ckpt, kshift, nsub, stream);
    case 64: return run_checkpoints<64, BF16>(a, pl, ckpt, kshift, nsub, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_checkpoints(const SelArgs& a, const SelPlan& pl, float* ckpt, int kshift, int nsub,
                              hipStream_t stream) {
  return a.bf16 ? dispatch_ckpt<true>(a, pl, ckpt, kshift, nsub, stream)
                : dispatch_ckpt<false>(a, pl, ckpt, kshift, nsub, stream);
}

#endif  // SSS_INST_NS

}  // namespace sss
