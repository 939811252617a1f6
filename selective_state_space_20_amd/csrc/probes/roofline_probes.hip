// roofline_probes.hip -- calibration kernels for the rooflines the benchmark reports.
//
// Not part of the scan library (built into its own libsss_probes.so, called only by
// bench.py --probes).  Two families:
//
//  * stream probes: what a plain HBM stream reaches on this chip (read-only, write-only and
//    copy, 16 bytes per lane and access, grid-stride over buffers far larger than the
//    last-level cache).  The HBM-bound kernels are judged against the copy rate;
//  * ALU probes: the issue cost per wave64 instruction of the VALU forms the scan is made
//    of (v_fma_f32, v_exp_f32, v_mul_f32 with a scalar operand) and of the scan's own
//    per-state step pattern, at 1..4 resident waves per SIMD, and whether the matrix core
//    (v_mfma_f32_4x4x1f32) issues alongside them.  Each wave times itself with
//    the shader clock (s_memtime) and the constant 100 MHz clock (s_memrealtime), so the
//    result is in clocks and the clock under load comes out too.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ stream probes
// mode 0: read-only (each thread folds its loads into one value, written once per thread),
// mode 1: write-only, mode 2: copy.  n16 = number of 16-byte chunks.
__global__ __launch_bounds__(256) void stream_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst,
                                                     int64_t n16, int mode, float* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (mode == 0) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (; i + 3 * stride < n16; i += 4 * stride) {
      const f32x4 a = __builtin_nontemporal_load(src + i);
      const f32x4 b = __builtin_nontemporal_load(src + i + stride);
      const f32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
      const f32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
      acc += (a + b) + (c + d);
    }
    for (; i < n16; i += stride) acc += __builtin_nontemporal_load(src + i);
    const float s = acc.x + acc.y + acc.z + acc.w;
    if (s == 1234.5f) sink[0] = s;  // never true for the probe's data: keeps the loads alive
  } else if (mode == 1) {
    const f32x4 v = {1.f, 2.f, 3.f, 4.f};
    for (; i < n16; i += stride) __builtin_nontemporal_store(v, dst + i);
  } else {
    for (; i + stride < n16; i += 2 * stride) {
      const f32x4 a = __builtin_nontemporal_load(src + i);
      const f32x4 b = __builtin_nontemporal_load(src + i + stride);
      __builtin_nontemporal_store(a, dst + i);
      __builtin_nontemporal_store(b, dst + i + stride);
    }
    for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
  }
}

// ------------------------------------------------------------------ ALU probes
// lane K of each 16-lane row, broadcast to the row (DPP row_newbcast:K)
template <int K>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + K, 0xF, 0xF, true));
}

// acc += (lane K of row's r) * h, the broadcast folded into the fmac as a DPP operand.  r is
// only ever written by loads and by VALU instructions at least two instructions earlier (the
// caller keeps an s_nop 1 between its last VALU write of r and the first use).
template <int K>
__device__ __forceinline__ void fmac_bcast(float& acc, float r, float h) {
  asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "+v"(acc) : "v"(r), "v"(h), "i"(K));
}

template <int... K, class F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, K...>, F&& f) {
  (f(std::integral_constant<int, K>{}), ...);
}

struct Rows {
  float b[16], c[16];  // wave-uniform rows: kernel arguments, hence SGPRs
};

constexpr int kOps = 16;  // independent chains per wave

// kind 0: v_fma_f32 (all VGPR operands)      kind 1: v_exp_f32
// kind 2: v_mul_f32 with an SGPR operand
// kind 3: one scan step of 16 states without read-out: per state arg = dl * a[n],
//         e = exp2(arg), h[n] = fma(e, h[n], dx * B[n])           (1 exp + 3 VALU)
// kind 4: the same plus the read-out y += C[n] * h[n]           (1 exp + 4 VALU)
// kind 5: kind 3 plus four independent v_mfma_f32_4x4x1f32 per iteration
// kind 6: sixteen independent v_mfma_f32_4x4x1f32 per iteration (on four accumulators)
// kind 7: v_mul_f32 with VGPR operands only (kind 2 without the scalar operand)
// kind 8: kind 4 with the B and C rows read from LDS instead of SGPRs: eight ds_read_b128
//         per iteration at a wave-uniform address (every lane reads the same 16 bytes)
// kind 9:  waves alternate roles by SIMD slot: role 0 issues kind 1 (exp), role 1 kind 0 (fma)
// kind 10: v_fmac_f32 with three VGPR operands (dst += a * b)
// kind 11: role 0 issues kind 1 (exp), role 1 kind 10 (fmac)
// kind 13: kind 8 with each step's instructions in phases: the 16 argument multiplies, then
//          the 16 exps, then the 64 remaining VALU instructions (scheduling barriers between)
// kind 14: kind 13 without the LDS rows (B and C as SGPR operands, as kind 4)
// kind 15: kind 13 with the update phase ordered by instruction: the 16 input-term multiplies,
//          then the 16 state fmas, then the 16 read-out fmas (no dependent neighbours)
// kind 16: kind 15 in groups of 4 states (each group: 4 mul | 4 exp | 4 mul | 4 fma | 4 fma)
// kind 17: kind 13 with the wave's priority raised (s_setprio 2) for its pairable phases
//          (argument multiplies, update) and lowered (0) for its exps
// kind 18: kind 13 with the priority raised for the exps and lowered for the rest
// kind 12: kind 4 with the B and C rows in one VGPR each (lane i of every 16-lane row holds
//          element i) and B[n], C[n] taken by the VALU ops through DPP row_newbcast:n
// Roles (kinds 9, 11): waves 4r .. 4r+3 of a workgroup fill one slot on each SIMD, so slot r
// takes role r & 1 and every SIMD with two or more waves holds both roles.
// Per iteration every kind issues kOps instructions of its main form (kinds 3/4: kOps
// states), plus two VALU updates of the step inputs in kinds 3 and 4.
template <int KIND>
__global__ __launch_bounds__(1024) void alu_kernel(int iters, Rows rows, uint64_t* __restrict__ out,
                                                   float* __restrict__ sink) {
  // 96 KB of the CU's 160 KB of LDS: no second workgroup fits beside this one
  __shared__ float pad[24 * 1024];
  const int lane = threadIdx.x & 63;
  float v[kOps], a[kOps];
#pragma unroll
  for (int k = 0; k < kOps; ++k) {
    v[k] = 0.25f + 0.01f * (float)((lane + k) & 7);
    a[k] = -0.5f - 0.03f * (float)k;
  }
  float dl = 0.01f + 1e-4f * (float)lane, dx = 0.5f, y0 = 0.0f, y1 = 0.0f;
  float brow = rows.b[lane & 15], crow = rows.c[lane & 15];
  f32x4 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float fb = 0.999f, fc = 1e-3f * (float)(lane & 3);
  pad[threadIdx.x * 24] = v[0];  // threadIdx.x < 1024: within the array
  __syncthreads();
  // rows for kind 8: 64 rows of 32 floats (B then C) at the start of the array
  for (int i = threadIdx.x; i < 64 * 32; i += blockDim.x) pad[i] = 0.5f + 1e-3f * (float)(i & 31);
  __syncthreads();
  int rowsel = 0;
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const int role = __builtin_amdgcn_readfirstlane((int)((threadIdx.x >> 8) & 1));
  float u[kOps];
#pragma unroll
  for (int k = 0; k < kOps; ++k) u[k] = 1e-3f * (float)(k + 1);
  auto step = [&]() {
    if constexpr (KIND == 15 || KIND == 16) {
      float bv[kOps], cv[kOps], e[kOps], uu[kOps];
      const f32x4* row = reinterpret_cast<const f32x4*>(pad + ((rowsel++) & 63) * 32);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 b4 = row[q], c4 = row[4 + q];
        bv[4 * q] = b4.x; bv[4 * q + 1] = b4.y; bv[4 * q + 2] = b4.z; bv[4 * q + 3] = b4.w;
        cv[4 * q] = c4.x; cv[4 * q + 1] = c4.y; cv[4 * q + 2] = c4.z; cv[4 * q + 3] = c4.w;
      }
      constexpr int G = KIND == 15 ? kOps : 4;
#pragma unroll
      for (int g0 = 0; g0 < kOps; g0 += G) {
#pragma unroll
        for (int k = g0; k < g0 + G; ++k) e[k] = dl * a[k];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = g0; k < g0 + G; ++k) e[k] = __builtin_amdgcn_exp2f(e[k]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = g0; k < g0 + G; ++k) uu[k] = dx * bv[k];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = g0; k < g0 + G; ++k) v[k] = __builtin_fmaf(e[k], v[k], uu[k]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = g0; k < g0 + G; ++k) {
          if (k & 1) y1 = __builtin_fmaf(cv[k], v[k], y1);
          else y0 = __builtin_fmaf(cv[k], v[k], y0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      dl = __builtin_fmaf(dl, 0.9999f, 1e-6f);
      dx = __builtin_fmaf(dx, 0.999f, 1e-4f);
    } else if constexpr (KIND == 13 || KIND == 14 || KIND == 17 || KIND == 18) {
      constexpr int kPv = KIND == 17 ? 2 : 0, kPe = KIND == 18 ? 2 : 0;  // phase priorities
      constexpr bool kPrio = KIND == 17 || KIND == 18;
      float bv[kOps], cv[kOps], e[kOps];
#pragma unroll
      for (int k = 0; k < kOps; ++k) {
        bv[k] = rows.b[k];
        cv[k] = rows.c[k];
      }
      if constexpr (KIND != 14) {
        const f32x4* row = reinterpret_cast<const f32x4*>(pad + ((rowsel++) & 63) * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 b4 = row[q], c4 = row[4 + q];
          bv[4 * q] = b4.x; bv[4 * q + 1] = b4.y; bv[4 * q + 2] = b4.z; bv[4 * q + 3] = b4.w;
          cv[4 * q] = c4.x; cv[4 * q + 1] = c4.y; cv[4 * q + 2] = c4.z; cv[4 * q + 3] = c4.w;
        }
      }
      if constexpr (kPrio) __builtin_amdgcn_s_setprio(kPv);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < kOps; ++k) e[k] = dl * a[k];
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kPrio) __builtin_amdgcn_s_setprio(kPe);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < kOps; ++k) e[k] = __builtin_amdgcn_exp2f(e[k]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kPrio) __builtin_amdgcn_s_setprio(kPv);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < kOps; ++k) {
        v[k] = __builtin_fmaf(e[k], v[k], dx * bv[k]);
        if (k & 1) y1 = __builtin_fmaf(cv[k], v[k], y1);
        else y0 = __builtin_fmaf(cv[k], v[k], y0);
      }
      dl = __builtin_fmaf(dl, 0.9999f, 1e-6f);
      dx = __builtin_fmaf(dx, 0.999f, 1e-4f);
      __builtin_amdgcn_sched_barrier(0);
    } else if constexpr (KIND == 12) {
      static_for(std::make_integer_sequence<int, kOps>{}, [&](auto kc) {
        constexpr int k = decltype(kc)::value;
        const float e = __builtin_amdgcn_exp2f(dl * a[k]);
        v[k] = __builtin_fmaf(e, v[k], dx * row_bcast<k>(brow));
        if (k & 1) fmac_bcast<k>(y1, crow, v[k]);
        else fmac_bcast<k>(y0, crow, v[k]);
      });
      dl = __builtin_fmaf(dl, 0.9999f, 1e-6f);
      dx = __builtin_fmaf(dx, 0.999f, 1e-4f);
      brow = __builtin_fmaf(brow, 0.999f, 1e-4f);  // a new step's rows
      crow = __builtin_fmaf(crow, 0.999f, 1e-4f);
      asm volatile("s_nop 1");
    } else if constexpr (KIND == 10) {
#pragma unroll
      for (int k = 0; k < kOps; ++k) v[k] = __builtin_fmaf(a[k], u[k], v[k]);
    } else if constexpr (KIND == 0) {
#pragma unroll
      for (int k = 0; k < kOps; ++k) v[k] = __builtin_fmaf(v[k], fb, fc);
    } else if constexpr (KIND == 1) {
#pragma unroll
      for (int k = 0; k < kOps; ++k) v[k] = __builtin_amdgcn_exp2f(-v[k]);
    } else if constexpr (KIND == 2) {
#pragma unroll
      for (int k = 0; k < kOps; ++k) v[k] = v[k] * rows.b[k];
    } else if constexpr (KIND == 7) {
#pragma unroll
      for (int k = 0; k < kOps; ++k) v[k] = v[k] * a[k];
    } else if constexpr (KIND == 6) {
#pragma unroll
      for (int k = 0; k < kOps; ++k) acc[k & 3] = __builtin_amdgcn_mfma_f32_4x4x1f32(v[k], a[k], acc[k & 3], 0, 0, 0);
    } else {
      if constexpr (KIND == 5) {
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[m] = __builtin_amdgcn_mfma_f32_4x4x1f32(dx, a[m], acc[m], 0, 0, 0);
      }
      float bv[kOps], cv[kOps];
#pragma unroll
      for (int k = 0; k < kOps; ++k) {
        bv[k] = rows.b[k];
        cv[k] = rows.c[k];
      }
      if constexpr (KIND == 8) {
        // this iteration's rows: 128 bytes at a wave-uniform LDS offset
        const f32x4* row = reinterpret_cast<const f32x4*>(pad + ((rowsel++) & 63) * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 b4 = row[q], c4 = row[4 + q];
          bv[4 * q] = b4.x; bv[4 * q + 1] = b4.y; bv[4 * q + 2] = b4.z; bv[4 * q + 3] = b4.w;
          cv[4 * q] = c4.x; cv[4 * q + 1] = c4.y; cv[4 * q + 2] = c4.z; cv[4 * q + 3] = c4.w;
        }
      }
#pragma unroll
      for (int k = 0; k < kOps; ++k) {
        const float e = __builtin_amdgcn_exp2f(dl * a[k]);
        v[k] = __builtin_fmaf(e, v[k], dx * bv[k]);
        if constexpr (KIND == 4 || KIND == 8) {
          if (k & 1) y1 = __builtin_fmaf(cv[k], v[k], y1);
          else y0 = __builtin_fmaf(cv[k], v[k], y0);
        }
      }
      // the step inputs change every iteration (as a new time step's do), so that nothing
      // is hoisted out of the loop
      dl = __builtin_fmaf(dl, 0.9999f, 1e-6f);
      dx = __builtin_fmaf(dx, 0.999f, 1e-4f);
    }
  };
  // two copies of the body per iteration, so that the registers of loop-carried values
  // rotate without moves
  if constexpr (KIND == 9 || KIND == 11) {
    // one loop per role, chosen once per wave
    if (role == 0) {
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < kOps; ++k) v[k] = __builtin_amdgcn_exp2f(-v[k]);
      }
    } else {
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < kOps; ++k)
          v[k] = KIND == 9 ? __builtin_fmaf(v[k], fb, fc) : __builtin_fmaf(a[k], u[k], v[k]);
      }
    }
  } else {
    for (int it = 0; it < iters; it += 2) {
      step();
      step();
    }
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = y0 + y1 + brow + crow;
#pragma unroll
  for (int m = 0; m < 4; ++m) s += acc[m].x + acc[m].y + acc[m].z + acc[m].w;
#pragma unroll
  for (int k = 0; k < kOps; ++k) s += v[k];
  if (s == 1234.5f) sink[0] = s + pad[((threadIdx.x + 1) & 1023) * 24];  // keeps every chain alive
  if (lane == 0) {
    const int wave = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
    out[3 * wave] = c1 - c0;
    out[3 * wave + 1] = r1 - r0;
    // HW_ID (hardware register 4): wave slot [3:0], SIMD [5:4], CU [11:8], ...
    out[3 * wave + 2] = (uint64_t)__builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);
  }
}

}  // namespace

extern "C" {

// One stream probe over `bytes` (a multiple of 16) on `stream`; `src`/`dst` device buffers
// of that size (dst unused in mode 0, src in mode 1), `sink` one device float.  Returns a
// hipError_t value.
int sss_probe_stream(int mode, const void* src, void* dst, int64_t bytes, float* sink, int grid, void* stream) {
  if (mode < 0 || mode > 2 || bytes <= 0 || (bytes & 15) != 0 || grid <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                     (const f32x4*)src, (f32x4*)dst, bytes / 16, mode, sink);
  return (int)hipGetLastError();
}

// One ALU probe: `grid` workgroups of 4 * waves_per_simd waves, each workgroup holding a
// whole compute unit (its LDS request leaves no room for a second one), `iters` (even) loop
// iterations per wave.  out[3 * wave] = shader clocks, out[3 * wave + 1] = 100 MHz ticks,
// out[3 * wave + 2] = the wave's HW_ID register, for grid * 4 * waves_per_simd waves.  Returns a hipError_t value.
int sss_probe_alu(int kind, int waves_per_simd, int iters, int grid, uint64_t* out, float* sink, void* stream) {
  if (waves_per_simd < 1 || waves_per_simd > 4 || iters < 2 || (iters & 1) != 0 || grid < 1) return (int)hipErrorInvalidValue;
  Rows rows;
  for (int k = 0; k < 16; ++k) {
    rows.b[k] = 0.5f + 0.01f * (float)k;
    rows.c[k] = 0.25f - 0.01f * (float)k;
  }
  const dim3 block(256u * (unsigned)waves_per_simd);
  const size_t lds = 0;
  hipStream_t st = (hipStream_t)stream;
  switch (kind) {
    case 0: hipLaunchKernelGGL(alu_kernel<0>, dim3((unsigned)grid), block, lds, st, iters, rows, out, sink); break;
    case 1: hipLaunchKernelGGL(alu_kernel<1>, dim3((unsigned)grid), block, lds, st, iters, rows, out, sink); break;
    case 2: hipLaunchKernelGGL(alu_kernel<2>, dim3((unsigned)grid), block, lds, st, iters, rows, out, sink); break;
    case 3: hipLaunchKernelGGL(alu_kernel<3>, dim3((unsigned)grid), block, lds, st, iters, rows, out, sink); break;
    case 4: hipLaunchKernelGGL(alu_kernel<4>, dim3((unsigned)grid), block, lds, st, iters, rows, out, sink); break;
    case 5: hipLaunchKernelGGL(alu_kernel<5>, dim3((unsigned)grid), block, lds, st, iters, rows, out, sink); break;
    case 6: hipLaunchKernelGGL(alu_kernel<6>, dim3((unsigned)grid), block, lds, st, iters, rows, out, sink); break;
    case 7: hipLaunchKernelGGL(alu_kernel<7>, dim3((unsigned)grid), block, lds, st, iters, rows, out, sink); break;
    case 8: hipLaunchKernelGGL(alu_kernel<8>, dim3((unsigned)grid), block, lds, st, iters, rows, out, sink); break;
    case 9: hipLaunchKernelGGL(alu_kernel<9>, dim3((unsigned)grid), block, lds, st, iters, rows, out, sink); break;
    case 10: hipLaunchKernelGGL(alu_kernel<10>, dim3((unsigned)grid), block, lds, st, iters, rows, out, sink); break;
    case 11: hipLaunchKernelGGL(alu_kernel<11>, dim3((unsigned)grid), block, lds, st, iters, rows, out, sink); break;
    case 12: hipLaunchKernelGGL(alu_kernel<12>, dim3((unsigned)grid), block, lds, st, iters, rows, out, sink); break;
    case 13: hipLaunchKernelGGL(alu_kernel<13>, dim3((unsigned)grid), block, lds, st, iters, rows, out, sink); break;
    case 14: hipLaunchKernelGGL(alu_kernel<14>, dim3((unsigned)grid), block, lds, st, iters, rows, out, sink); break;
    case 15: hipLaunchKernelGGL(alu_kernel<15>, dim3((unsigned)grid), block, lds, st, iters, rows, out, sink); break;
    case 16: hipLaunchKernelGGL(alu_kernel<16>, dim3((unsigned)grid), block, lds, st, iters, rows, out, sink); break;
    case 17: hipLaunchKernelGGL(alu_kernel<17>, dim3((unsigned)grid), block, lds, st, iters, rows, out, sink); break;
    case 18: hipLaunchKernelGGL(alu_kernel<18>, dim3((unsigned)grid), block, lds, st, iters, rows, out, sink); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // extern "C"
