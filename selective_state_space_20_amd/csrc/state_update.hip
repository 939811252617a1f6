// state_update.hip -- gfx950 kernel for one recurrent-inference step of the selective scan.
//
// "Selective Scan trong Mamba toi uu chuoi dai the nao?" (section "Selective Scan thay doi
// inference chuoi dai nhu the nao?"): when tokens are generated one at a time only the
// state h (batch, dim, dstate) is carried, so each token costs one update of it:
//   h[b,d,n] = exp(delta[b,d]*A[d,n]) * h[b,d,n] + delta[b,d]*B[b,n]*x[b,d]      (in place)
//   y[b,d]   = (sum_n C[b,n]*h[b,d,n] + D[d]*x[b,d]) * silu(z[b,d])
//
// The step is bound by moving the state (8 bytes per state element: read and write back),
// so the mapping follows the state's layout: lanes walk (d, n) of a batch row in memory
// order, four states per lane, so that every state load and store of a wave is one
// contiguous 1 KiB piece of 16-byte vectors, and each thread carries four batch rows whose
// loads are all in flight together.  The lanes of a channel are adjacent and reduce C*h
// with DPP lane permutes inside their 16-lane row; the first of them writes y.
#include "common.h"
#include "kernels.h"

namespace sss {

template <bool BF16>
__device__ __forceinline__ float load_io(const void* p, int64_t i) {
  if (BF16) return __builtin_bit_cast(float, (uint32_t)static_cast<const uint16_t*>(p)[i] << 16);
  return static_cast<const float*>(p)[i];
}

typedef float f4v __attribute__((ext_vector_type(4)));

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over each group of LPC adjacent lanes (LPC = 1, 2, 4, 8 or 16, groups aligned to LPC);
// every lane of a group ends with the sum.  Pairs first (quad_perm 1,0,3,2), then pairs of
// pairs (quad_perm 2,3,0,1); each quad then holds one value, so mirroring the 8-lane half-row
// (row_half_mirror) and then the 16-lane row (row_mirror) meets the partner quad and the
// partner half.  All inside one DPP row: no LDS round trip.
template <int LPC>
__device__ __forceinline__ float group_sum(float p) {
  static_assert(LPC == 1 || LPC == 2 || LPC == 4 || LPC == 8 || LPC == 16, "lanes per channel");
  if constexpr (LPC >= 2) p += dpp_mov<0xB1>(p);   // quad_perm [1,0,3,2]
  if constexpr (LPC >= 4) p += dpp_mov<0x4E>(p);   // quad_perm [2,3,0,1]
  if constexpr (LPC >= 8) p += dpp_mov<0x141>(p);  // row_half_mirror
  if constexpr (LPC >= 16) p += dpp_mov<0x140>(p); // row_mirror
  return p;
}

// Each lane owns PL = min(4, NS) adjacent states of one channel (a 16-byte piece of the
// state, of A and of B/C) for R batch rows; the LPC = NS / PL lanes of a channel are
// adjacent and reduce C*h through DPP (group_sum).  All R rows' loads are issued before any of
// them is used, so that a wave keeps R KiB of state in flight (one KiB per row and wave).
// blockIdx.x = row group * bpb + k; rows past the batch load the last row and store nothing.
template <int NS, bool BF16, bool HAS_Z, int R>
__global__ __launch_bounds__(256) void sel_update_kernel(const void* __restrict__ x, const void* __restrict__ delta,
                                                         const float* __restrict__ A, const float* __restrict__ Bm,
                                                         const float* __restrict__ Cm, const float* __restrict__ Dsk,
                                                         const void* __restrict__ z, float* __restrict__ state,
                                                         float* __restrict__ y, int64_t batch, int dim,
                                                         unsigned bpb /* blocks per row group */) {
  constexpr int PL = NS >= 4 ? 4 : NS;
  constexpr int LPC = NS / PL;
  const unsigned rg = blockIdx.x / bpb;
  const int li = (int)(blockIdx.x - rg * bpb) * 256 + (int)threadIdx.x;  // lane index within a row
  // Lanes past the row's end form whole channel groups (LPC divides 64); they work on the
  // row's last channel so that every lane takes part in the shuffles, and store nothing.
  const bool live = li < dim * LPC;
  const int d = (live ? li : dim * LPC - 1) / LPC;  // LPC is a power of two
  const int j = (live ? li : dim * LPC - 1) - d * LPC;

  float av[PL];
  if constexpr (PL == 4) {
    const f4v a4 = *reinterpret_cast<const f4v*>(A + (int64_t)d * NS + j * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) av[i] = fmaxf(a4[i] * kLog2e, -kFltMax);  // -inf clamped: 0*a2 = 0
  } else {
#pragma unroll
    for (int i = 0; i < PL; ++i) av[i] = fmaxf(A[(int64_t)d * NS + i] * kLog2e, -kFltMax);
  }
  const float dd = Dsk != nullptr ? Dsk[d] : 0.0f;

  float hv[R][PL], bv[R][PL], cv[R][PL], xv[R], dv[R], zv[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t b = min((int64_t)rg * R + r, batch - 1);
    const int64_t c = b * dim + d;
    xv[r] = load_io<BF16>(x, c);
    dv[r] = load_io<BF16>(delta, c);
    zv[r] = HAS_Z ? load_io<BF16>(z, c) : 0.0f;
    if constexpr (PL == 4) {
      const f4v s4 = *reinterpret_cast<const f4v*>(state + c * NS + j * 4);
      const f4v b4 = *reinterpret_cast<const f4v*>(Bm + b * NS + j * 4);
      const f4v c4 = *reinterpret_cast<const f4v*>(Cm + b * NS + j * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hv[r][i] = s4[i];
        bv[r][i] = b4[i];
        cv[r][i] = c4[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        hv[r][i] = state[c * NS + i];
        bv[r][i] = Bm[b * NS + i];
        cv[r][i] = Cm[b * NS + i];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t b = (int64_t)rg * R + r;
    const bool row = b < batch;
    const int64_t c = b * dim + d;
    const float dx = dv[r] * xv[r];
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      hv[r][i] = __builtin_fmaf(fast_exp2(dv[r] * av[i]), hv[r][i], dx * bv[r][i]);
      part = __builtin_fmaf(cv[r][i], hv[r][i], part);
    }
    if (live && row) {
      if constexpr (PL == 4) {
        const f4v o = {hv[r][0], hv[r][1], hv[r][2], hv[r][3]};
        *reinterpret_cast<f4v*>(state + c * NS + j * 4) = o;
      } else {
#pragma unroll
        for (int i = 0; i < PL; ++i) state[c * NS + i] = hv[r][i];
      }
    }
    part = group_sum<LPC>(part);
    if (live && row && j == 0) {
      float out = __builtin_fmaf(dd, xv[r], part);
      if (HAS_Z) out *= silu(zv[r]);
      y[c] = out;
    }
  }
}

template <int NS, bool BF16>
static hipError_t run_update(const UpdArgs& a, hipStream_t stream) {
  constexpr int LPC = NS >= 4 ? NS / 4 : 1;
  constexpr int R = 4;  // batch rows per thread
  const unsigned bpb = (unsigned)((a.dim * LPC + 255) / 256);
  const dim3 grid((unsigned)(bpb * ((a.batch + R - 1) / R))), block(256);
  if (a.z != nullptr)
    hipLaunchKernelGGL((sel_update_kernel<NS, BF16, true, R>), grid, block, 0, stream, a.x, a.delta, a.A, a.B, a.C,
                       a.Dsk, a.z, a.state, a.y, a.batch, (int)a.dim, bpb);
  else
    hipLaunchKernelGGL((sel_update_kernel<NS, BF16, false, R>), grid, block, 0, stream, a.x, a.delta, a.A, a.B, a.C,
                       a.Dsk, a.z, a.state, a.y, a.batch, (int)a.dim, bpb);
  return hipGetLastError();
}

template <bool BF16>
static hipError_t dispatch_update(const UpdArgs& a, hipStream_t stream) {
  switch (a.dstate) {
    case 1: return run_update<1, BF16>(a, stream);
    case 2: return run_update<2, BF16>(a, stream);
    case 4: return run_update<4, BF16>(a, stream);
    case 8: return run_update<8, BF16>(a, stream);
    case 16: return run_update<16, BF16>(a, stream);
    case 32: return run_update<32, BF16>(a, stream);
    case 64: return run_update<64, BF16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_update(const UpdArgs& a, hipStream_t stream) {
  return a.bf16 ? dispatch_update<true>(a, stream) : dispatch_update<false>(a, stream);
}

}  // namespace sss
