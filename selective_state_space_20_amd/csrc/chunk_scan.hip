// chunk_scan.hip -- single-pass selective scan with a workgroup-level scan of affine pairs.
//
// The recurrence h_t = Abar_t h_{t-1} + u_t (Abar_t = exp(delta_t A[d,n]), u_t = delta_t
// B_t[n] x_t) is a chain of affine steps; their composition is associative ("Selective Scan
// trong Mamba toi uu chuoi dai the nao?", section "Scan bien recurrence thanh phep toan co the
// song song hoa ra sao?": (a2,b2) (x) (a1,b1) = (a2 a1, a2 b1 + b2), and the prefix over the
// pairs, Hinh 2, is the tree scan built here across waves).
//
// One workgroup = WAVES waves on one batch row and 64 consecutive channels (lanes = channels,
// so every x/delta/z/y access is one contiguous row piece per wave), walking the whole
// sequence in chunks of WAVES * KS steps.  For each chunk:
//   A. wave v takes steps [v KS, (v+1) KS) of the chunk: computes Abar and u for its KS steps
//      and N states (each exp once), keeps them in registers, and folds them from zero into
//      its pair (P_v = prod Abar, h_v = end state from zero);
//   C. the WAVES pairs go through LDS; wave w owns states {w SPW .. w SPW + SPW - 1} and scans
//      the pairs of its states in order from the chunk's entering state, writing the state
//      entering every wave's steps (and keeping the next chunk's entering state);
//   B. wave v replays its KS steps from its entering state with the kept Abar and u, and
//      writes y = (sum_n C_t[n] h_t[n] + D x_t) silu(z_t).
// Nothing is computed twice and no state goes to HBM; the cost is the replay's two fmas per
// state and step plus the pair exchange through LDS.  B_t / C_t rows of the chunk are staged in
// LDS (one 16-byte piece per lane of waves 0..3) and read by broadcast.
#include "common.h"
#include "kernels.h"

namespace sss {
namespace {

constexpr int kChunkWaves = 8;   // waves per workgroup (two per SIMD)
constexpr int kChunkSteps = 4;   // steps per wave and chunk (KS)
constexpr int kChunkLen = kChunkWaves * kChunkSteps;

typedef uint32_t u32x4c __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_n(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

struct ChunkArgs {
  const void* x;
  const void* delta;
  const float* A;
  const float* B;
  const float* C;
  const float* Dsk;
  const void* z;
  const float* h0;
  float* y;
  float* h_last;
  int64_t L, D;
  int ngroups;
};

// LDS (floats): rows [2][kChunkLen][2][NS] | pairs [2][WAVES][NS][64] | entering [WAVES][NS][64]
template <int NS>
constexpr int chunk_lds_floats() {
  return 2 * kChunkLen * 2 * NS + 2 * kChunkWaves * NS * 64 + kChunkWaves * NS * 64;
}

template <int NS, bool BF16, bool HAS_Z>
__global__ __launch_bounds__(64 * kChunkWaves, 2) void sel_chunk_kernel(ChunkArgs g) {
  constexpr int N = NS;
  constexpr int KS = kChunkSteps, W = kChunkWaves, CH = kChunkLen;
  constexpr int SPW = NS >= W ? NS / W : 1;          // states owned per wave in the scan
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int RowF = 2 * NS;                      // floats per step in the row tile (B, C)
  static_assert((CH * RowF * 4) % (16 * 64) == 0 && CH * RowF * 4 <= 16 * 64 * 4, "row tile = 1..4 waves x 1 KB");
  constexpr int kRowWaves = CH * RowF * 4 / (16 * 64);  // waves that load the row tile

  extern __shared__ float lds[];
  float* const rows = lds;                               // [2][CH][B NS | C NS]
  float* const pairs = lds + 2 * CH * RowF;              // [2 (P, h)][W][NS][64]
  float* const hin = pairs + 2 * W * NS * 64;            // [W][NS][64]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t b = blockIdx.x / g.ngroups;
  const int grp = blockIdx.x % g.ngroups;
  const int64_t d0 = (int64_t)grp * 64;
  const int64_t dc = min(d0 + lane, g.D - 1);  // lanes past the last channel mirror channel D-1
  const int64_t L = g.L;

  float a2[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) a2[n] = fmaxf(g.A[dc * N + n] * kLog2e, -kFltMax);
  const float Dd = g.Dsk ? g.Dsk[dc] : 0.0f;
  // the states this wave scans, and their entering value for the current chunk
  float carry[SPW];
#pragma unroll
  for (int k = 0; k < SPW; ++k) {
    const int n = wave * SPW + k;
    carry[k] = (n < NS && g.h0) ? g.h0[(b * g.D + dc) * N + n] : 0.0f;
  }

  // streamed rows: this wave's steps of a chunk start at row (chunk * CH + wave * KS)
  const int64_t row0 = b * L;
  const char* xb = (const char*)g.x + (row0 * g.D + d0) * ES;
  const char* db = (const char*)g.delta + (row0 * g.D + d0) * ES;
  const char* zb = HAS_Z ? (const char*)g.z + (row0 * g.D + d0) * ES : xb;
  const uint32_t vo = (uint32_t)(dc - d0) * ES;
  const int rstride = (int)(g.D * ES);
  const __amdgpu_buffer_rsrc_t rx = rsrc_n(xb, 0x7FFFFFFF), rd = rsrc_n(db, 0x7FFFFFFF), rz = rsrc_n(zb, 0x7FFFFFFF);
  const __amdgpu_buffer_rsrc_t ry = rsrc_n(g.y + row0 * g.D + d0, 0x7FFFFFFF);
  const uint32_t yvo = (uint32_t)(dc - d0) * 4;
  const int ystride = (int)(g.D * 4);
  // B / C rows of this batch row (the range stops at the sequence end: zeros past it)
  const int64_t bc_bytes = L * N * 4;
  const uint32_t bc_n = bc_bytes < 0x7FFFFFF0 ? (uint32_t)bc_bytes : 0x7FFFFFF0u;
  const __amdgpu_buffer_rsrc_t rb = rsrc_n(g.B + row0 * N, bc_n), rc = rsrc_n(g.C + row0 * N, bc_n);

  auto ld = [&](__amdgpu_buffer_rsrc_t r, int64_t t) -> uint32_t {
    const int tt = (int)(t < L ? t : L - 1);  // past the end: a clamped (unused) row
    if (BF16) return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)vo, tt * rstride, 2);
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)vo, tt * rstride, 2);
  };
  auto wid = [](uint32_t v) -> float { return BF16 ? __builtin_bit_cast(float, v << 16) : __builtin_bit_cast(float, v); };

  // row tile loads: lane piece i of a wave < kRowWaves covers 16 bytes of the interleaved
  // [step][B | C] tile of a chunk; B and C are separate arrays, so each piece takes 4 floats of
  // one of them: piece p -> step p / (RowF/4), tensor by (p % (RowF/4)) < NS/4
  u32x4c grow = {0u, 0u, 0u, 0u};
  const int piece = wave * 64 + lane;
  const int pstep = piece / (RowF / 4), pq = piece % (RowF / 4);
  const bool p_is_c = pq >= NS / 4;
  const int pcol = (p_is_c ? pq - NS / 4 : pq) * 4;
  auto rows_load = [&](int64_t chunk) {
    if (wave < kRowWaves) {
      const int64_t t = chunk * CH + pstep;
      const int off = (int)((t * N + pcol) * 4);  // past the end: outside the range, zeros
      grow = __builtin_amdgcn_raw_buffer_load_b128(p_is_c ? rc : rb, 0, off < 0 ? 0x7FFFFFF0 : off, 0);
    }
  };
  auto rows_store = [&](int buf) {
    if (wave < kRowWaves)
      *reinterpret_cast<u32x4c*>(rows + buf * (CH * RowF) + pstep * RowF + (p_is_c ? NS : 0) + pcol) = grow;
  };

  uint32_t xq[KS], dq[KS], zq[KS];  // this wave's raw inputs of the current chunk
  auto inputs_load = [&](int64_t chunk) {
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const int64_t t = chunk * CH + wave * KS + i;
      xq[i] = ld(rx, t);
      dq[i] = ld(rd, t);
      if constexpr (HAS_Z) zq[i] = ld(rz, t);
    }
  };

  const int64_t nchunks = (L + CH - 1) / CH;
  rows_load(0);
  inputs_load(0);
  for (int64_t c = 0; c < nchunks; ++c) {
    const int buf = (int)(c & 1);
    rows_store(buf);
    rows_load(c + 1);
    __syncthreads();  // rows[buf] complete; every wave is done with the previous chunk's LDS
    const float* crow = rows + buf * (CH * RowF);

    // ---- A: decays and input terms of this wave's KS steps, folded from zero
    float ab[KS][NS], uu[KS][NS], h[NS];
    float xv[KS];
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const int64_t t = c * CH + wave * KS + i;
      const bool live = t < L;  // wave-uniform; steps past the end are the identity pair
      xv[i] = wid(xq[i]);
      const float dl = live ? wid(dq[i]) : 0.0f;
      const float dx = dl * xv[i];
      const float* brow = crow + (wave * KS + i) * RowF;
      float bq[NS];
#pragma unroll
      for (int q = 0; q < NS / 4; ++q) {
        const float4 v4 = reinterpret_cast<const float4*>(brow)[q];
        bq[4 * q] = v4.x; bq[4 * q + 1] = v4.y; bq[4 * q + 2] = v4.z; bq[4 * q + 3] = v4.w;
      }
#pragma unroll
      for (int n = 0; n < NS; ++n) ab[i][n] = dl * a2[n];
      __builtin_amdgcn_sched_barrier(0x14);
#pragma unroll
      for (int n = 0; n < NS; ++n) ab[i][n] = fast_exp2(ab[i][n]);
      __builtin_amdgcn_sched_barrier(0x14);
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        uu[i][n] = dx * bq[n];
        h[n] = i == 0 ? uu[i][n] : __builtin_fmaf(ab[i][n], h[n], uu[i][n]);
      }
    }
    // the wave's pair: P = product of its decays, h = its end state from zero
    float* const pP = pairs + (0 * W + wave) * NS * 64 + lane;
    float* const pH = pairs + (1 * W + wave) * NS * 64 + lane;
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      float p = ab[0][n];
#pragma unroll
      for (int i = 1; i < KS; ++i) p *= ab[i][n];
      pP[n * 64] = p;
      pH[n * 64] = h[n];
    }
    // next chunk's inputs are in flight during the scan and the replay
    uint32_t xc[KS], zc[KS];
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      xc[i] = xq[i];
      zc[i] = HAS_Z ? zq[i] : 0u;
    }
    inputs_load(c + 1);
    __syncthreads();

    // ---- C: scan of the WAVES pairs, by state; wave w owns states w*SPW ..
#pragma unroll
    for (int k = 0; k < SPW; ++k) {
      const int n = wave * SPW + k;
      if (n < NS) {
        float H = carry[k];
#pragma unroll
        for (int v = 0; v < W; ++v) {
          hin[(v * NS + n) * 64 + lane] = H;
          H = __builtin_fmaf(pairs[(0 * W + v) * NS * 64 + n * 64 + lane], H,
                             pairs[(1 * W + v) * NS * 64 + n * 64 + lane]);
        }
        carry[k] = H;
      }
    }
    __syncthreads();

    // ---- B: replay this wave's steps from its entering state, read out and store
#pragma unroll
    for (int n = 0; n < NS; ++n) h[n] = hin[(wave * NS + n) * 64 + lane];
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const int64_t t = c * CH + wave * KS + i;
      const float* cr = crow + (wave * KS + i) * RowF + NS;
      float y0 = Dd * xv[i], y1 = 0.0f;
#pragma unroll
      for (int q = 0; q < NS / 4; ++q) {
        const float4 c4 = reinterpret_cast<const float4*>(cr)[q];
        const float cq[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int n = 4 * q + k;
          h[n] = __builtin_fmaf(ab[i][n], h[n], uu[i][n]);
          if (n & 1) y1 = __builtin_fmaf(cq[k], h[n], y1);
          else y0 = __builtin_fmaf(cq[k], h[n], y0);
        }
      }
      float out = y0 + y1;
      if constexpr (HAS_Z) out *= silu(wid(zc[i]));
      (void)xc;
      if (t < L) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, out), ry, (int)yvo,
                                                       (int)t * ystride, 2);
    }
  }
  // the final state: steps past the end are identity pairs, so the last chunk's exit state is
  // the state after step L-1
  if (g.h_last != nullptr && (lane == 0 || d0 + lane < g.D)) {
#pragma unroll
    for (int k = 0; k < SPW; ++k) {
      const int n = wave * SPW + k;
      if (n < NS) g.h_last[(b * g.D + dc) * N + n] = carry[k];
    }
  }
}

template <int NS, bool BF16>
hipError_t run_chunk(const SelArgs& a, hipStream_t stream) {
  ChunkArgs g{a.x, a.delta, a.A, a.B, a.C, a.Dsk, a.z, a.h0, a.y, a.h_last, a.seqlen, a.dim,
              (int)((a.dim + 63) / 64)};
  const dim3 grid((unsigned)(a.batch * g.ngroups)), block(64u * kChunkWaves);
  const size_t lds = (size_t)chunk_lds_floats<NS>() * 4;  // up to 104 KB: above the default limit
  if (a.z != nullptr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&sel_chunk_kernel<NS, BF16, true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((sel_chunk_kernel<NS, BF16, true>), grid, block, lds, stream, g);
  } else {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&sel_chunk_kernel<NS, BF16, false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((sel_chunk_kernel<NS, BF16, false>), grid, block, lds, stream, g);
  }
  return hipGetLastError();
}

}  // namespace

bool chunk_scan_supported(const SelArgs& a) {
  // plain form, time-major, 4/8/16 states; every buffer offset of one batch row (steps x dim
  // fp32 outputs, steps x dstate rows) stays a 31-bit byte offset
  return !a.bdl && !a.exact_zoh && !a.softplus && a.delta_bias == nullptr &&
         (a.dstate == 4 || a.dstate == 8 || a.dstate == 16) && a.seqlen * a.dim * 4 < ((int64_t)1 << 31) &&
         (a.seqlen + kChunkLen) * a.dstate * 4 < ((int64_t)1 << 31);
}

hipError_t launch_chunk_scan(const SelArgs& a, hipStream_t stream) {
  switch (a.dstate * 2 + (a.bf16 ? 1 : 0)) {
    case 8: return run_chunk<4, false>(a, stream);
    case 9: return run_chunk<4, true>(a, stream);
    case 16: return run_chunk<8, false>(a, stream);
    case 17: return run_chunk<8, true>(a, stream);
    case 32: return run_chunk<16, false>(a, stream);
    case 33: return run_chunk<16, true>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sss
