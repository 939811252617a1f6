// selective_scan.hip -- gfx950 kernels for the selective (Mamba) scan.
//
// Computes, per batch b, channel d, state n (see include/sss.h):
//   Abar_t = exp(delta_t*A[d,n]),  h_t = Abar_t*h_{t-1} + delta_t*B_t[n]*x_t,
//   y_t = (sum_n C_t[n]*h_t[n] + D[d]*x_t) * silu(z_t)
// The recurrence is the selective SSM of "Selective Scan trong Mamba toi uu chuoi dai the
// nao?" (sections "Tai sao Mamba can Selective Scan?", "Selection pha vo convolution
// kernel co dinh"); it is evaluated as a scan of affine pairs (a, b) composed with
// (a2,b2)(x)(a1,b1) = (a2*a1, a2*b1 + b2), identity (1, 0) (section "Scan bien recurrence
// thanh phep toan co the song song hoa ra sao?"), fused so that the (B,L,D,N) state never
// leaves registers (sections "Tai sao chi parallel scan van chua du nhanh?" and "Kernel
// fusion").
//
// Mapping (one wave = one channel):
//   * a chunk of 64*K consecutive steps is split into 64 sub-chunks of K steps; lane j owns
//     sub-chunk j and keeps its K values of delta, delta*x and the running y in registers;
//   * for each state n (outer loop): Abar = exp2(delta * A*log2e) and u = delta*x*B for the
//     K steps, a sequential fold into the lane pair, a 6-level DPP inclusive scan of the 64
//     lane pairs, the carry entering the chunk applied, then a re-walk of the K steps from the
//     lane's entering state that accumulates C*h into y (K exps per lane per state, none
//     recomputed);
//   * the chunk carry leaves through lane 63 and is kept, per state, in lane n of one VGPR.
//   * B and C are pre-transposed to (batch, N, L) so that the per-state slice of a chunk is
//     contiguous; each state's slice is staged once per workgroup into LDS (double-buffered,
//     padded blocks read with 16-byte ds_read) and shared by the workgroup's channels.
//   * x, delta, z tiles are loaded row-wise (coalesced along d) into padded LDS blocks and
//     read back per lane; y leaves through the same LDS transpose.
//   * Long sequences over few channels use a two-pass split: pass 1 computes each time
//     segment's end state from a zero state plus its total delta; pass 2 folds the earlier
//     segments into the entering state and produces the outputs.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace sss {

struct SelParams {
  const void* x;
  const void* delta;
  const float* A;
  const float* BT;  // (batch, N, lpad)
  const float* CT;  // (batch, N, lpad)
  const float* Dsk;
  const void* z;
  const float* h0;
  float* y;
  float* h_last;
  float* seg_state;  // (batch, S, dim, N)
  float* seg_dsum;   // (batch, S, dim)
  int64_t batch, L, D, lpad, seg_len;
  int N, S, wpb, ntiles, vec4;
};

// ------------------------------------------------------------------ B/C transpose
// (batch, L, N) -> (batch, N, lpad), zero in [L, lpad).  Tile: 64 steps x N states.
__global__ __launch_bounds__(256) void bc_transpose_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                           int64_t L, int64_t lpad, int N, int64_t ntt) {
  __shared__ float tile[64 * 65];
  const int64_t blk = blockIdx.x;
  const int64_t b = blk / ntt;
  const int64_t t0 = (blk % ntt) * 64;
  const float* s = src + b * L * N;
  float* o = dst + b * (int64_t)N * lpad;
  const int tot = 64 * N;
  for (int i = threadIdx.x; i < tot; i += blockDim.x) {  // coalesced over (t, n)
    int tt = i / N, n = i - tt * N;
    int64_t t = t0 + tt;
    tile[n * 65 + tt] = (t < L) ? s[t * N + n] : 0.0f;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < tot; i += blockDim.x) {  // coalesced over t for each n
    int n = i >> 6, tt = i & 63;
    int64_t t = t0 + tt;
    if (t < lpad) o[(int64_t)n * lpad + t] = tile[n * 65 + tt];
  }
}

// ------------------------------------------------------------------ tile staging
// Rows [t0, t0 + 64*K) x channels [d0, d0 + wpb) of a (batch, L, D) tensor into LDS blocks:
// block (c*64 + j) holds steps j*K .. j*K+K-1 of channel c (element size ES), padded to BLK.
// Rows at or past tend, and channels past D, read as 0.
template <int K, bool BF16>
__device__ __forceinline__ void stage_tile(unsigned char* __restrict__ lds, const void* __restrict__ gsrc,
                                           int64_t b, int64_t t0, int64_t tend, int64_t L, int64_t D,
                                           int64_t d0, int wpb, int vec4) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int BLK = K * ES + 16;
  constexpr int CHUNK = 64 * K;
  const int nthr = blockDim.x;
  if (vec4) {
    const int G = wpb >> 2;  // 4-channel groups per row
    const int units = CHUNK * G;
    for (int u = threadIdx.x; u < units; u += nthr) {
      const int row = u / G, g = u - row * G;
      const int64_t t = t0 + row;
      const int c0 = g * 4;
      const int64_t off = (b * L + t) * D + d0 + c0;
      const int jb = row / K, ib = row - jb * K;
      unsigned char* dst = lds + (c0 * 64 + jb) * BLK + ib * ES;
      if (BF16) {
        uint2 v = make_uint2(0u, 0u);
        if (t < tend && d0 + c0 < D) v = *reinterpret_cast<const uint2*>((const uint16_t*)gsrc + off);
        *reinterpret_cast<uint16_t*>(dst + 0 * 64 * BLK) = (uint16_t)(v.x & 0xFFFFu);
        *reinterpret_cast<uint16_t*>(dst + 1 * 64 * BLK) = (uint16_t)(v.x >> 16);
        *reinterpret_cast<uint16_t*>(dst + 2 * 64 * BLK) = (uint16_t)(v.y & 0xFFFFu);
        *reinterpret_cast<uint16_t*>(dst + 3 * 64 * BLK) = (uint16_t)(v.y >> 16);
      } else {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < tend && d0 + c0 < D) v = *reinterpret_cast<const float4*>((const float*)gsrc + off);
        *reinterpret_cast<float*>(dst + 0 * 64 * BLK) = v.x;
        *reinterpret_cast<float*>(dst + 1 * 64 * BLK) = v.y;
        *reinterpret_cast<float*>(dst + 2 * 64 * BLK) = v.z;
        *reinterpret_cast<float*>(dst + 3 * 64 * BLK) = v.w;
      }
    }
  } else {
    const int units = CHUNK * wpb;
    for (int u = threadIdx.x; u < units; u += nthr) {
      const int row = u / wpb, c = u - row * wpb;
      const int64_t t = t0 + row;
      const int64_t dd = d0 + c;
      const int jb = row / K, ib = row - jb * K;
      unsigned char* dst = lds + (c * 64 + jb) * BLK + ib * ES;
      const bool ok = t < tend && dd < D;
      const int64_t off = (b * L + t) * D + dd;
      if (BF16)
        *reinterpret_cast<uint16_t*>(dst) = ok ? ((const uint16_t*)gsrc)[off] : (uint16_t)0;
      else
        *reinterpret_cast<float*>(dst) = ok ? ((const float*)gsrc)[off] : 0.0f;
    }
  }
}

// Read this lane's K values of a staged tile block as floats.
template <int K, bool BF16>
__device__ __forceinline__ void read_block(const unsigned char* __restrict__ blk, float (&v)[K]) {
  if (BF16) {
#pragma unroll
    for (int q = 0; q < K / 8; ++q) {
      uint4 w = *reinterpret_cast<const uint4*>(blk + q * 16);
      v[q * 8 + 0] = bf16_lo(w.x); v[q * 8 + 1] = bf16_hi(w.x);
      v[q * 8 + 2] = bf16_lo(w.y); v[q * 8 + 3] = bf16_hi(w.y);
      v[q * 8 + 4] = bf16_lo(w.z); v[q * 8 + 5] = bf16_hi(w.z);
      v[q * 8 + 6] = bf16_lo(w.w); v[q * 8 + 7] = bf16_hi(w.w);
    }
  } else {
#pragma unroll
    for (int q = 0; q < K / 4; ++q) {
      float4 w = *reinterpret_cast<const float4*>(blk + q * 16);
      v[q * 4 + 0] = w.x; v[q * 4 + 1] = w.y; v[q * 4 + 2] = w.z; v[q * 4 + 3] = w.w;
    }
  }
}

// ------------------------------------------------------------------ the scan kernel
// PASS 1: segment end states (from a zero state) and segment delta sums, segments 0..S-2.
// PASS 2: outputs y (and h_last from the last segment), entering state folded from h0 and
//         the pass-1 segment states.
template <int K, bool BF16, int PASS>
__global__ __launch_bounds__(256) void sel_scan_kernel(SelParams p) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int CHUNK = 64 * K;
  constexpr int BLK_IN = K * ES + 16;
  constexpr int BLK_Y = K * 4 + 16;
  constexpr int BLK_BC = K + 4;  // floats
  extern __shared__ __align__(16) unsigned char smem[];

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nthr = blockDim.x;
  const int wpb = p.wpb;
  const int NL = wpb * 64;
  const int N = p.N;

  const int szX = max(2 * NL * BLK_IN, NL * BLK_Y);
  unsigned char* regX = smem;
  float* regBC = reinterpret_cast<float*>(smem + szX);  // [buf][tensor][64][BLK_BC]; z tile aliases

  uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = (int)(lid % (uint32_t)p.ntiles);
  lid /= (uint32_t)p.ntiles;
  const int64_t b = (int64_t)(lid % (uint32_t)p.batch);
  const int s = (int)(lid / (uint32_t)p.batch);
  const int64_t d0 = (int64_t)tile * wpb;
  const int64_t d = d0 + wv;
  const bool dvalid = d < p.D;
  const int64_t tbeg = (int64_t)s * p.seg_len;
  const int64_t tend = min(tbeg + p.seg_len, p.L);

  // Per-state vectors of this wave's channel: lane n holds state n (N <= 64).
  float a2vec = 0.0f;  // A[d,n] * log2(e), -inf clamped to -FLT_MAX so that 0*a2 = 0
  if (dvalid && lane < N) a2vec = fmaxf(p.A[d * N + lane] * kLog2e, -kFltMax);
  float hcvec = 0.0f;  // state entering the current chunk
  if (PASS == 2 && dvalid && lane < N) {
    float h = p.h0 ? p.h0[(b * p.D + d) * N + lane] : 0.0f;
    for (int s2 = 0; s2 < s; ++s2) {
      const float ds = p.seg_dsum[(b * p.S + s2) * p.D + d];
      const float st = p.seg_state[((b * p.S + s2) * p.D + d) * N + lane];
      h = __builtin_fmaf(fast_exp2(a2vec * ds), h, st);
    }
    hcvec = h;
  }
  const float Dd = (PASS == 2 && p.Dsk != nullptr && dvalid) ? p.Dsk[d] : 0.0f;
  float dsum_seg = 0.0f;

  const int nq = CHUNK / 4;  // float4 units of one state's chunk slice
  for (int64_t t0 = tbeg; t0 < tend; t0 += CHUNK) {
    // ---- stage x and delta, then each lane takes its K steps
    stage_tile<K, BF16>(regX, p.x, b, t0, tend, p.L, p.D, d0, wpb, p.vec4);
    stage_tile<K, BF16>(regX + NL * BLK_IN, p.delta, b, t0, tend, p.L, p.D, d0, wpb, p.vec4);
    // B/C slices of state 0 -> buffer 0
    for (int u = threadIdx.x; u < (PASS == 2 ? 2 : 1) * nq; u += nthr) {
      const int tsr = u / nq, q = u - tsr * nq;
      const int64_t t = t0 + 4 * q;
      const float* src = (tsr == 0 ? p.BT : p.CT) + (b * N + 0) * p.lpad;
      float4 v = (t < p.lpad) ? *reinterpret_cast<const float4*>(src + t) : make_float4(0.f, 0.f, 0.f, 0.f);
      const int jb = (4 * q) / K, ib = (4 * q) - jb * K;
      *reinterpret_cast<float4*>(regBC + ((0 * 2 + tsr) * 64 + jb) * BLK_BC + ib) = v;
    }
    __syncthreads();

    float dl[K], dx[K], yv[K];
    {
      float xv[K];
      read_block<K, BF16>(regX + (wv * 64 + lane) * BLK_IN, xv);
      read_block<K, BF16>(regX + NL * BLK_IN + (wv * 64 + lane) * BLK_IN, dl);
#pragma unroll
      for (int i = 0; i < K; ++i) {
        dx[i] = dl[i] * xv[i];
        yv[i] = Dd * xv[i];
      }
    }
    float sumd = 0.0f;
#pragma unroll
    for (int i = 0; i < K; ++i) sumd += dl[i];
    if (PASS == 1) dsum_seg += wave_sum(sumd);

    for (int n = 0; n < N; ++n) {
      if (n > 0) __syncthreads();
      const int buf = n & 1;
      // prefetch the slices of state n+1 into registers (written to the other buffer below)
      float4 pre[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
      int preu[2] = {-1, -1};
      if (n + 1 < N) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int u = threadIdx.x + r * nthr;
          if (u < (PASS == 2 ? 2 : 1) * nq) {
            const int tsr = u / nq, q = u - tsr * nq;
            const int64_t t = t0 + 4 * q;
            const float* src = (tsr == 0 ? p.BT : p.CT) + (b * N + n + 1) * p.lpad;
            if (t < p.lpad) pre[r] = *reinterpret_cast<const float4*>(src + t);
            preu[r] = u;
          }
        }
      }
      const float a2 = lane_value(a2vec, n);
      const float hc = lane_value(hcvec, n);
      const float* bb = regBC + ((buf * 2 + 0) * 64 + lane) * BLK_BC;
      float ab[K], uu[K];
      float bacc = 0.0f;
#pragma unroll
      for (int q = 0; q < K / 4; ++q) {
        const float4 bv = *reinterpret_cast<const float4*>(bb + 4 * q);
        const float bq[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * q + e;
          ab[i] = fast_exp2(dl[i] * a2);
          uu[i] = dx[i] * bq[e];
          bacc = __builtin_fmaf(ab[i], bacc, uu[i]);
        }
      }
      float a = fast_exp2(a2 * sumd);
      float bs = bacc;
      wave_scan_pairs(a, bs);
      const float v = __builtin_fmaf(a, hc, bs);  // state after this lane's last step
      hcvec = set_lane(hcvec, lane_value(v, 63), n);
      if (PASS == 2) {
        float h = dpp_or<0x138, 0xF>(hc, v);  // wave_shr:1 -> state entering this lane's steps
        const float* cc = regBC + ((buf * 2 + 1) * 64 + lane) * BLK_BC;
#pragma unroll
        for (int q = 0; q < K / 4; ++q) {
          const float4 cv = *reinterpret_cast<const float4*>(cc + 4 * q);
          const float cq[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * q + e;
            h = __builtin_fmaf(ab[i], h, uu[i]);
            yv[i] = __builtin_fmaf(cq[e], h, yv[i]);
          }
        }
      }
      if (n + 1 < N) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          if (preu[r] >= 0) {
            const int tsr = preu[r] / nq, q = preu[r] - tsr * nq;
            const int jb = (4 * q) / K, ib = (4 * q) - jb * K;
            *reinterpret_cast<float4*>(regBC + (((buf ^ 1) * 2 + tsr) * 64 + jb) * BLK_BC + ib) = pre[r];
          }
        }
      }
    }
    __syncthreads();  // B/C buffers free; x/delta tiles long consumed

    if (PASS == 2) {
      if (p.z != nullptr) {
        stage_tile<K, BF16>(reinterpret_cast<unsigned char*>(regBC), p.z, b, t0, tend, p.L, p.D, d0, wpb, p.vec4);
        __syncthreads();
        float zv[K];
        read_block<K, BF16>(reinterpret_cast<unsigned char*>(regBC) + (wv * 64 + lane) * BLK_IN, zv);
#pragma unroll
        for (int i = 0; i < K; ++i) yv[i] *= silu(zv[i]);
      }
      // y tile (fp32) -> LDS -> coalesced rows
      float* yb = reinterpret_cast<float*>(regX + (wv * 64 + lane) * BLK_Y);
#pragma unroll
      for (int q = 0; q < K / 4; ++q)
        *reinterpret_cast<float4*>(yb + 4 * q) = make_float4(yv[4 * q], yv[4 * q + 1], yv[4 * q + 2], yv[4 * q + 3]);
      __syncthreads();
      if (p.vec4) {
        const int G = wpb >> 2;
        for (int u = threadIdx.x; u < CHUNK * G; u += nthr) {
          const int row = u / G, g = u - row * G;
          const int64_t t = t0 + row;
          const int c0 = g * 4;
          if (t < tend && d0 + c0 < p.D) {
            const int jb = row / K, ib = row - jb * K;
            const float* src = reinterpret_cast<const float*>(regX) + (c0 * 64 + jb) * (BLK_Y / 4) + ib;
            float4 v = make_float4(src[0], src[64 * (BLK_Y / 4)], src[2 * 64 * (BLK_Y / 4)], src[3 * 64 * (BLK_Y / 4)]);
            *reinterpret_cast<float4*>(p.y + (b * p.L + t) * p.D + d0 + c0) = v;
          }
        }
      } else {
        for (int u = threadIdx.x; u < CHUNK * wpb; u += nthr) {
          const int row = u / wpb, c = u - row * wpb;
          const int64_t t = t0 + row;
          if (t < tend && d0 + c < p.D) {
            const int jb = row / K, ib = row - jb * K;
            p.y[(b * p.L + t) * p.D + d0 + c] = reinterpret_cast<const float*>(regX)[(c * 64 + jb) * (BLK_Y / 4) + ib];
          }
        }
      }
      __syncthreads();  // y tile read before the next chunk restages regX
    }
  }

  if (!dvalid) return;
  if (PASS == 1) {
    if (lane == 0) p.seg_dsum[(b * p.S + s) * p.D + d] = dsum_seg;
    if (lane < N) p.seg_state[((b * p.S + s) * p.D + d) * N + lane] = hcvec;
  } else if (p.h_last != nullptr && s == p.S - 1) {
    if (lane < N) p.h_last[(b * p.D + d) * N + lane] = hcvec;
  }
}

// ------------------------------------------------------------------ host side
static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

static int lds_bytes(int k, bool bf16, int wpb) {
  const int es = bf16 ? 2 : 4;
  const int nl = wpb * 64;
  const int blk_in = k * es + 16, blk_y = k * 4 + 16;
  const int szx = std::max(2 * nl * blk_in, nl * blk_y);
  const int szbc = std::max(2 * 2 * 64 * (k + 4) * 4, nl * blk_in);
  return szx + szbc;
}

SelPlan plan_selective(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int num_cus) {
  SelPlan pl{};
  pl.k = env_int("SSS_K", 16) == 8 ? 8 : 16;
  pl.wpb = 4;
  pl.vec4 = (dim % 4 == 0) ? 1 : 0;
  const int64_t chunk = 64 * pl.k;
  // one wave per (channel, segment); aim for >= 8 waves per CU before splitting time
  const int64_t waves = batch * dim;
  const int64_t target = (int64_t)std::max(num_cus, 1) * 8;
  int64_t S = 1;
  if (waves < target) S = (target + waves - 1) / waves;
  const int64_t max_seg = (seqlen + chunk - 1) / chunk;  // at least one chunk per segment
  S = std::min<int64_t>(S, max_seg);
  S = std::min<int64_t>(S, 256);
  const int forced = env_int("SSS_FORCE_SEGMENTS", 0);
  if (forced > 0) S = std::min<int64_t>(forced, max_seg);
  if (S < 1) S = 1;
  int64_t seg_len = (seqlen + S - 1) / S;
  seg_len = (seg_len + chunk - 1) / chunk * chunk;
  S = (seqlen + seg_len - 1) / seg_len;
  pl.segments = (int)S;
  pl.seg_len = seg_len;
  pl.lpad = (seqlen + 3) / 4 * 4;
  size_t off = 0;
  pl.ws_bt = off;
  off = align_up(off + (size_t)batch * dstate * pl.lpad * 4, 256);
  pl.ws_ct = off;
  off = align_up(off + (size_t)batch * dstate * pl.lpad * 4, 256);
  pl.ws_state = off;
  off = align_up(off + (S > 1 ? (size_t)batch * S * dim * dstate * 4 : 0), 256);
  pl.ws_dsum = off;
  off = align_up(off + (S > 1 ? (size_t)batch * S * dim * 4 : 0), 256);
  pl.ws_total = off;
  return pl;
}

template <int K, bool BF16, int PASS>
static hipError_t launch_pass(const SelParams& sp, int nwg, int wpb, hipStream_t stream) {
  const int lds = lds_bytes(K, BF16, wpb);
  hipLaunchKernelGGL((sel_scan_kernel<K, BF16, PASS>), dim3(nwg), dim3(64 * wpb), lds, stream, sp);
  return hipGetLastError();
}

template <int K, bool BF16>
static hipError_t run_passes(const SelParams& sp, const SelPlan& pl, hipStream_t stream) {
  const int64_t per_seg = (int64_t)sp.ntiles * sp.batch;
  hipError_t e = hipSuccess;
  if (pl.segments > 1) {
    e = launch_pass<K, BF16, 1>(sp, (int)(per_seg * (pl.segments - 1)), pl.wpb, stream);
    if (e != hipSuccess) return e;
  }
  return launch_pass<K, BF16, 2>(sp, (int)(per_seg * pl.segments), pl.wpb, stream);
}

hipError_t launch_selective(const SelArgs& a, const SelPlan& pl, hipStream_t stream) {
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  float* bt = reinterpret_cast<float*>(ws + pl.ws_bt);
  float* ct = reinterpret_cast<float*>(ws + pl.ws_ct);
  const int64_t ntt = (pl.lpad + 63) / 64;
  hipLaunchKernelGGL(bc_transpose_kernel, dim3((unsigned)(a.batch * ntt)), dim3(256), 0, stream, a.B, bt,
                     a.seqlen, pl.lpad, a.dstate, ntt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bc_transpose_kernel, dim3((unsigned)(a.batch * ntt)), dim3(256), 0, stream, a.C, ct,
                     a.seqlen, pl.lpad, a.dstate, ntt);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  SelParams sp{};
  sp.x = a.x;
  sp.delta = a.delta;
  sp.A = a.A;
  sp.BT = bt;
  sp.CT = ct;
  sp.Dsk = a.Dsk;
  sp.z = a.z;
  sp.h0 = a.h0;
  sp.y = a.y;
  sp.h_last = a.h_last;
  sp.seg_state = pl.segments > 1 ? reinterpret_cast<float*>(ws + pl.ws_state) : nullptr;
  sp.seg_dsum = pl.segments > 1 ? reinterpret_cast<float*>(ws + pl.ws_dsum) : nullptr;
  sp.batch = a.batch;
  sp.L = a.seqlen;
  sp.D = a.dim;
  sp.lpad = pl.lpad;
  sp.seg_len = pl.seg_len;
  sp.N = a.dstate;
  sp.S = pl.segments;
  sp.wpb = pl.wpb;
  sp.ntiles = (int)((a.dim + pl.wpb - 1) / pl.wpb);
  sp.vec4 = pl.vec4;
  if (pl.k == 8)
    return a.bf16 ? run_passes<8, true>(sp, pl, stream) : run_passes<8, false>(sp, pl, stream);
  return a.bf16 ? run_passes<16, true>(sp, pl, stream) : run_passes<16, false>(sp, pl, stream);
}

}  // namespace sss
