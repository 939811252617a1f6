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
// its affine pair (prod A, state from zero), pass 2 folds the earlier segments' pairs into
// the entering state and streams the outputs.
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
  float* seg_a;  // (S, batch*dim): product of A over the segment
  float* seg_b;  // (S, batch*dim): segment end state from a zero state
  int64_t batch, L, D, seg_len;
  int S;
};

constexpr int kU = 8;  // steps per load batch

template <int PASS>
__global__ __launch_bounds__(64) void ew_scan_kernel(EwParams p) {
  const int64_t nch = p.batch * p.D;
  const int64_t nblk_ch = (nch + 63) / 64;
  const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t cblk = lid % nblk_ch;
  const int s = (int)(lid / nblk_ch);
  const int64_t ch = cblk * 64 + threadIdx.x;
  if (ch >= nch) return;
  const int64_t b = ch / p.D, d = ch - b * p.D;
  const int64_t tbeg = (int64_t)s * p.seg_len;
  const int64_t tend = min(tbeg + p.seg_len, p.L);
  const int64_t D = p.D;
  const int64_t base = b * p.L * D + d;

  float h = 0.0f;
  float aprod = 1.0f;
  if (PASS == 2) {
    h = p.h0 ? p.h0[ch] : 0.0f;
    for (int s2 = 0; s2 < s; ++s2) h = __builtin_fmaf(p.seg_a[(int64_t)s2 * nch + ch], h, p.seg_b[(int64_t)s2 * nch + ch]);
  }

  float ra[2][kU], rb[2][kU], rx[2][kU], rc[2][kU];
  auto load = [&](int slot, int64_t t0) {
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      const int64_t t = t0 + i;
      const bool ok = t < tend;
      const int64_t o = base + t * D;
      ra[slot][i] = ok ? __builtin_nontemporal_load(p.A + o) : 1.0f;
      rb[slot][i] = ok ? __builtin_nontemporal_load(p.B + o) : 0.0f;
      rx[slot][i] = ok ? __builtin_nontemporal_load(p.x + o) : 0.0f;
      if (PASS == 2) rc[slot][i] = ok ? __builtin_nontemporal_load(p.C + o) : 0.0f;
    }
  };
  int64_t t0 = tbeg;
  if (t0 < tend) load(0, t0);
  int slot = 0;
  for (; t0 < tend; t0 += kU) {
    if (t0 + kU < tend) load(slot ^ 1, t0 + kU);
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      h = __builtin_fmaf(ra[slot][i], h, rb[slot][i] * rx[slot][i]);
      if (PASS == 1) {
        aprod *= ra[slot][i];
      } else {
        const int64_t t = t0 + i;
        if (t < tend) __builtin_nontemporal_store(rc[slot][i] * h, p.y + base + t * D);
      }
    }
    slot ^= 1;
  }
  if (PASS == 1) {
    p.seg_a[(int64_t)s * nch + ch] = aprod;
    p.seg_b[(int64_t)s * nch + ch] = h;
  } else if (p.h_last != nullptr && s == p.S - 1) {
    p.h_last[ch] = h;
  }
}

static size_t align_up_ew(size_t v, size_t a) { return (v + a - 1) / a * a; }

EwPlan plan_elementwise(int64_t batch, int64_t seqlen, int64_t dim, int num_cus) {
  EwPlan pl{};
  const int64_t nch = batch * dim;
  const int64_t waves = (nch + 63) / 64;
  const int64_t target = (int64_t)std::max(num_cus, 1) * 2;  // two streaming waves per CU
  int64_t S = 1;
  if (waves < target) S = (target + waves - 1) / waves;
  const int64_t max_seg = (seqlen + kU - 1) / kU;
  S = std::min<int64_t>(S, max_seg);
  S = std::min<int64_t>(S, 1024);
  const int forced = env_int("SSS_FORCE_SEGMENTS", 0);
  if (forced > 0) S = std::min<int64_t>(forced, max_seg);
  if (S < 1) S = 1;
  int64_t seg_len = (seqlen + S - 1) / S;
  seg_len = (seg_len + kU - 1) / kU * kU;
  S = (seqlen + seg_len - 1) / seg_len;
  pl.segments = (int)S;
  pl.seg_len = seg_len;
  pl.ws_total = S > 1 ? align_up_ew((size_t)S * nch * 4, 256) * 2 : 0;
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
  const int64_t nch = a.batch * a.dim;
  if (pl.segments > 1) {
    unsigned char* ws = static_cast<unsigned char*>(a.workspace);
    p.seg_a = reinterpret_cast<float*>(ws);
    p.seg_b = reinterpret_cast<float*>(ws + pl.ws_total / 2);
  }
  const int64_t nblk = (nch + 63) / 64;
  if (pl.segments > 1) {
    hipLaunchKernelGGL(ew_scan_kernel<1>, dim3((unsigned)(nblk * (pl.segments - 1))), dim3(64), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(ew_scan_kernel<2>, dim3((unsigned)(nblk * pl.segments)), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sss
