// api.cpp -- the C ABI of libsss.so (declared in include/sss.h): argument validation,
// launch planning and dispatch to the gfx950 kernels.  No device memory is allocated here.
#include "sss.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "kernels.h"

namespace sss {

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (v == nullptr || *v == '\0') return dflt;
  return std::atoi(v);
}

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];  // 0 = unknown

// Compute units of `device` (cached); -1 if it cannot be queried.
int device_cus(int device) {
  if (device < 0 || device >= kMaxDevices) return -1;
  int v = g_cus[device].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    return -1;
  }
  g_cus[device].store(cus, std::memory_order_relaxed);
  return cus;
}

int current_device_cus() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  return device_cus(dev);
}

// Sizes in bytes with overflow checks; false when a product leaves [0, 2^62).
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > (int64_t(1) << 62) / a) return false;
  *out = a * b;
  return true;
}

struct Range {
  uintptr_t lo, hi;
};

bool overlap(const void* p, int64_t bytes, const void* q, int64_t qbytes) {
  if (p == nullptr || q == nullptr || bytes <= 0 || qbytes <= 0) return false;
  uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + (uintptr_t)qbytes && b < a + (uintptr_t)bytes;
}

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace sss

using namespace sss;

extern "C" {

const char* sss_status_string(int status) {
  switch (status) {
    case SSS_OK: return "SSS_OK";
    case SSS_ERR_NULL_ARG: return "SSS_ERR_NULL_ARG: a required pointer is NULL";
    case SSS_ERR_BAD_DIM: return "SSS_ERR_BAD_DIM: a dimension is < 1 or a size is too large";
    case SSS_ERR_UNSUPPORTED: return "SSS_ERR_UNSUPPORTED: dstate not in {1,2,4,8,16,32,64}, unknown dtype or misaligned pointer";
    case SSS_ERR_WORKSPACE: return "SSS_ERR_WORKSPACE: workspace missing or smaller than the size query";
    case SSS_ERR_ALIAS: return "SSS_ERR_ALIAS: an output overlaps an input, another output or the workspace";
    case SSS_ERR_HIP: return "SSS_ERR_HIP: no usable HIP device or a launch failed";
    default: return "unknown sss status";
  }
}

constexpr int64_t kMaxSelDim = (int64_t)1 << 24;  // largest dim of either call

static int sel_dims_ok(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  if (batch < 1 || seqlen < 1 || dim < 1 || dstate < 1) return SSS_ERR_BAD_DIM;
  int64_t e = 0, t = 0;
  if (!mul_ok(batch, seqlen, &t) || !mul_ok(t, dim, &e) || !mul_ok(e, 4, &t)) return SSS_ERR_BAD_DIM;
  if (!mul_ok(batch, seqlen, &t) || !mul_ok(t, dstate, &e) || !mul_ok(e, 4, &t)) return SSS_ERR_BAD_DIM;
  if (dim > kMaxSelDim) return SSS_ERR_BAD_DIM;                              // 32-bit buffer offsets
  if (batch * ((dim + 3) / 4) > (int64_t)1 << 30) return SSS_ERR_BAD_DIM;  // grid size
  if (dstate > 64 || (dstate & (dstate - 1)) != 0) return SSS_ERR_UNSUPPORTED;
  return SSS_OK;
}

size_t selective_scan_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int device) {
  return selective_scan_fwd_ex_workspace_size(batch, seqlen, dim, dstate, 0u, device);
}

static constexpr unsigned kKnownFlags = SSS_EXACT_ZOH | SSS_DELTA_SOFTPLUS | SSS_LAYOUT_BDL;
// channel-major rows: a lane's row offset (up to 64 rows of seqlen fp32 values) stays a
// 32-bit buffer offset
static constexpr int64_t kMaxBdlSeqlen = ((int64_t)1 << 23) - 1;

size_t selective_scan_fwd_ex_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                            unsigned flags, int device) {
  if (sel_dims_ok(batch, seqlen, dim, dstate) != SSS_OK || (flags & ~kKnownFlags) != 0) return 0;
  const bool bdl = (flags & SSS_LAYOUT_BDL) != 0;
  if (bdl && seqlen > kMaxBdlSeqlen) return 0;
  int cus = device_cus(device);
  if (cus <= 0) cus = 256;
  return plan_selective(batch, seqlen, dim, dstate, cus, bdl).ws_total;
}

int selective_scan_fwd(const void* x, const void* delta, const float* A, const float* B, const float* C,
                       const float* D_skip, const void* z, const float* h0, float* y, float* h_last,
                       int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                       void* workspace, size_t workspace_bytes, sss_stream_t stream) {
  return selective_scan_fwd_ex(x, delta, A, B, C, D_skip, z, h0, y, h_last, nullptr, 0u, batch, seqlen, dim, dstate,
                               io_dtype, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace sss {
// Validation, planning and launch of the forward call.  max_ws > 0 limits the plan's
// workspace to max_ws bytes (fewer time segments when the usual plan needs more).
int sel_fwd_impl(const void* x, const void* delta, const float* A, const float* B, const float* C,
                 const float* D_skip, const void* z, const float* h0, float* y, float* h_last,
                 const float* delta_bias, unsigned flags, int64_t batch, int64_t seqlen, int64_t dim,
                 int64_t dstate, int io_dtype, void* workspace, size_t workspace_bytes, size_t max_ws,
                 void* stream, bool save_states, float* states, size_t states_bytes) {
  if (!x || !delta || !A || !B || !C || !y) return SSS_ERR_NULL_ARG;
  int st = sel_dims_ok(batch, seqlen, dim, dstate);
  if (st != SSS_OK) return st;
  if (io_dtype != SSS_F32 && io_dtype != SSS_BF16) return SSS_ERR_UNSUPPORTED;
  if ((flags & ~kKnownFlags) != 0) return SSS_ERR_UNSUPPORTED;
  const bool bdl = (flags & SSS_LAYOUT_BDL) != 0;
  if (bdl && seqlen > kMaxBdlSeqlen) return SSS_ERR_BAD_DIM;
  const void* ptrs[] = {x, delta, A, B, C, D_skip, z, h0, y, h_last, workspace, delta_bias, states};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SSS_ERR_UNSUPPORTED;
  const int64_t es = io_dtype == SSS_BF16 ? 2 : 4;
  const int64_t E = batch * seqlen * dim;
  const int64_t y_bytes = E * 4, hl_bytes = batch * dim * dstate * 4;
  const void* in_p[] = {x, delta, A, B, C, D_skip, z, h0, delta_bias};
  const int64_t in_b[] = {E * es, E * es, dim * dstate * 4, batch * seqlen * dstate * 4,
                          batch * seqlen * dstate * 4, dim * 4, E * es, batch * dim * dstate * 4, dim * 4};
  for (int i = 0; i < 9; ++i) {
    if (overlap(y, y_bytes, in_p[i], in_b[i])) return SSS_ERR_ALIAS;
    if (overlap(h_last, hl_bytes, in_p[i], in_b[i])) return SSS_ERR_ALIAS;
  }
  if (overlap(y, y_bytes, h_last, hl_bytes)) return SSS_ERR_ALIAS;
  const int cus = current_device_cus();
  if (cus <= 0) return SSS_ERR_HIP;
  const SelPlan pl = plan_selective(batch, seqlen, dim, dstate, cus, bdl, max_ws);
  // threads of the widest launch: 64 per channel group (padded to whole workgroups of 4)
  // and segment; must fit a 1-D grid
  const int64_t wg_groups = ((dim + 63) / 64 + 3) / 4 * 4;
  if ((double)batch * (double)wg_groups * 64.0 * (double)pl.segments > 2147483647.0) return SSS_ERR_BAD_DIM;
  if (pl.ws_total > 0) {
    if (workspace == nullptr || workspace_bytes < pl.ws_total) return SSS_ERR_WORKSPACE;
    const int64_t wb = (int64_t)pl.ws_total;
    if (overlap(workspace, wb, y, y_bytes) || overlap(workspace, wb, h_last, hl_bytes)) return SSS_ERR_ALIAS;
    for (int i = 0; i < 9; ++i)
      if (overlap(workspace, wb, in_p[i], in_b[i])) return SSS_ERR_ALIAS;
  }
  // the saved segment entering states (plain form only): a caller buffer in place of the
  // workspace's slots, so that they outlive the call
  const int64_t sb = save_states && pl.segments > 1 ? (int64_t)pl.segments * batch * dstate * dim * 4 : 0;
  if (save_states) {
    if (flags != 0) return SSS_ERR_UNSUPPORTED;
    if (sb > 0) {
      if (states == nullptr) return SSS_ERR_NULL_ARG;
      if (states_bytes < (size_t)sb) return SSS_ERR_WORKSPACE;
      if (overlap(states, sb, y, y_bytes) || overlap(states, sb, h_last, hl_bytes) ||
          overlap(states, sb, workspace, (int64_t)pl.ws_total))
        return SSS_ERR_ALIAS;
      for (int i = 0; i < 9; ++i)
        if (overlap(states, sb, in_p[i], in_b[i])) return SSS_ERR_ALIAS;
    }
  }
  SelArgs a{};
  a.x = x;
  a.delta = delta;
  a.A = A;
  a.B = B;
  a.C = C;
  a.Dsk = D_skip;
  a.z = z;
  a.h0 = h0;
  a.y = y;
  a.h_last = h_last;
  a.batch = batch;
  a.seqlen = seqlen;
  a.dim = dim;
  a.dstate = (int)dstate;
  a.bf16 = io_dtype == SSS_BF16;
  a.workspace = workspace;
  a.delta_bias = delta_bias;
  a.softplus = (flags & SSS_DELTA_SOFTPLUS) != 0;
  a.exact_zoh = (flags & SSS_EXACT_ZOH) != 0;
  a.bdl = bdl;
  a.states = sb > 0 ? states : nullptr;
  // the single-pass form with the workgroup pair scan: forced on (1) or off (0) by SSS_CHUNKED
  // (never when the states are saved: it forms none)
  const int chunked_env = env_int("SSS_CHUNKED", -1);
  const bool chunked = !save_states && chunk_scan_supported(a) && chunked_env == 1;
  if (env_int("SSS_LOG", 0)) {
    static const char* const kRows[] = {"time-major", "step", "piece", "tile"};
    if (chunked)
      std::fprintf(stderr, "[sss] selective_scan_fwd B=%lld L=%lld D=%lld N=%lld %s flags=%u: single pass, "
                   "workgroup pair scan\n", (long long)batch, (long long)seqlen, (long long)dim, (long long)dstate,
                   io_dtype == SSS_BF16 ? "bf16" : "f32", flags);
    else
      std::fprintf(stderr,
                   "[sss] selective_scan_fwd B=%lld L=%lld D=%lld N=%lld %s flags=%u: segments=%d seg_len=%lld rows=%s "
                   "ws=%zu\n",
                   (long long)batch, (long long)seqlen, (long long)dim, (long long)dstate,
                   io_dtype == SSS_BF16 ? "bf16" : "f32", flags, pl.segments, (long long)pl.seg_len,
                   kRows[selective_row_mode(a, pl)], pl.ws_total);
  }
  hipError_t e = chunked ? launch_chunk_scan(a, reinterpret_cast<hipStream_t>(stream))
                         : launch_selective(a, pl, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? SSS_OK : SSS_ERR_HIP;
}
}  // namespace sss

extern "C" {

int selective_scan_fwd_ex(const void* x, const void* delta, const float* A, const float* B, const float* C,
                          const float* D_skip, const void* z, const float* h0, float* y, float* h_last,
                          const float* delta_bias, unsigned flags, int64_t batch, int64_t seqlen, int64_t dim,
                          int64_t dstate, int io_dtype, void* workspace, size_t workspace_bytes,
                          sss_stream_t stream) {
  return sel_fwd_impl(x, delta, A, B, C, D_skip, z, h0, y, h_last, delta_bias, flags, batch, seqlen, dim, dstate,
                      io_dtype, workspace, workspace_bytes, 0, stream);
}

size_t selective_scan_states_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int device) {
  if (sel_dims_ok(batch, seqlen, dim, dstate) != SSS_OK) return 0;
  int cus = device_cus(device);
  if (cus <= 0) cus = 256;
  const SelPlan pl = plan_selective(batch, seqlen, dim, dstate, cus);
  return pl.segments > 1 ? (size_t)pl.segments * batch * dstate * dim * 4 : 0;
}

int selective_scan_fwd_save(const void* x, const void* delta, const float* A, const float* B, const float* C,
                            const float* D_skip, const void* z, const float* h0, float* y, float* h_last,
                            float* states, size_t states_bytes, int64_t batch, int64_t seqlen, int64_t dim,
                            int64_t dstate, int io_dtype, void* workspace, size_t workspace_bytes,
                            sss_stream_t stream) {
  return sel_fwd_impl(x, delta, A, B, C, D_skip, z, h0, y, h_last, nullptr, 0u, batch, seqlen, dim, dstate, io_dtype,
                      workspace, workspace_bytes, 0, stream, true, states, states_bytes);
}


size_t selective_scan_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int device) {
  if (sel_dims_ok(batch, seqlen, dim, dstate) != SSS_OK) return 0;
  int cus = device_cus(device);
  if (cus <= 0) cus = 256;
  return plan_selective_bwd(batch, seqlen, dim, dstate, cus).ws_total;
}

}  // extern "C"

namespace sss {
// The gradients call: validation, plan, launch.  states: the segment entering states a
// selective_scan_fwd_save call left (nullptr: recomputed).
static int sel_bwd_impl(const void* x, const void* delta, const float* A, const float* B, const float* C,
                        const float* D_skip, const void* z, const float* h0, const float* dy, const float* dh_last,
                        float* dx, float* ddelta, float* dA, float* dB, float* dC, float* dD, float* dz, float* dh0,
                        int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype, const float* states,
                        size_t states_bytes, bool use_states, void* workspace, size_t workspace_bytes,
                        sss_stream_t stream, const float* delta_bias = nullptr, unsigned flags = 0u,
                        float* ddelta_bias = nullptr) {
  if (!x || !delta || !A || !B || !C || !dy || !dx || !ddelta || !dA || !dB || !dC) return SSS_ERR_NULL_ARG;
  if ((D_skip && !dD) || (z && !dz) || (delta_bias && !ddelta_bias)) return SSS_ERR_NULL_ARG;
  if ((flags & ~(unsigned)SSS_DELTA_SOFTPLUS) != 0) return SSS_ERR_UNSUPPORTED;
  int st = sel_dims_ok(batch, seqlen, dim, dstate);
  if (st != SSS_OK) return st;
  if (dim * dstate * 4 >= ((int64_t)1 << 31)) return SSS_ERR_BAD_DIM;  // checkpoint rows: 32-bit offsets
  if (io_dtype != SSS_F32 && io_dtype != SSS_BF16) return SSS_ERR_UNSUPPORTED;
  const void* ptrs[] = {x, delta, A, B, C, D_skip, z, h0, dy, dh_last, dx, ddelta, dA, dB, dC, dD, dz, dh0, workspace,
                        states, delta_bias, ddelta_bias};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SSS_ERR_UNSUPPORTED;
  const int64_t es = io_dtype == SSS_BF16 ? 2 : 4;
  const int64_t E = batch * seqlen * dim, H = batch * dim * dstate * 4, BC = batch * seqlen * dstate * 4;
  const void* in_p[] = {x, delta, A, B, C, D_skip, z, h0, dy, dh_last, delta_bias};
  const int64_t in_b[] = {E * es, E * es, dim * dstate * 4, BC, BC, dim * 4, E * es, H, E * 4, H, dim * 4};
  void* out_p[] = {dx, ddelta, dA, dB, dC, dD, dz, dh0, delta_bias ? ddelta_bias : nullptr};
  const int64_t out_b[] = {E * 4, E * 4, dim * dstate * 4, BC, BC, dim * 4, E * 4, H, dim * 4};
  for (int i = 0; i < 9; ++i) {
    for (int j = 0; j < 11; ++j)
      if (overlap(out_p[i], out_b[i], in_p[j], in_b[j])) return SSS_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlap(out_p[i], out_b[i], out_p[j], out_b[j])) return SSS_ERR_ALIAS;
  }
  const int cus = current_device_cus();
  if (cus <= 0) return SSS_ERR_HIP;
  const BwdPlan bp = plan_selective_bwd(batch, seqlen, dim, dstate, cus);
  const int64_t wg_groups = (dim + 63) / 64;
  if ((double)batch * (double)wg_groups * (double)bp.fwd.segments > 2147483647.0 / 64) return SSS_ERR_BAD_DIM;
  if (workspace == nullptr || workspace_bytes < bp.ws_total) return SSS_ERR_WORKSPACE;
  const int64_t wb = (int64_t)bp.ws_total;
  for (int i = 0; i < 11; ++i)
    if (overlap(workspace, wb, in_p[i], in_b[i])) return SSS_ERR_ALIAS;
  for (int i = 0; i < 9; ++i)
    if (overlap(workspace, wb, out_p[i], out_b[i])) return SSS_ERR_ALIAS;
  // saved states: exactly the forward plan's slots
  const int64_t sb = bp.fwd.segments > 1 ? (int64_t)bp.fwd.segments * batch * dstate * dim * 4 : 0;
  if (use_states && sb > 0) {
    if (states == nullptr) return SSS_ERR_NULL_ARG;
    if (states_bytes < (size_t)sb) return SSS_ERR_WORKSPACE;
    if (overlap(states, sb, workspace, wb)) return SSS_ERR_ALIAS;
    for (int i = 0; i < 8; ++i)
      if (overlap(states, sb, out_p[i], out_b[i])) return SSS_ERR_ALIAS;
  }
  if (env_int("SSS_LOG", 0))
    std::fprintf(stderr,
                 "[sss] selective_scan_bwd B=%lld L=%lld D=%lld N=%lld flags=%u bias=%d: segments=%d seg_len=%lld K=%d "
                 "checkpoint every %d ws=%zu\n",
                 (long long)batch, (long long)seqlen, (long long)dim, (long long)dstate, flags, delta_bias ? 1 : 0,
                 bp.fwd.segments,
                 (long long)bp.fwd.seg_len, bp.K, bp.KC, bp.ws_total);
  BwdArgs a{};
  a.fwd.x = x;
  a.fwd.delta = delta;
  a.fwd.A = A;
  a.fwd.B = B;
  a.fwd.C = C;
  a.fwd.Dsk = D_skip;
  a.fwd.z = z;
  a.fwd.h0 = h0;
  a.fwd.batch = batch;
  a.fwd.seqlen = seqlen;
  a.fwd.dim = dim;
  a.fwd.dstate = (int)dstate;
  a.fwd.bf16 = io_dtype == SSS_BF16;
  a.fwd.workspace = workspace;
  a.dy = dy;
  a.dh_last = dh_last;
  a.dx = dx;
  a.ddelta = ddelta;
  a.dA = dA;
  a.dB = dB;
  a.dC = dC;
  a.dD = dD;
  a.dz = dz;
  a.dh0 = dh0;
  a.fwd.delta_bias = delta_bias;
  a.fwd.softplus = (flags & SSS_DELTA_SOFTPLUS) != 0;
  a.ddelta_bias = delta_bias ? ddelta_bias : nullptr;
  a.states_ready = use_states && sb > 0;
  a.fwd.states = a.states_ready ? const_cast<float*>(states) : nullptr;  // read only
  return launch_selective_bwd(a, bp, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? SSS_OK : SSS_ERR_HIP;
}
}  // namespace sss

extern "C" {

int selective_scan_bwd(const void* x, const void* delta, const float* A, const float* B, const float* C,
                       const float* D_skip, const void* z, const float* h0, const float* dy, const float* dh_last,
                       float* dx, float* ddelta, float* dA, float* dB, float* dC, float* dD, float* dz, float* dh0,
                       int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype, void* workspace,
                       size_t workspace_bytes, sss_stream_t stream) {
  return sel_bwd_impl(x, delta, A, B, C, D_skip, z, h0, dy, dh_last, dx, ddelta, dA, dB, dC, dD, dz, dh0, batch,
                      seqlen, dim, dstate, io_dtype, nullptr, 0, false, workspace, workspace_bytes, stream);
}

int selective_scan_bwd_ex(const void* x, const void* delta, const float* A, const float* B, const float* C,
                          const float* D_skip, const void* z, const float* h0, const float* dy, const float* dh_last,
                          const float* delta_bias, unsigned flags, float* dx, float* ddelta, float* dA, float* dB,
                          float* dC, float* dD, float* dz, float* dh0, float* ddelta_bias, int64_t batch,
                          int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype, void* workspace,
                          size_t workspace_bytes, sss_stream_t stream) {
  return sel_bwd_impl(x, delta, A, B, C, D_skip, z, h0, dy, dh_last, dx, ddelta, dA, dB, dC, dD, dz, dh0, batch,
                      seqlen, dim, dstate, io_dtype, nullptr, 0, false, workspace, workspace_bytes, stream, delta_bias,
                      flags, ddelta_bias);
}

int selective_scan_bwd_saved(const void* x, const void* delta, const float* A, const float* B, const float* C,
                             const float* D_skip, const void* z, const float* h0, const float* dy,
                             const float* dh_last, const float* states, size_t states_bytes, float* dx, float* ddelta,
                             float* dA, float* dB, float* dC, float* dD, float* dz, float* dh0, int64_t batch,
                             int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype, void* workspace,
                             size_t workspace_bytes, sss_stream_t stream) {
  return sel_bwd_impl(x, delta, A, B, C, D_skip, z, h0, dy, dh_last, dx, ddelta, dA, dB, dC, dD, dz, dh0, batch,
                      seqlen, dim, dstate, io_dtype, states, states_bytes, true, workspace, workspace_bytes, stream);
}

int selective_state_update(const void* x, const void* delta, const float* A, const float* B, const float* C,
                           const float* D_skip, const void* z, float* state, float* y, int64_t batch, int64_t dim,
                           int64_t dstate, int io_dtype, sss_stream_t stream) {
  if (!x || !delta || !A || !B || !C || !state || !y) return SSS_ERR_NULL_ARG;
  if (batch < 1 || dim < 1 || dstate < 1 || dim > kMaxSelDim) return SSS_ERR_BAD_DIM;
  int64_t e = 0, t = 0;
  if (!mul_ok(batch, dim, &e) || !mul_ok(e, dstate, &t) || t > ((int64_t)1 << 31)) return SSS_ERR_BAD_DIM;
  // grid: ceil(dim * lanes per channel / 256) blocks per batch row, one row after another
  if ((double)batch * (double)((dim * std::max<int64_t>(dstate / 4, 1) + 255) / 256) > 2147483647.0)
    return SSS_ERR_BAD_DIM;
  if (dstate > 64 || (dstate & (dstate - 1)) != 0) return SSS_ERR_UNSUPPORTED;
  if (io_dtype != SSS_F32 && io_dtype != SSS_BF16) return SSS_ERR_UNSUPPORTED;
  const void* ptrs[] = {x, delta, A, B, C, D_skip, z, state, y};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SSS_ERR_UNSUPPORTED;
  const int64_t es = io_dtype == SSS_BF16 ? 2 : 4;
  const int64_t st_bytes = batch * dim * dstate * 4, y_bytes = batch * dim * 4;
  const void* in_p[] = {x, delta, A, B, C, D_skip, z};
  const int64_t in_b[] = {e * es, e * es, dim * dstate * 4, batch * dstate * 4, batch * dstate * 4, dim * 4, e * es};
  for (int i = 0; i < 7; ++i) {
    if (overlap(state, st_bytes, in_p[i], in_b[i])) return SSS_ERR_ALIAS;
    if (overlap(y, y_bytes, in_p[i], in_b[i])) return SSS_ERR_ALIAS;
  }
  if (overlap(y, y_bytes, state, st_bytes)) return SSS_ERR_ALIAS;
  if (current_device_cus() <= 0) return SSS_ERR_HIP;
  UpdArgs a{};
  a.x = x;
  a.delta = delta;
  a.A = A;
  a.B = B;
  a.C = C;
  a.Dsk = D_skip;
  a.z = z;
  a.state = state;
  a.y = y;
  a.batch = batch;
  a.dim = dim;
  a.dstate = (int)dstate;
  a.bf16 = io_dtype == SSS_BF16;
  return launch_update(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? SSS_OK : SSS_ERR_HIP;
}

int causal_conv1d_fwd(const void* x, const float* weight, const float* bias, void* out, int64_t batch,
                      int64_t seqlen, int64_t dim, int64_t width, int io_dtype, int apply_silu, sss_stream_t stream) {
  if (!x || !weight || !out) return SSS_ERR_NULL_ARG;
  if (batch < 1 || seqlen < 1 || dim < 1 || width < 1 || dim > kMaxSelDim) return SSS_ERR_BAD_DIM;
  int64_t e = 0, t = 0;
  if (!mul_ok(batch, seqlen, &t) || !mul_ok(t, dim, &e) || !mul_ok(e, 4, &t)) return SSS_ERR_BAD_DIM;
  if (width > 8) return SSS_ERR_UNSUPPORTED;
  if (io_dtype != SSS_F32 && io_dtype != SSS_BF16) return SSS_ERR_UNSUPPORTED;
  const void* ptrs[] = {x, weight, bias, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SSS_ERR_UNSUPPORTED;
  const int64_t es = io_dtype == SSS_BF16 ? 2 : 4;
  if (overlap(out, e * es, x, e * es) || overlap(out, e * es, weight, dim * width * 4) ||
      overlap(out, e * es, bias, dim * 4))
    return SSS_ERR_ALIAS;
  const int cus = current_device_cus();
  if (cus <= 0) return SSS_ERR_HIP;
  const ConvPlan pl = plan_conv1d(batch, seqlen, dim, io_dtype == SSS_BF16, cus);
  if (env_int("SSS_LOG", 0))
    std::fprintf(stderr, "[sss] causal_conv1d_fwd B=%lld L=%lld D=%lld W=%lld: segments=%d seg_len=%lld cpl=%d\n",
                 (long long)batch, (long long)seqlen, (long long)dim, (long long)width, pl.segments,
                 (long long)pl.seg_len, pl.cpl);
  if ((double)batch * (double)((dim + 63) / 64) * (double)pl.segments > 2147483647.0 / 64) return SSS_ERR_BAD_DIM;
  ConvArgs a{};
  a.x = x;
  a.w = weight;
  a.bias = bias;
  a.out = out;
  a.batch = batch;
  a.seqlen = seqlen;
  a.dim = dim;
  a.width = (int)width;
  a.bf16 = io_dtype == SSS_BF16;
  a.silu = apply_silu != 0;
  return launch_conv1d(a, pl, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? SSS_OK : SSS_ERR_HIP;
}

static int ew_dims_ok(int64_t batch, int64_t seqlen, int64_t dim) {
  if (batch < 1 || seqlen < 1 || dim < 1) return SSS_ERR_BAD_DIM;
  int64_t e = 0, t = 0;
  if (!mul_ok(batch, seqlen, &t) || !mul_ok(t, dim, &e) || !mul_ok(e, 4, &t)) return SSS_ERR_BAD_DIM;
  if (dim > kMaxSelDim) return SSS_ERR_BAD_DIM;                     // 32-bit buffer offsets
  if (batch * ((dim + 63) / 64) > (int64_t)1 << 30) return SSS_ERR_BAD_DIM;
  return SSS_OK;
}

size_t elementwise_scan_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int device) {
  if (ew_dims_ok(batch, seqlen, dim) != SSS_OK) return 0;
  int cus = device_cus(device);
  if (cus <= 0) cus = 256;
  return plan_elementwise(batch, seqlen, dim, cus).ws_total;
}

int elementwise_scan(const float* x, const float* A, const float* B, const float* C, const float* h0, float* y,
                     float* h_last, int64_t batch, int64_t seqlen, int64_t dim, void* workspace,
                     size_t workspace_bytes, sss_stream_t stream) {
  if (!x || !A || !B || !C || !y) return SSS_ERR_NULL_ARG;
  int st = ew_dims_ok(batch, seqlen, dim);
  if (st != SSS_OK) return st;
  const void* ptrs[] = {x, A, B, C, h0, y, h_last, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SSS_ERR_UNSUPPORTED;
  const int64_t E = batch * seqlen * dim * 4, H = batch * dim * 4;
  const void* in_p[] = {x, A, B, C, h0};
  const int64_t in_b[] = {E, E, E, E, H};
  for (int i = 0; i < 5; ++i) {
    if (overlap(y, E, in_p[i], in_b[i])) return SSS_ERR_ALIAS;
    if (overlap(h_last, H, in_p[i], in_b[i])) return SSS_ERR_ALIAS;
  }
  if (overlap(y, E, h_last, H)) return SSS_ERR_ALIAS;
  const int cus = current_device_cus();
  if (cus <= 0) return SSS_ERR_HIP;
  const EwPlan pl = plan_elementwise(batch, seqlen, dim, cus);
  // one wave per (batch, 64-channel group, segment) must fit a 1-D grid
  if ((double)batch * (double)((dim + 63) / 64) * (double)pl.segments > 2147483647.0 / 64) return SSS_ERR_BAD_DIM;
  if (pl.ws_total > 0) {
    if (workspace == nullptr || workspace_bytes < pl.ws_total) return SSS_ERR_WORKSPACE;
    const int64_t wb = (int64_t)pl.ws_total;
    if (overlap(workspace, wb, y, E) || overlap(workspace, wb, h_last, H)) return SSS_ERR_ALIAS;
    for (int i = 0; i < 5; ++i)
      if (overlap(workspace, wb, in_p[i], in_b[i])) return SSS_ERR_ALIAS;
  }
  if (env_int("SSS_LOG", 0))
    std::fprintf(stderr, "[sss] elementwise_scan B=%lld L=%lld D=%lld: segments=%d seg_len=%lld cpl=%d ws=%zu\n",
                 (long long)batch, (long long)seqlen, (long long)dim, pl.segments, (long long)pl.seg_len, pl.cpl,
                 pl.ws_total);
  EwArgs a{};
  a.x = x;
  a.A = A;
  a.B = B;
  a.C = C;
  a.h0 = h0;
  a.y = y;
  a.h_last = h_last;
  a.batch = batch;
  a.seqlen = seqlen;
  a.dim = dim;
  a.workspace = workspace;
  hipError_t e = launch_elementwise(a, pl, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? SSS_OK : SSS_ERR_HIP;
}

}  // extern "C"
