// kernels.h -- launch interface between the C-ABI host code and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sss {

// Launch plan of the selective scan (chosen on the host, see selective_scan.hip).
struct SelPlan {
  int segments;      // time segments S (S > 1: segment states, carry, then outputs)
  int64_t seg_len;   // steps per segment (multiple of the load batch)
  size_t ws_state, ws_dsum, ws_bc, ws_total;  // workspace offsets / total bytes
};

struct SelArgs {
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
  int64_t batch, seqlen, dim;
  int dstate;
  int bf16;
  void* workspace;
  const float* delta_bias;  // nullable: added to delta before use
  int softplus;             // step size = softplus(delta (+ bias))
  int exact_zoh;            // input term expm1(delta*A)/A * B instead of delta * B
  int bdl;                  // x/delta/z/y (batch, dim, seqlen), B/C (batch, dstate, seqlen)
  float* states;            // nullable: the segment entering states [S][batch][dstate][dim] live
                            // here instead of in the workspace (kept for the backward pass)
};

// max_ws > 0: at most max_ws bytes of workspace (fewer segments if the usual plan needs more)
SelPlan plan_selective(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int num_cus, bool bdl = false,
                       size_t max_ws = 0);
hipError_t launch_selective(const SelArgs& a, const SelPlan& plan, hipStream_t stream);
// single-pass form with the workgroup-level pair scan (chunk_scan.hip): which calls it takes,
// and the launch (no workspace)
bool chunk_scan_supported(const SelArgs& a);
hipError_t launch_chunk_scan(const SelArgs& a, hipStream_t stream);
// the whole forward call (api.cpp): validation, plan (workspace at most max_ws bytes when
// max_ws > 0), launch; returns an sss_status
int sel_fwd_impl(const void* x, const void* delta, const float* A, const float* B, const float* C,
                 const float* D_skip, const void* z, const float* h0, float* y, float* h_last,
                 const float* delta_bias, unsigned flags, int64_t batch, int64_t seqlen, int64_t dim,
                 int64_t dstate, int io_dtype, void* workspace, size_t workspace_bytes, size_t max_ws,
                 void* stream, bool save_states = false, float* states = nullptr, size_t states_bytes = 0);
// how the forward kernels walk the rows: 0 time-major; channel-major 1 one step per access,
// 2 16-byte pieces per lane, 3 tiles staged through LDS
int selective_row_mode(const SelArgs& a, const SelPlan& plan);
// pass 1 + carry only: the workspace's state slots hold the state entering each segment
hipError_t launch_segment_states(const SelArgs& a, const SelPlan& plan, hipStream_t stream);
// the state before every 2^kshift-th step of every segment, into
// ckpt[s][batch][channel group][j][dstate + 1][64 lanes] (ceil(dim / 64) groups); with adj_mu
// (more than one segment) also the adjoint of every segment folded from zero at its end into
// adj_mu[s][batch][dstate][dim], dy (batch, seqlen, dim) being the output gradient, and every
// segment's delta sum into the workspace's sums.  Without `local`, after
// launch_segment_states (or with states kept by the forward call): the checkpoints are the
// states.  With `local` (adj_mu, more than one segment) every segment starts from zero: the
// checkpoints hold the states from zero and, in row dstate, the delta sum of the segment's
// steps before them, and the state slots end up holding the entering states (end states
// from zero, then the carry)
hipError_t launch_checkpoints(const SelArgs& a, const SelPlan& plan, float* ckpt, int kshift, int nsub,
                              const float* dy, float* adj_mu, bool local, hipStream_t stream);

// Backward pass of the selective scan (selective_bwd.hip).
struct BwdPlan {
  SelPlan fwd;     // segments of the forward pass (its workspace comes first)
  int K, KC, nsub; // steps per sub-chunk, checkpoint spacing (a multiple of K), checkpoints
                   // per segment
  size_t off_mu, off_ckpt, off_bc, off_pa, off_pd, off_pdb, ws_total;
};

struct BwdArgs {
  SelArgs fwd;  // forward inputs (y / h_last unused)
  const float* dy;
  const float* dh_last;
  float* dx;
  float* ddelta;
  float* dA;
  float* dB;
  float* dC;
  float* dD;
  float* dz;
  float* dh0;
  float* ddelta_bias;  // with the delta front end (fwd.delta_bias / fwd.softplus): d/d bias
  bool states_ready;  // fwd.states already holds the segment entering states (saved by the forward)
};

BwdPlan plan_selective_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int num_cus);
hipError_t launch_selective_bwd(const BwdArgs& a, const BwdPlan& plan, hipStream_t stream);

struct EwPlan {
  int segments;
  int64_t seg_len;
  size_t ws_total;
  int cpl;  // adjacent channels per lane (1, 2 or 4)
};

struct EwArgs {
  const float* x;
  const float* A;
  const float* B;
  const float* C;
  const float* h0;
  float* y;
  float* h_last;
  int64_t batch, seqlen, dim;
  void* workspace;
};

EwPlan plan_elementwise(int64_t batch, int64_t seqlen, int64_t dim, int num_cus);
hipError_t launch_elementwise(const EwArgs& a, const EwPlan& plan, hipStream_t stream);

struct UpdArgs {
  const void* x;
  const void* delta;
  const float* A;
  const float* B;
  const float* C;
  const float* Dsk;
  const void* z;
  float* state;
  float* y;
  int64_t batch, dim;
  int dstate;
  int bf16;
};

hipError_t launch_update(const UpdArgs& a, hipStream_t stream);

struct ConvPlan {
  int segments;
  int64_t seg_len;
  int cpl;  // channels per lane (adjacent), 1 or 8 bytes' worth
};

struct ConvArgs {
  const void* x;
  const float* w;
  const float* bias;
  void* out;
  int64_t batch, seqlen, dim;
  int width;
  int bf16;
  int silu;
};

ConvPlan plan_conv1d(int64_t batch, int64_t seqlen, int64_t dim, bool bf16, int num_cus);
hipError_t launch_conv1d(const ConvArgs& a, const ConvPlan& plan, hipStream_t stream);

int env_int(const char* name, int dflt);

}  // namespace sss
