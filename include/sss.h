/*
 * sss.h -- C ABI of the MI355X (gfx950) selective-scan library, libsss.so.
 *
 * Five operations, all fully computed by hand-written HIP kernels on the device:
 *
 *  selective_scan_fwd  -- the selective (input-dependent) state-space recurrence of
 *      "Selective Scan trong Mamba toi uu chuoi dai the nao?" (thecsnote.cc), sections
 *      "Tai sao Mamba can Selective Scan?" and "Selection pha vo convolution kernel co
 *      dinh": per batch b, channel d and state n, with zero-order-hold decay
 *        Abar_t[n] = exp(delta_t * A[d,n]),
 *        h_t[n]    = Abar_t[n] * h_{t-1}[n] + delta_t * B_t[n] * x_t,
 *        y_t       = (sum_n C_t[n] * h_t[n] + D[d] * x_t) * silu(z_t)   (D, z optional),
 *      h_{-1} = h0 (or 0), read-out after the update, final state h_{L-1} returned.
 *      delta arrives already passed through softplus: the projections that produce
 *      delta, B and C are outside this library ("15. Selective (Data-Dependent) SSM
 *      Scan", Problem: the data-dependent parameters are given); selective_scan_fwd_ex
 *      applies the bias and softplus itself, among its other options.
 *
 *  selective_scan_bwd -- its gradients (training), with the states recomputed;
 *      selective_scan_bwd_ex the same through the delta bias and softplus;
 *      selective_scan_fwd_save / selective_scan_bwd_saved the same pair with the forward
 *      call's segment entering states kept for the gradients call.
 *
 *  selective_state_update -- one decode step of the same recurrence on a carried state
 *      (in place), for token-by-token generation.
 *
 *  causal_conv1d_fwd -- the causal depthwise convolution (+ silu) that produces the
 *      scan's input x in the Mamba block.
 *
 *  elementwise_scan -- the per-channel form of "15. Selective (Data-Dependent) SSM
 *      Scan" (Reference solution): h = A_t*h + B_t*x_t, y_t = C_t*h.
 *
 * Conventions (all calls)
 *  - Pointers are DEVICE pointers owned by the caller.  Inputs are read-only; outputs
 *    may not overlap any input (SSS_ERR_ALIAS); the decode step's state is the one
 *    in/out buffer.  Every pointer must be 16-byte aligned (SSS_ERR_UNSUPPORTED otherwise).
 *  - Layout is row-major, all indices 64-bit:
 *      x, delta, z, y : (batch, seqlen, dim)        -- dim fastest
 *      B, C           : (batch, seqlen, dstate)
 *      A              : (dim, dstate)                -- selective form
 *      D_skip         : (dim)
 *      h0, h_last     : (batch, dim, dstate)         -- (batch, dim) for elementwise
 *  - Work is enqueued on `stream` and the call returns without synchronising.  Launch
 *    failures come back as SSS_ERR_HIP; a fault inside a kernel shows up at the
 *    caller's next synchronisation.
 *  - All validation happens before any device work; a rejected call writes nothing.
 *  - Workspace: caller-allocated device memory of at least *_workspace_size() bytes
 *    (may be NULL when that size is 0).  It is stream-ordered scratch: do not share
 *    one workspace between calls that may run concurrently.
 *  - The library allocates no device memory and keeps no state between calls other
 *    than a per-device cache of the compute-unit count.  Calls are thread-safe.
 *  - Environment: SSS_FORCE_SEGMENTS=<S> forces the number of time segments (the
 *    two-pass split) for testing; SSS_LOG=1 prints the chosen launch plan to stderr;
 *    SSS_WAVES_PER_SIMD / SSS_CONV_WAVES_PER_CU override the occupancy targets the
 *    selective-scan and convolution plans aim at, SSS_EW_CPL (1, 2 or 4) the channels per
 *    lane of the elementwise scan (tuning only).  SSS_CHUNKED=1 runs the plain time-major
 *    forward call (4, 8 or 16 states, no options) as one pass with a workgroup-level scan of the
 *    affine pairs instead of the two-pass split (measured slower on MI355X; kept for comparison
 *    and tests).
 */
#ifndef SSS_H_
#define SSS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP stream handle (same type as hip/hip_runtime_api.h's hipStream_t). */
typedef struct ihipStream_t* sss_stream_t;

/* dtype of x, delta and z for selective_scan_fwd; every other tensor is float32. */
typedef enum { SSS_F32 = 0, SSS_BF16 = 1 } sss_dtype;

typedef enum {
  SSS_OK = 0,
  SSS_ERR_NULL_ARG = -1,    /* a required pointer is NULL                             */
  SSS_ERR_BAD_DIM = -2,     /* a dimension is < 1, a size overflows, or dim > 2^24    */
  SSS_ERR_UNSUPPORTED = -3, /* dstate not in {1,2,4,8,16,32,64}, unknown dtype, or a
                               pointer not 16-byte aligned                             */
  SSS_ERR_WORKSPACE = -4,   /* workspace smaller than the size query (or NULL)        */
  SSS_ERR_ALIAS = -5,       /* an output overlaps an input or another output           */
  SSS_ERR_HIP = -6          /* no usable device, or a HIP launch/runtime error         */
} sss_status;

/* Bytes of workspace selective_scan_fwd needs for these sizes on `device`
 * (0 on invalid sizes).  Depends on the launch plan, hence on the device. */
size_t selective_scan_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                         int device);

/* Selective scan (Mamba form).  Required: x, delta (io_dtype), A, B, C (float32), y.
 * Optional (NULL): D_skip, z (io_dtype), h0 (NULL = zero state), h_last.
 * y and h_last are float32.  Returns an sss_status. */
int selective_scan_fwd(const void* x, const void* delta, const float* A, const float* B, const float* C,
                       const float* D_skip, const void* z, const float* h0, float* y, float* h_last,
                       int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                       void* workspace, size_t workspace_bytes, sss_stream_t stream);

/* Bytes of workspace selective_scan_bwd needs for these sizes on `device`. */
size_t selective_scan_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int device);

/* Gradients of the selective scan (plain form: first-order input term, no delta options),
 * for training: with L = sum(dy * y) + sum(dh_last * h_last) over selective_scan_fwd's
 * outputs, writes dL/d of every input.  The states are recomputed, not stored ("Selective
 * Scan trong Mamba toi uu chuoi dai the nao?", section "Recomputation: doi mot it compute
 * lay it memory hon"), and the adjoint runs backwards in time:
 *   lambda_t = C_t dv_t + exp(delta_{t+1} A) lambda_{t+1},  dv_t = dy_t silu(z_t).
 * Inputs as selective_scan_fwd, plus dy (batch, seqlen, dim) float32 and dh_last
 * (batch, dim, dstate) float32 (NULL = 0).  Outputs, all float32, caller-owned:
 *   dx, ddelta, dz (batch, seqlen, dim); dA (dim, dstate); dB, dC (batch, seqlen, dstate);
 *   dD (dim); dh0 (batch, dim, dstate).
 * Required: x, delta, A, B, C, dy, dx, ddelta, dA, dB, dC; dD when D_skip is given and dz
 * when z is given (SSS_ERR_NULL_ARG otherwise); dh0 optional (gradient of the initial
 * state, zero or h0).  Outputs may not overlap inputs, each other or the workspace.
 * dim * dstate * 4 must stay below 2^31 (SSS_ERR_BAD_DIM).
 * Workspace: at least selective_scan_bwd_workspace_size() bytes (never zero).  The sums
 * over channels (dB, dC) and over time (dA, dD) are formed from per-wave / per-segment
 * partials in a fixed order: results are deterministic.  Returns an sss_status. */
int selective_scan_bwd(const void* x, const void* delta, const float* A, const float* B, const float* C,
                       const float* D_skip, const void* z, const float* h0, const float* dy, const float* dh_last,
                       float* dx, float* ddelta, float* dA, float* dB, float* dC, float* dD, float* dz, float* dh0,
                       int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype, void* workspace,
                       size_t workspace_bytes, sss_stream_t stream);

/* selective_scan_bwd_ex: the gradients through the delta front end of selective_scan_fwd_ex
 * (the step size is delta + delta_bias[d], then softplus of it with SSS_DELTA_SOFTPLUS: "Selective
 * Scan trong Mamba toi uu chuoi dai the nao?", section "Selection pha vo convolution kernel co
 * dinh", where the step is a softplus of a bias plus a projection of the input; the pages give
 * no gradient, this is the chain rule through that front end).  The loss is that of
 * selective_scan_bwd over selective_scan_fwd_ex's outputs for the same delta_bias and flags.
 * Arguments as selective_scan_bwd, plus:
 *   delta_bias (dim) float32, nullable (no bias); flags: 0 or SSS_DELTA_SOFTPLUS (any other
 *   bit, the exact hold and the channel-major layout included: SSS_ERR_UNSUPPORTED);
 *   ddelta_bias (dim) float32 output, required when delta_bias is given (SSS_ERR_NULL_ARG),
 *   ignored otherwise: the sum over batch and time of ddelta.
 * ddelta is the gradient with respect to the STORED delta: the step size's gradient times
 * sigmoid(delta + bias) under softplus (the slope of softplus), times 1 with the bias alone.
 * With delta_bias NULL and flags 0 it is exactly selective_scan_bwd.  Same workspace size,
 * overlap rules (delta_bias is an input, ddelta_bias an output) and determinism.  Returns an
 * sss_status. */
int selective_scan_bwd_ex(const void* x, const void* delta, const float* A, const float* B, const float* C,
                          const float* D_skip, const void* z, const float* h0, const float* dy, const float* dh_last,
                          const float* delta_bias, unsigned flags, float* dx, float* ddelta, float* dA, float* dB,
                          float* dC, float* dD, float* dz, float* dh0, float* ddelta_bias, int64_t batch,
                          int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype, void* workspace,
                          size_t workspace_bytes, sss_stream_t stream);

/* Training pair that keeps the forward call's segment entering states instead of recomputing
 * them in the gradients call.  Only the state at each time segment's start is kept, a
 * fraction (segments / seqlen) of the state the recurrence forms; everything else is still
 * recomputed ("Selective Scan trong Mamba toi uu chuoi dai the nao?", section
 * "Recomputation: doi mot it compute lay it memory hon").
 *
 * selective_scan_states_size: bytes of that buffer for these sizes on `device` (0 when the
 * plan has a single time segment: nothing to keep; 0 as well on invalid sizes).  Layout
 * [segments][batch][dstate][dim] float32, opaque to the caller; it depends only on the sizes
 * and the device (the forward call's plan), so the size query is the contract. */
size_t selective_scan_states_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int device);

/* selective_scan_fwd_save: exactly selective_scan_fwd (same arguments, results bitwise the
 * same), and the segment entering states left in `states` (caller-owned device buffer of at
 * least selective_scan_states_size() bytes; may be NULL when that is 0; it may not overlap
 * any input, output or the workspace: SSS_ERR_ALIAS; too small: SSS_ERR_WORKSPACE). */
int selective_scan_fwd_save(const void* x, const void* delta, const float* A, const float* B, const float* C,
                            const float* D_skip, const void* z, const float* h0, float* y, float* h_last,
                            float* states, size_t states_bytes, int64_t batch, int64_t seqlen, int64_t dim,
                            int64_t dstate, int io_dtype, void* workspace, size_t workspace_bytes,
                            sss_stream_t stream);

/* selective_scan_bwd_saved: selective_scan_bwd (same arguments, the same gradients up to
 * rounding) with the segment entering states read from `states` instead of recomputed: its
 * checkpoint pass starts every time segment from its kept entering state, where
 * selective_scan_bwd starts each from zero and adds the decayed entering state to the
 * checkpoints afterwards (the scan is linear in its state: the same values summed in another
 * order; bitwise the same when the plan has a single segment).  `states` must hold what selective_scan_fwd_save
 * wrote for the same x, delta, A, B, h0, sizes, dtype and device (C, D, z do not enter the
 * states), unmodified since; the library cannot check that, and anything else gives wrong
 * gradients.  Read only; NULL allowed when selective_scan_states_size() is 0.  Size and
 * overlap rules as for selective_scan_fwd_save (the inputs may share it: it is read only). */
int selective_scan_bwd_saved(const void* x, const void* delta, const float* A, const float* B, const float* C,
                             const float* D_skip, const void* z, const float* h0, const float* dy,
                             const float* dh_last, const float* states, size_t states_bytes, float* dx, float* ddelta,
                             float* dA, float* dB, float* dC, float* dD, float* dz, float* dh0, int64_t batch,
                             int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype, void* workspace,
                             size_t workspace_bytes, sss_stream_t stream);

/* One decode step of the selective scan ("Selective Scan trong Mamba toi uu chuoi dai the
 * nao?", section "Selective Scan thay doi inference chuoi dai nhu the nao?": generation
 * carries only the state from token to token), for one token per batch row:
 *   state[b,d,n] = exp(delta[b,d]*A[d,n]) * state[b,d,n] + delta[b,d]*B[b,n]*x[b,d]
 *   y[b,d]       = (sum_n C[b,n]*state[b,d,n] + D[d]*x[b,d]) * silu(z[b,d])
 * i.e. exactly selective_scan_fwd over a length-1 sequence with h0 = h_last = state.
 * Layouts: x, delta, z (batch, dim) in io_dtype; B, C (batch, dstate); A (dim, dstate);
 * D_skip (dim); state (batch, dim, dstate) float32, read and overwritten IN PLACE (the
 * only buffer that is both input and output); y (batch, dim) float32.
 * Required: x, delta, A, B, C, state, y.  Optional (NULL): D_skip, z.  No workspace.
 * Errors as above; state and y may not overlap any other argument (SSS_ERR_ALIAS);
 * batch*dim*dstate must not exceed 2^31 (SSS_ERR_BAD_DIM).  Returns an sss_status. */
int selective_state_update(const void* x, const void* delta, const float* A, const float* B, const float* C,
                           const float* D_skip, const void* z, float* state, float* y, int64_t batch, int64_t dim,
                           int64_t dstate, int io_dtype, sss_stream_t stream);

/* Options of selective_scan_fwd_ex (bit flags). */
typedef enum {
  SSS_EXACT_ZOH = 1u,      /* input term expm1(delta*A[d,n])/A[d,n] * B_t[n] * x_t, the exact
                              zero-order hold of the Python example in "Selective Scan trong
                              Mamba ..." (delta * B_t[n] where A[d,n] == 0), instead of the
                              first-order delta * B_t[n] * x_t                                 */
  SSS_DELTA_SOFTPLUS = 2u, /* step size softplus(delta (+ delta_bias[d])): the front end that
                              turns the projected delta into a positive step                  */
  SSS_LAYOUT_BDL = 4u      /* channel-major operands, time fastest: x, delta, z, y are
                              (batch, dim, seqlen) and B, C are (batch, dstate, seqlen); A,
                              D_skip, h0, h_last and delta_bias keep their layouts.  seqlen
                              must stay below 2^23 (SSS_ERR_BAD_DIM).  Rows of a multiple of 8
                              (bf16) / 4 (fp32) steps stream as 16-byte pieces per lane      */
} sss_flags;

/* Bytes of workspace selective_scan_fwd_ex needs for these sizes and flags on `device` (0 on
 * invalid sizes or flags).  SSS_LAYOUT_BDL adds time-major copies of B and C. */
size_t selective_scan_fwd_ex_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                            unsigned flags, int device);

/* selective_scan_fwd with options: `delta_bias` (dim) float32, nullable, is added to delta
 * before use (and before softplus); `flags` is a combination of sss_flags (unknown bits:
 * SSS_ERR_UNSUPPORTED).  With delta_bias == NULL and flags == 0 it is selective_scan_fwd.
 * Workspace: at least selective_scan_fwd_ex_workspace_size() bytes for the same flags.
 * Layouts as selective_scan_fwd unless SSS_LAYOUT_BDL; ownership and errors the same. */
int selective_scan_fwd_ex(const void* x, const void* delta, const float* A, const float* B, const float* C,
                          const float* D_skip, const void* z, const float* h0, float* y, float* h_last,
                          const float* delta_bias, unsigned flags, int64_t batch, int64_t seqlen, int64_t dim,
                          int64_t dstate, int io_dtype, void* workspace, size_t workspace_bytes,
                          sss_stream_t stream);

/* Causal depthwise convolution that feeds the scan in the Mamba block ("Toan Canh Tien Hoa
 * Kien Truc AI ...", section "5.3. Toi uu hoa Kernel Fusion cho Mamba SSM": the
 * causal_conv1d kernel), per channel d with `width` taps:
 *   out[b,t,d] = bias[d] + sum_{k<width} weight[d,k] * x[b, t-(width-1)+k, d]
 * with x = 0 before t = 0, then silu(out) if apply_silu.  x and out (batch, seqlen, dim) in
 * io_dtype (a bf16 out is rounded to nearest even); weight (dim, width) and bias (dim,
 * nullable) float32.  Required: x, weight, out.  width in 1..8 (SSS_ERR_UNSUPPORTED
 * otherwise).  out may not overlap x, weight or bias.  No workspace.  Returns an sss_status. */
int causal_conv1d_fwd(const void* x, const float* weight, const float* bias, void* out, int64_t batch,
                      int64_t seqlen, int64_t dim, int64_t width, int io_dtype, int apply_silu, sss_stream_t stream);

/* Bytes of workspace elementwise_scan needs for these sizes on `device`. */
size_t elementwise_scan_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int device);

/* Elementwise scan, all float32.  Required: x, A, B, C, y.  Optional: h0, h_last. */
int elementwise_scan(const float* x, const float* A, const float* B, const float* C, const float* h0, float* y,
                     float* h_last, int64_t batch, int64_t seqlen, int64_t dim, void* workspace,
                     size_t workspace_bytes, sss_stream_t stream);

/* Scratch bytes of selective_scan_fwd_noalloc (a device array held by every GPU the library
 * runs on, until the process ends). */
#define SSS_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)

/* selective_scan_fwd for callers that cannot allocate device memory: code being captured into
 * a HIP graph, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, layouts,
 * results and errors as selective_scan_fwd, without the workspace: the call's scratch (the
 * segment states of the time split) lives in a file-scope device array of
 * SSS_NOALLOC_SCRATCH_BYTES per GPU, and the call allocates nothing (no hipMalloc, no
 * allocating library routine).  The launch plan is sized to that array (fewer time segments
 * where the usual plan would need more scratch; a single segment needs none, so no valid shape
 * is refused for its size), so results may differ from selective_scan_fwd's by rounding order.
 * All calls on one GPU share its array: calls that may overlap on one GPU (other streams or
 * host threads) race, and the caller must order them.  The array keeps the last call's
 * contents; nothing in it needs clearing.  Returns an sss_status (SSS_ERR_HIP if the array's
 * address cannot be obtained on the current device). */
int selective_scan_fwd_noalloc(const void* x, const void* delta, const float* A, const float* B, const float* C,
                               const float* D_skip, const void* z, const float* h0, float* y, float* h_last,
                               int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                               sss_stream_t stream);

/* Human-readable name of a status code (static string). */
const char* sss_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SSS_H_ */
