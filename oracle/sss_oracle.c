/*
 * sss_oracle.c -- plain, slow, fp64 CPU oracle for the selective scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
 * leg use it.  It shares no code, header, table or constant with the HIP path.
 *
 * Every floating-point input is read in its stored type (fp32, or the raw 16
 * bits of a bf16 value, widened exactly to fp32 and then to double) and all
 * arithmetic is done in double with libm's exp/expm1.  Channels (b, d) are
 * independent, so the only parallelism is an OpenMP loop over channels; the
 * arithmetic inside a channel is exactly the stepwise definition.
 *
 * Sources (web pages on the subject; cited by title and section):
 *  [P1] "Selective Scan trong Mamba toi uu chuoi dai the nao?" (thecsnote.cc):
 *       sections "Tai sao Mamba can Selective Scan?" (discrete SSM recurrence
 *       and readout), "Selection pha vo convolution kernel co dinh"
 *       (time-varying A_t, B_t, C_t and Delta_t), "Scan bien recurrence ..."
 *       (affine step as a pair, the compose rule and its identity), and the
 *       Python example (zero-order hold with diagonal A, sequential loop,
 *       prefix fold from the identity).
 *  [P3] "15. Selective (Data-Dependent) SSM Scan" (cartesia-pytorch problems):
 *       "Step-by-Step Approach" (update then read out from the updated state)
 *       and "Reference solution" (elementwise per-channel recurrence).
 *  The selective (Mamba) form with D skip, optional silu(z) gate, initial and
 *  final state, and the first-order input term Delta_t*B_t*x_t is the reading
 *  of those pages that the build targets (B-bar = Delta*B: the plain reading;
 *  the exact zero-order-hold B-bar of the P1 example is kept as an option).
 */
#include <math.h>
#include <stdlib.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_ERR_ARG -1

/* dtype codes for x / delta / z */
#define OR_F32 0
#define OR_BF16 1

/* Exact widening of a stored value to double. */
static double load_val(const void* p, int64_t i, int dtype) {
  if (dtype == OR_BF16) {
    uint16_t bits = ((const uint16_t*)p)[i];
    uint32_t w = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
  }
  return (double)((const float*)p)[i];
}

/* softplus(v) = log(1 + e^v), written so that neither branch overflows. */
static double softplus(double v) { return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v)); }

/* The step size actually used: the stored delta, plus the per-channel bias if one is
 * given, then through softplus if asked (the front end that produces delta in Mamba,
 * [P1] "Selection pha vo convolution kernel co dinh": Delta as a function of the input). */
static double delta_value(const void* delta, int64_t e, int dtype, const float* dbias, int64_t d, int sp) {
  double v = load_val(delta, e, dtype);
  if (dbias) v += (double)dbias[d];
  return sp ? softplus(v) : v;
}

/* Thread count of the next parallel region: nthreads if positive, else the process default
 * (taken on first use), so that a call with an explicit count does not change later calls. */
static int g_default_threads = 0;

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (g_default_threads == 0) g_default_threads = omp_get_max_threads();
  omp_set_num_threads(nthreads > 0 ? nthreads : g_default_threads);
#else
  (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return g_default_threads > 0 ? g_default_threads : omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Selective form, one channel (b, d) -- [P1] "Tai sao ..." / "Selection ...":
 *   h_{-1} = h0[b,d,:] (or 0)
 *   for t: Abar_t[n] = exp(Delta_t * A[d,n])
 *          h_t[n]    = Abar_t[n] * h_{t-1}[n] + Bbar_t[n] * x_t
 *          y_t       = sum_n C_t[n] * h_t[n]  (+ D[d] * x_t)  (* silu(z_t))
 *   with Bbar_t[n] = Delta_t * B_t[n]                      (exact_zoh == 0)
 *     or Bbar_t[n] = expm1(Delta_t*A[d,n]) / A[d,n] * B_t[n] (exact_zoh != 0,
 *        the P1 Python example's zero-order hold; Delta_t when A[d,n] == 0).
 *   The readout uses the state after the update ([P3] step 4).  Delta_t is the stored
 *   value, optionally plus dbias[d] and through softplus (delta_value).
 * Layouts: x, delta, z (B, L, D); B, C (B, L, N); A (D, N); D (D);
 *          h0, h_last (B, D, N).  Outputs: y_out[t * y_stride] for t < L,
 *          hl_out[n] for n < N.
 */
static void sel_channel(const void* x, const void* delta, const float* A, const float* Bm, const float* Cm,
                        const float* Dsk, const void* z, const float* h0, int64_t b, int64_t d, int64_t L,
                        int64_t Dm, int64_t N, int dtype, int exact_zoh, const float* dbias, int sp,
                        double* y_out, int64_t y_stride, double* hl_out, double* h /* scratch N */) {
  for (int64_t n = 0; n < N; ++n) h[n] = h0 ? (double)h0[(b * Dm + d) * N + n] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    int64_t e = (b * L + t) * Dm + d;
    double xt = load_val(x, e, dtype);
    double dt = delta_value(delta, e, dtype, dbias, d, sp);
    const float* Bt = Bm + (b * L + t) * N;
    const float* Ct = Cm + (b * L + t) * N;
    double v = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      double a = (double)A[d * N + n];
      double abar = exp(dt * a);
      double bbar;
      if (exact_zoh)
        bbar = (a != 0.0 ? expm1(dt * a) / a : dt) * (double)Bt[n];
      else
        bbar = dt * (double)Bt[n];
      h[n] = abar * h[n] + bbar * xt;
      v += (double)Ct[n] * h[n];
    }
    if (Dsk) v += (double)Dsk[d] * xt;
    if (z) {
      double zt = load_val(z, e, dtype);
      v *= zt / (1.0 + exp(-zt));
    }
    y_out[t * y_stride] = v;
  }
  if (hl_out)
    for (int64_t n = 0; n < N; ++n) hl_out[n] = h[n];
}

static int sel_args_ok(const void* x, const void* delta, const float* A, const float* Bm, const float* Cm,
                       int64_t batch, int64_t L, int64_t Dm, int64_t N, int dtype) {
  if (!x || !delta || !A || !Bm || !Cm) return 0;
  if (batch < 1 || L < 1 || Dm < 1 || N < 1 || N > 4096) return 0;
  if (dtype != OR_F32 && dtype != OR_BF16) return 0;
  return 1;
}

/* Full tensor: y (B, L, D) double, h_last (B, D, N) double (nullable). */
int oracle_selective_scan(const void* x, const void* delta, const float* A, const float* Bm, const float* Cm,
                          const float* Dsk, const void* z, const float* h0, double* y, double* h_last,
                          int64_t batch, int64_t L, int64_t Dm, int64_t N, int dtype, int exact_zoh,
                          const float* dbias, int sp, int nthreads) {
  if (!sel_args_ok(x, delta, A, Bm, Cm, batch, L, Dm, N, dtype) || !y) return OR_ERR_ARG;
  set_threads(nthreads);
  int64_t nch = batch * Dm;
#pragma omp parallel
  {
    double hbuf[4096];
#pragma omp for schedule(dynamic, 1)
    for (int64_t c = 0; c < nch; ++c) {
      int64_t b = c / Dm, d = c % Dm;
      sel_channel(x, delta, A, Bm, Cm, Dsk, z, h0, b, d, L, Dm, N, dtype, exact_zoh, dbias, sp, y + b * L * Dm + d, Dm,
                  h_last ? h_last + (b * Dm + d) * N : 0, hbuf);
    }
  }
  return OR_OK;
}

/* Chosen channels only: chan[k] = b * D + d.  y_out (nchan, L), hl_out (nchan, N) (nullable). */
int oracle_selective_scan_channels(const void* x, const void* delta, const float* A, const float* Bm,
                                   const float* Cm, const float* Dsk, const void* z, const float* h0,
                                   const int64_t* chan, int64_t nchan, double* y_out, double* hl_out,
                                   int64_t batch, int64_t L, int64_t Dm, int64_t N, int dtype, int exact_zoh,
                                   const float* dbias, int sp, int nthreads) {
  if (!sel_args_ok(x, delta, A, Bm, Cm, batch, L, Dm, N, dtype) || !chan || !y_out || nchan < 0)
    return OR_ERR_ARG;
  for (int64_t k = 0; k < nchan; ++k)
    if (chan[k] < 0 || chan[k] >= batch * Dm) return OR_ERR_ARG;
  set_threads(nthreads);
#pragma omp parallel
  {
    double hbuf[4096];
#pragma omp for schedule(dynamic, 1)
    for (int64_t k = 0; k < nchan; ++k) {
      int64_t b = chan[k] / Dm, d = chan[k] % Dm;
      sel_channel(x, delta, A, Bm, Cm, Dsk, z, h0, b, d, L, Dm, N, dtype, exact_zoh, dbias, sp, y_out + k * L, 1,
                  hl_out ? hl_out + k * N : 0, hbuf);
    }
  }
  return OR_OK;
}

/*
 * One recurrent-inference step of the selective form -- [P1] "Selective Scan thay doi
 * inference chuoi dai nhu the nao?" (generation carries only the state from token to
 * token) with the update and readout of "Tai sao ..." / "Selection ...":
 *   for each (b, d, n): h = exp(Delta[b,d] * A[d,n]) * state[b,d,n] + Delta[b,d] * B[b,n] * x[b,d]
 *   y[b,d] = (sum_n C[b,n] * h[b,d,n] + D[d] * x[b,d]) * silu(z[b,d])   (D, z optional)
 * Layouts: x, delta, z (B, D); B, C (B, N); A (D, N); D (D); state (B, D, N) fp32 in;
 * y (B, D) and state_out (B, D, N) in double.
 */
int oracle_selective_state_update(const void* x, const void* delta, const float* A, const float* Bm,
                                  const float* Cm, const float* Dsk, const void* z, const float* state,
                                  double* y, double* state_out, int64_t batch, int64_t Dm, int64_t N, int dtype,
                                  int nthreads) {
  if (!x || !delta || !A || !Bm || !Cm || !state || !y || !state_out) return OR_ERR_ARG;
  if (batch < 1 || Dm < 1 || N < 1 || N > 4096) return OR_ERR_ARG;
  if (dtype != OR_F32 && dtype != OR_BF16) return OR_ERR_ARG;
  set_threads(nthreads);
  int64_t nch = batch * Dm;
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < nch; ++c) {
    int64_t b = c / Dm, d = c % Dm;
    double xv = load_val(x, c, dtype);
    double dv = load_val(delta, c, dtype);
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      double h = exp(dv * (double)A[d * N + n]) * (double)state[c * N + n] + dv * (double)Bm[b * N + n] * xv;
      state_out[c * N + n] = h;
      acc += (double)Cm[b * N + n] * h;
    }
    if (Dsk) acc += (double)Dsk[d] * xv;
    if (z) {
      double zv = load_val(z, c, dtype);
      acc *= zv / (1.0 + exp(-zv));
    }
    y[c] = acc;
  }
  return OR_OK;
}

/*
 * Gradients of the selective form (first-order input term, no delta front end) by the
 * adjoint of the recurrence, walked backwards in time -- the training path of [P1]
 * "Recomputation: doi mot it compute lay it memory hon" (the states are recomputed here by
 * a forward sweep per channel, then the adjoint runs from t = L-1 down to 0):
 *   a_t = exp(Delta_t A_n), h_t = a_t h_{t-1} + Delta_t B_t[n] x_t,
 *   v_t = sum_n C_t[n] h_t[n] + D x_t, y_t = v_t * silu(z_t)
 *   dv_t = dy_t * silu(z_t);  dz_t = dy_t * v_t * silu'(z_t)
 *   lambda_t[n] = C_t[n] dv_t + a_{t+1}[n] lambda_{t+1}[n],  lambda_{L-1} += dh_last[n]
 *   dx_t = D dv_t + sum_n lambda_t Delta_t B_t[n]
 *   dDelta_t = sum_n lambda_t (B_t[n] x_t + A_n a_t h_{t-1})
 *   dA_n += lambda_t Delta_t a_t h_{t-1};  dB_t[n] += lambda_t Delta_t x_t (sum over d);
 *   dC_t[n] += dv_t h_t[n] (sum over d);  dD += dv_t x_t;  dh0 = a_0 lambda_0.
 * dy (B, L, D) and dh_last (B, D, N, nullable) are double.  Outputs in double: dx, ddelta,
 * dz (B, L, D; dz only with z), dA (D, N), dB, dC (B, L, N), dD (D), dh0 (B, D, N) (each
 * nullable where its input is optional).
 */
/*
 * The same gradients with the front end (delta_value): the step size used is
 * dt = softplus(delta + dbias[d]) (sp) or delta + dbias[d], and ddelta is the gradient with
 * respect to the stored delta -- the step-size gradient times dsoftplus/dv = sigmoid(v),
 * v = delta + dbias[d] -- and ddbias[d] (nullable) its sum over b and t (the chain rule through
 * the front end; reading of the build, the pages give the front end but no gradient).
 */
int oracle_selective_scan_bwd_ex(const void* x, const void* delta, const float* A, const float* Bm, const float* Cm,
                                 const float* Dsk, const void* z, const float* h0, const double* dy,
                                 const double* dh_last, const float* dbias, int sp, double* dx, double* ddelta,
                                 double* dA, double* dB, double* dC, double* dD, double* dz, double* dh0,
                                 double* ddbias, int64_t batch, int64_t L, int64_t Dm, int64_t N, int dtype,
                                 int nthreads);

int oracle_selective_scan_bwd(const void* x, const void* delta, const float* A, const float* Bm, const float* Cm,
                              const float* Dsk, const void* z, const float* h0, const double* dy,
                              const double* dh_last, double* dx, double* ddelta, double* dA, double* dB, double* dC,
                              double* dD, double* dz, double* dh0, int64_t batch, int64_t L, int64_t Dm, int64_t N,
                              int dtype, int nthreads) {
  return oracle_selective_scan_bwd_ex(x, delta, A, Bm, Cm, Dsk, z, h0, dy, dh_last, NULL, 0, dx, ddelta, dA, dB, dC,
                                      dD, dz, dh0, NULL, batch, L, Dm, N, dtype, nthreads);
}

int oracle_selective_scan_bwd_ex(const void* x, const void* delta, const float* A, const float* Bm, const float* Cm,
                                 const float* Dsk, const void* z, const float* h0, const double* dy,
                                 const double* dh_last, const float* dbias, int sp, double* dx, double* ddelta,
                                 double* dA, double* dB, double* dC, double* dD, double* dz, double* dh0,
                                 double* ddbias, int64_t batch, int64_t L, int64_t Dm, int64_t N, int dtype,
                                 int nthreads) {
  if (!sel_args_ok(x, delta, A, Bm, Cm, batch, L, Dm, N, dtype) || !dy || !dx || !ddelta || !dA || !dB || !dC)
    return OR_ERR_ARG;
  set_threads(nthreads);
  int64_t nch = batch * Dm;
  memset(dA, 0, sizeof(double) * Dm * N);
  memset(dB, 0, sizeof(double) * batch * L * N);
  memset(dC, 0, sizeof(double) * batch * L * N);
  if (dD) memset(dD, 0, sizeof(double) * Dm);
  if (ddbias) memset(ddbias, 0, sizeof(double) * Dm);
#pragma omp parallel
  {
    double* hs = (double*)malloc(sizeof(double) * (L + 1) * N);   /* h_{t-1} for t = 0..L */
    double* vs = (double*)malloc(sizeof(double) * L);
    double* lam = (double*)malloc(sizeof(double) * N);
    double* lB = (double*)calloc((size_t)(batch * L * N), sizeof(double));
    double* lC = (double*)calloc((size_t)(batch * L * N), sizeof(double));
    double* lA = (double*)calloc((size_t)(Dm * N), sizeof(double));
    double* lD = (double*)calloc((size_t)Dm, sizeof(double));
    double* lDb = (double*)calloc((size_t)Dm, sizeof(double));
#pragma omp for schedule(dynamic, 1)
    for (int64_t c = 0; c < nch; ++c) {
      int64_t b = c / Dm, d = c % Dm;
      /* forward: hs[(t+1)*N + n] = h_t, hs[n] = h_{-1} */
      for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? (double)h0[c * N + n] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        int64_t e = (b * L + t) * Dm + d;
        double xt = load_val(x, e, dtype), dt = delta_value(delta, e, dtype, dbias, d, sp);
        double v = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          double hn = exp(dt * (double)A[d * N + n]) * hs[t * N + n] + dt * (double)Bm[(b * L + t) * N + n] * xt;
          hs[(t + 1) * N + n] = hn;
          v += (double)Cm[(b * L + t) * N + n] * hn;
        }
        if (Dsk) v += (double)Dsk[d] * xt;
        vs[t] = v;
      }
      /* adjoint, backwards in time; lam holds a_{t+1} lambda_{t+1} on entry to step t */
      for (int64_t n = 0; n < N; ++n) lam[n] = dh_last ? dh_last[c * N + n] : 0.0;
      for (int64_t t = L - 1; t >= 0; --t) {
        int64_t e = (b * L + t) * Dm + d;
        double xt = load_val(x, e, dtype), dt = delta_value(delta, e, dtype, dbias, d, sp);
        double g = 1.0;
        if (z) {
          double zt = load_val(z, e, dtype);
          double sg = 1.0 / (1.0 + exp(-zt));
          g = zt * sg;
          if (dz) dz[e] = dy[e] * vs[t] * sg * (1.0 + zt * (1.0 - sg));
        }
        double dv = dy[e] * g;
        double gx = Dsk ? (double)Dsk[d] * dv : 0.0, gd = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          double an = (double)A[d * N + n];
          double Bn = (double)Bm[(b * L + t) * N + n], Cn = (double)Cm[(b * L + t) * N + n];
          double at = exp(dt * an);
          double l = Cn * dv + lam[n];                  /* lambda_t */
          double hp = hs[t * N + n];                    /* h_{t-1} */
          gx += l * dt * Bn;
          gd += l * (Bn * xt + an * at * hp);
          lA[d * N + n] += l * dt * at * hp;
          lB[(b * L + t) * N + n] += l * dt * xt;
          lC[(b * L + t) * N + n] += dv * hs[(t + 1) * N + n];
          lam[n] = at * l;                              /* a_t lambda_t, for step t-1 */
        }
        if (Dsk) lD[d] += dv * xt;
        dx[e] = gx;
        if (sp) { /* d softplus(v) / dv = sigmoid(v) */
          double vr = load_val(delta, e, dtype) + (dbias ? (double)dbias[d] : 0.0);
          gd *= 1.0 / (1.0 + exp(-vr));
        }
        ddelta[e] = gd;
        lDb[d] += gd;
      }
      if (dh0)
        for (int64_t n = 0; n < N; ++n) dh0[c * N + n] = lam[n];
    }
#pragma omp critical
    {
      for (int64_t i = 0; i < batch * L * N; ++i) {
        dB[i] += lB[i];
        dC[i] += lC[i];
      }
      for (int64_t i = 0; i < Dm * N; ++i) dA[i] += lA[i];
      if (dD)
        for (int64_t i = 0; i < Dm; ++i) dD[i] += lD[i];
      if (ddbias)
        for (int64_t i = 0; i < Dm; ++i) ddbias[i] += lDb[i];
    }
    free(lDb);
    free(hs);
    free(vs);
    free(lam);
    free(lB);
    free(lC);
    free(lA);
    free(lD);
  }
  return OR_OK;
}

/*
 * Causal depthwise convolution in front of the scan -- [P5] "5.3. Toi uu hoa Kernel Fusion
 * cho Mamba SSM" names the causal_conv1d kernel of the Mamba block; the operation is the
 * usual one (reading of the build): per channel d, width W,
 *   out[b,t,d] = bias[d] + sum_{k<W} w[d,k] * x[b, t-(W-1)+k, d]   (x = 0 before t = 0)
 * then optionally silu(out).  Layouts: x (B, L, D) in dtype; w (D, W); bias (D), nullable;
 * out (B, L, D) double.
 */
int oracle_causal_conv1d(const void* x, const float* w, const float* bias, double* out, int64_t batch, int64_t L,
                         int64_t Dm, int64_t W, int dtype, int apply_silu, int nthreads) {
  if (!x || !w || !out || batch < 1 || L < 1 || Dm < 1 || W < 1) return OR_ERR_ARG;
  if (dtype != OR_F32 && dtype != OR_BF16) return OR_ERR_ARG;
  set_threads(nthreads);
  int64_t nch = batch * Dm;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t c = 0; c < nch; ++c) {
    int64_t b = c / Dm, d = c % Dm;
    for (int64_t t = 0; t < L; ++t) {
      double v = bias ? (double)bias[d] : 0.0;
      for (int64_t k = 0; k < W; ++k) {
        int64_t ts = t - (W - 1) + k;
        if (ts >= 0) v += (double)w[d * W + k] * load_val(x, (b * L + ts) * Dm + d, dtype);
      }
      if (apply_silu) v = v / (1.0 + exp(-v));
      out[(b * L + t) * Dm + d] = v;
    }
  }
  return OR_OK;
}

/*
 * Elementwise form, one channel -- [P3] "Reference solution":
 *   h = h0[b,d] (or 0); for t: h = A_t*h + B_t*x_t; y_t = C_t*h.
 * All of x, A, B, C are (B, L, D) fp32; h0, h_last (B, D).
 */
static void ew_channel(const float* x, const float* A, const float* Bm, const float* Cm, const float* h0,
                       int64_t b, int64_t d, int64_t L, int64_t Dm, double* y_out, int64_t y_stride,
                       double* hl_out) {
  double h = h0 ? (double)h0[b * Dm + d] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    int64_t e = (b * L + t) * Dm + d;
    h = (double)A[e] * h + (double)Bm[e] * (double)x[e];
    y_out[t * y_stride] = (double)Cm[e] * h;
  }
  if (hl_out) *hl_out = h;
}

int oracle_elementwise_scan(const float* x, const float* A, const float* Bm, const float* Cm, const float* h0,
                            double* y, double* h_last, int64_t batch, int64_t L, int64_t Dm, int nthreads) {
  if (!x || !A || !Bm || !Cm || !y || batch < 1 || L < 1 || Dm < 1) return OR_ERR_ARG;
  set_threads(nthreads);
  int64_t nch = batch * Dm;
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < nch; ++c) {
    int64_t b = c / Dm, d = c % Dm;
    ew_channel(x, A, Bm, Cm, h0, b, d, L, Dm, y + b * L * Dm + d, Dm, h_last ? h_last + c : 0);
  }
  return OR_OK;
}

int oracle_elementwise_scan_channels(const float* x, const float* A, const float* Bm, const float* Cm,
                                     const float* h0, const int64_t* chan, int64_t nchan, double* y_out,
                                     double* hl_out, int64_t batch, int64_t L, int64_t Dm, int nthreads) {
  if (!x || !A || !Bm || !Cm || !chan || !y_out || nchan < 0 || batch < 1 || L < 1 || Dm < 1) return OR_ERR_ARG;
  for (int64_t k = 0; k < nchan; ++k)
    if (chan[k] < 0 || chan[k] >= batch * Dm) return OR_ERR_ARG;
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t k = 0; k < nchan; ++k) {
    int64_t b = chan[k] / Dm, d = chan[k] % Dm;
    ew_channel(x, A, Bm, Cm, h0, b, d, L, Dm, y_out + k * L, 1, hl_out ? hl_out + k : 0);
  }
  return OR_OK;
}

/*
 * Second, independent evaluation by pairs -- [P1] "Scan bien recurrence ...":
 * each step is the affine map T_t(h) = a_t*h + b_t, written as the pair (a_t, b_t);
 * two steps compose as (a2, b2) (x) (a1, b1) = (a2*a1, a2*b1 + b2) with identity (1, 0).
 * The sequence is cut into chunks of `chunk` steps (the last one may be short):
 *   1. fold each chunk's pairs from the identity into one chunk pair;
 *   2. fold the chunk pairs in order, starting from the pair (0, h0), to get
 *      the state entering every chunk;
 *   3. replay each chunk from its entering state, producing every h_t.
 * It reaches the same states as the stepwise loop up to rounding order.
 */
typedef struct {
  double a, b;
} pair_t;

static pair_t compose(pair_t cur, pair_t prefix) { /* cur (x) prefix : apply prefix, then cur */
  pair_t r;
  r.a = cur.a * prefix.a;
  r.b = cur.a * prefix.b + cur.b;
  return r;
}

/* step pair of the selective form for (b, t, d, n). */
static pair_t sel_step(const void* x, const void* delta, const float* A, const float* Bm, int64_t b, int64_t t,
                       int64_t d, int64_t n, int64_t L, int64_t Dm, int64_t N, int dtype, int exact_zoh) {
  int64_t e = (b * L + t) * Dm + d;
  double xt = load_val(x, e, dtype), dt = load_val(delta, e, dtype);
  double a = (double)A[d * N + n];
  double Bn = (double)Bm[(b * L + t) * N + n];
  pair_t p;
  p.a = exp(dt * a);
  p.b = (exact_zoh ? (a != 0.0 ? expm1(dt * a) / a : dt) : dt) * Bn * xt;
  return p;
}

int oracle_selective_scan_chunked(const void* x, const void* delta, const float* A, const float* Bm,
                                  const float* Cm, const float* Dsk, const void* z, const float* h0, double* y,
                                  double* h_last, int64_t batch, int64_t L, int64_t Dm, int64_t N, int dtype,
                                  int exact_zoh, int64_t chunk, int nthreads) {
  if (!sel_args_ok(x, delta, A, Bm, Cm, batch, L, Dm, N, dtype) || !y || chunk < 1) return OR_ERR_ARG;
  set_threads(nthreads);
  int64_t nchunks = (L + chunk - 1) / chunk;
  int64_t nch = batch * Dm;
  for (int64_t i = 0; i < batch * L * Dm; ++i) y[i] = 0.0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t c = 0; c < nch; ++c) {
    int64_t b = c / Dm, d = c % Dm;
    for (int64_t n = 0; n < N; ++n) {
      /* entering state of the whole sequence as the pair (0, h0) */
      pair_t run;
      run.a = 0.0;
      run.b = h0 ? (double)h0[(b * Dm + d) * N + n] : 0.0;
      for (int64_t k = 0; k < nchunks; ++k) {
        int64_t t0 = k * chunk, t1 = t0 + chunk < L ? t0 + chunk : L;
        /* 1. chunk pair */
        pair_t agg = {1.0, 0.0};
        for (int64_t t = t0; t < t1; ++t)
          agg = compose(sel_step(x, delta, A, Bm, b, t, d, n, L, Dm, N, dtype, exact_zoh), agg);
        /* 3. replay from the entering state run.b, accumulating C_t[n]*h_t[n] into y */
        pair_t pre = run;
        for (int64_t t = t0; t < t1; ++t) {
          pre = compose(sel_step(x, delta, A, Bm, b, t, d, n, L, Dm, N, dtype, exact_zoh), pre);
          y[(b * L + t) * Dm + d] += (double)Cm[(b * L + t) * N + n] * pre.b;
        }
        /* 2. state entering the next chunk */
        run = compose(agg, run);
      }
      if (h_last) h_last[(b * Dm + d) * N + n] = run.b;
    }
    for (int64_t t = 0; t < L; ++t) {
      int64_t e = (b * L + t) * Dm + d;
      double v = y[e];
      if (Dsk) v += (double)Dsk[d] * load_val(x, e, dtype);
      if (z) {
        double zt = load_val(z, e, dtype);
        v *= zt / (1.0 + exp(-zt));
      }
      y[e] = v;
    }
  }
  return OR_OK;
}

int oracle_elementwise_scan_chunked(const float* x, const float* A, const float* Bm, const float* Cm,
                                    const float* h0, double* y, double* h_last, int64_t batch, int64_t L,
                                    int64_t Dm, int64_t chunk, int nthreads) {
  if (!x || !A || !Bm || !Cm || !y || batch < 1 || L < 1 || Dm < 1 || chunk < 1) return OR_ERR_ARG;
  set_threads(nthreads);
  int64_t nchunks = (L + chunk - 1) / chunk;
  int64_t nch = batch * Dm;
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < nch; ++c) {
    int64_t b = c / Dm, d = c % Dm;
    pair_t run;
    run.a = 0.0;
    run.b = h0 ? (double)h0[b * Dm + d] : 0.0;
    for (int64_t k = 0; k < nchunks; ++k) {
      int64_t t0 = k * chunk, t1 = t0 + chunk < L ? t0 + chunk : L;
      pair_t agg = {1.0, 0.0};
      for (int64_t t = t0; t < t1; ++t) {
        int64_t e = (b * L + t) * Dm + d;
        pair_t s = {(double)A[e], (double)Bm[e] * (double)x[e]};
        agg = compose(s, agg);
      }
      pair_t pre = run;
      for (int64_t t = t0; t < t1; ++t) {
        int64_t e = (b * L + t) * Dm + d;
        pair_t s = {(double)A[e], (double)Bm[e] * (double)x[e]};
        pre = compose(s, pre);
        y[e] = (double)Cm[e] * pre.b;
      }
      run = compose(agg, run);
    }
    if (h_last) h_last[c] = run.b;
  }
  return OR_OK;
}
