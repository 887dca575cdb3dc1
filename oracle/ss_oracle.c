/*
 * ss_oracle.c -- fp64 CPU reference ("oracle") for the selective state-space scan (S6).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct definition that the GPU
 * library is checked against.  Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark load it.  The GPU library neither links nor calls it, and it shares no code,
 * header, table or helper with the GPU library.
 *
 * Sources (web pages; section names as printed on each page):
 *   [P1] "Mamba: Linear-Time Sequence Modeling with Selective State Spaces" reading guide
 *        (xyznot.com), sections "Método", "O Mecanismo de Seleção (S6)",
 *        "Expansão de Estado Ciente de Hardware", "Perguntas".
 *   [P2] "O que é um modelo Mamba?" (ibm.com), the state and output equations, the
 *        discretisation paragraphs and the Mamba-block walk-through.
 *   [P5] "Как работает Mamba (State Space Model) и чем она лучше трансформера?" (aivaro.ru),
 *        section 3 "Selective Scan" and its simplified selective_scan sketch.
 *
 * What is computed, for every independent row (b, d) of the (batch, d_inner) grid:
 *   s_t     = delta[b,t,d] + delta_bias[d]                     [P1 S6: tau(Parameter + s(x))]
 *   dt_t    = softplus(s_t)  (or s_t when softplus is off)     [P1 S6; P5 section 3]
 *   Abar    = exp(dt_t * A[d,n])                               [P1 Method: ZOH Abar = exp(dA)]
 *   Bbar    = dt_t * B[b,t,n]                                  [P5 sketch: B_bar = delta * B]
 *             or, with zoh_exact, (exp(dt A) - 1)/A * B        [P1 Method: exact ZOH Bbar]
 *   h_t[n]  = Abar * h_{t-1}[n] + Bbar * u[b,t,d]              [P1 Method recurrence]
 *   y_t     = sum_n C[b,t,n] h_t[n] + D[d] u[b,t,d]            [P1 Method y_t = C h_t; P2 output
 *                                                               equation with D; P5 D*u skip]
 *   out     = y_t * silu(z[b,t,d]) when z is given             [P2 Mamba block: SSM output
 *                                                               multiplied by the activated gate]
 * with h_{-1} = h0 (zeros when absent, as in the P5 sketch).  The state is diagonal: each
 * channel d carries its own N-vector, and A is stored (d_inner, d_state) [P2: diagonal A].
 * B and C have shape (batch, seqlen, d_state) and are shared by all channels [P1 S6; P5].
 *
 * Everything is evaluated in IEEE double with libm exp/log1p/expm1, sequentially in t.  Inputs
 * are read exactly: fp32 as is, bf16 by placing its 16 bits in the top half of a float.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC ss_oracle.c -lm   (no -ffast-math).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_F64 = 2 };

/* Read element i of an io-dtype array exactly (bf16 -> fp32 is a 16-bit shift; f64 is only used
 * for an input u that the convolution front end below produced in double). */
static double rd(const void* p, int64_t i, int dtype) {
  if (dtype == OR_F64) return ((const double*)p)[i];
  if (dtype == OR_BF16) {
    uint32_t bits = ((uint32_t)((const uint16_t*)p)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  return (double)((const float*)p)[i];
}

/* softplus(s) = log(1 + e^s), written without overflow or cancellation [P1 S6, tau = softplus]. */
static double softplus(double s) { return (s > 0.0 ? s : 0.0) + log1p(exp(-fabs(s))); }

/* silu(z) = z * sigmoid(z) [P2 Mamba block: the gate's activation; SiLU is the one the block uses]. */
static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Step size dt for one (b, t, d) element [P1 S6]. */
static double step_size(double raw, const float* delta_bias, int64_t d, int delta_softplus) {
  double s = raw + (delta_bias ? (double)delta_bias[d] : 0.0);
  return delta_softplus ? softplus(s) : s;
}

/* Input coefficient Bbar / B for one state: dt (first-order form, [P5 sketch]) or the exact ZOH
 * factor (exp(dt a) - 1) / a, which tends to dt as a -> 0 [P1 Method]. */
static double bbar_factor(double dt, double a, int zoh_exact) {
  if (!zoh_exact) return dt;
  if (a == 0.0) return dt;
  return expm1(dt * a) / a;
}

/*
 * Whole-sequence prefill, sequential in t (RNN mode [P1 Method; P2 discretised recurrence]).
 *
 * Layouts (row-major, contiguous):
 *   u, delta, z : (batch, seqlen, d_inner)   io dtype
 *   B, C        : (batch, seqlen, d_state)   io dtype
 *   A           : (d_inner, d_state) f32;  D, delta_bias : (d_inner) f32, NULL = 0
 *   h0          : (batch, d_inner, d_state) f64, NULL = zeros
 *   rows        : row ids r = b*d_inner + d to evaluate; NULL = all rows in order
 *   out         : (nrows, seqlen) f64, out[i*seqlen + t] for rows[i]
 *   h_last      : (nrows, d_state) f64 or NULL
 * u is read as u_dtype (the io dtype, or f64 when it comes from oracle_conv_silu).
 * Returns 0, or -1 on a bad argument.
 */
int oracle_scan_fwd(const void* u, const void* delta, const float* A, const void* B,
                    const void* C, const float* D, const void* z, const float* delta_bias,
                    int delta_softplus, const double* h0, int zoh_exact, int io_dtype,
                    int u_dtype, int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                    const int64_t* rows, int64_t nrows, double* out, double* h_last,
                    int nthreads) {
  if (!u || !delta || !A || !B || !C || !out) return -1;
  if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state < 1 || d_state > 256) return -1;
  if (io_dtype != OR_F32 && io_dtype != OR_BF16) return -1;
  if (u_dtype != io_dtype && u_dtype != OR_F64) return -1;
  if (!rows) nrows = batch * d_inner;
  if (nthreads < 1) nthreads = 1;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : bad)
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t r = rows ? rows[i] : i;
    if (r < 0 || r >= batch * d_inner) { bad = 1; continue; }
    int64_t b = r / d_inner, d = r % d_inner;
    double h[256];
    for (int64_t n = 0; n < d_state; ++n) h[n] = h0 ? h0[r * d_state + n] : 0.0;
    for (int64_t t = 0; t < seqlen; ++t) {
      int64_t e = (b * seqlen + t) * d_inner + d;      /* (b, t, d) element */
      int64_t bc = (b * seqlen + t) * d_state;         /* (b, t, 0) of B and C */
      double x = rd(u, e, u_dtype);
      double dt = step_size(rd(delta, e, io_dtype), delta_bias, d, delta_softplus);
      double y = 0.0;
      for (int64_t n = 0; n < d_state; ++n) {
        double a = (double)A[d * d_state + n];
        double abar = exp(dt * a);
        double bbar = bbar_factor(dt, a, zoh_exact) * rd(B, bc + n, io_dtype);
        h[n] = abar * h[n] + bbar * x;
        y += rd(C, bc + n, io_dtype) * h[n];
      }
      if (D) y += (double)D[d] * x;
      if (z) y *= silu(rd(z, e, io_dtype));
      out[i * seqlen + t] = y;
    }
    if (h_last)
      for (int64_t n = 0; n < d_state; ++n) h_last[i * d_state + n] = h[n];
  }
  return bad ? -1 : 0;
}

/*
 * The same prefill through the associative decomposition over time blocks of `chunk` steps
 * [P1 "Parallel Associative Scan"; P2: the recurrence split into small independent blocks that
 * are combined hierarchically].  Inside a block each state is run from zero while the running
 * product of Abar is kept; the true state is then
 *     h_t = hloc_t + (prod_{s<=t in block} Abar_s) * h_in,
 * and h_in for the next block is the true state at the block's end.  Arguments and layouts are
 * those of oracle_scan_fwd.  Used to pin that decomposition against the sequential form.
 */
int oracle_scan_fwd_chunked(const void* u, const void* delta, const float* A, const void* B,
                            const void* C, const float* D, const void* z,
                            const float* delta_bias, int delta_softplus, const double* h0,
                            int zoh_exact, int io_dtype, int u_dtype, int64_t batch,
                            int64_t seqlen,
                            int64_t d_inner, int64_t d_state, int64_t chunk, double* out,
                            double* h_last) {
  if (!u || !delta || !A || !B || !C || !out) return -1;
  if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state < 1 || d_state > 256 || chunk < 1)
    return -1;
  if (u_dtype != io_dtype && u_dtype != OR_F64) return -1;
  for (int64_t r = 0; r < batch * d_inner; ++r) {
    int64_t b = r / d_inner, d = r % d_inner;
    double h_in[256], hloc[256], prod[256];
    for (int64_t n = 0; n < d_state; ++n) h_in[n] = h0 ? h0[r * d_state + n] : 0.0;
    for (int64_t t0 = 0; t0 < seqlen; t0 += chunk) {
      int64_t t1 = t0 + chunk < seqlen ? t0 + chunk : seqlen;
      for (int64_t n = 0; n < d_state; ++n) { hloc[n] = 0.0; prod[n] = 1.0; }
      for (int64_t t = t0; t < t1; ++t) {
        int64_t e = (b * seqlen + t) * d_inner + d;
        int64_t bc = (b * seqlen + t) * d_state;
        double x = rd(u, e, u_dtype);
        double dt = step_size(rd(delta, e, io_dtype), delta_bias, d, delta_softplus);
        double y = 0.0;
        for (int64_t n = 0; n < d_state; ++n) {
          double a = (double)A[d * d_state + n];
          double abar = exp(dt * a);
          hloc[n] = abar * hloc[n] + bbar_factor(dt, a, zoh_exact) * rd(B, bc + n, io_dtype) * x;
          prod[n] *= abar;
          y += rd(C, bc + n, io_dtype) * (hloc[n] + prod[n] * h_in[n]);
        }
        if (D) y += (double)D[d] * x;
        if (z) y *= silu(rd(z, e, io_dtype));
        out[r * seqlen + t] = y;
      }
      for (int64_t n = 0; n < d_state; ++n) h_in[n] = hloc[n] + prod[n] * h_in[n];
    }
    if (h_last)
      for (int64_t n = 0; n < d_state; ++n) h_last[r * d_state + n] = h_in[n];
  }
  return 0;
}

/*
 * One decode step (single token) on a resident state [P1 Perguntas: a fixed-size D x N state
 * per layer, advanced once per generated token; P2: constant memory at inference].
 * Exactly one t-iteration of oracle_scan_fwd with h read from and written back to `state`.
 *
 *   state            : (batch, d_inner, d_state) f64, updated in place for the selected rows
 *   u, delta, z      : (batch, d_inner) io dtype;  B, C : (batch, d_state) io dtype
 *   rows / nrows     : as in oracle_scan_fwd;  out : (nrows) f64
 */
int oracle_state_update(double* state, const void* u, const void* delta, const float* A,
                        const void* B, const void* C, const float* D, const void* z,
                        const float* delta_bias, int delta_softplus, int zoh_exact,
                        int io_dtype, int u_dtype, int64_t batch, int64_t d_inner,
                        int64_t d_state, const int64_t* rows, int64_t nrows, double* out,
                        int nthreads) {
  if (!state || !u || !delta || !A || !B || !C || !out) return -1;
  if (batch < 0 || d_inner < 0 || d_state < 1 || d_state > 256) return -1;
  if (io_dtype != OR_F32 && io_dtype != OR_BF16) return -1;
  if (u_dtype != io_dtype && u_dtype != OR_F64) return -1;
  if (!rows) nrows = batch * d_inner;
  if (nthreads < 1) nthreads = 1;
  int bad = 0;
#pragma omp parallel for schedule(static) num_threads(nthreads) reduction(| : bad)
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t r = rows ? rows[i] : i;
    if (r < 0 || r >= batch * d_inner) { bad = 1; continue; }
    int64_t b = r / d_inner, d = r % d_inner;
    double x = rd(u, r, u_dtype);
    double dt = step_size(rd(delta, r, io_dtype), delta_bias, d, delta_softplus);
    double y = 0.0;
    for (int64_t n = 0; n < d_state; ++n) {
      double a = (double)A[d * d_state + n];
      double* h = &state[r * d_state + n];
      *h = exp(dt * a) * (*h) + bbar_factor(dt, a, zoh_exact) * rd(B, b * d_state + n, io_dtype) * x;
      y += rd(C, b * d_state + n, io_dtype) * (*h);
    }
    if (D) y += (double)D[d] * x;
    if (z) y *= silu(rd(z, r, io_dtype));
    out[i] = y;
  }
  return bad ? -1 : 0;
}

/*
 * Front end of the block's SSM path [P2 Mamba block: x_proj goes through a one-dimensional
 * convolution whose output passes SiLU, giving x_act, the SSM's input].  The convolution is
 * depthwise (one kernel per channel) over time and causal (output t sees inputs up to t only, as
 * a sequence model run token by token must; [P5] installs the causal-conv1d package), width k:
 *   u[b,t,d] = silu( conv_b[d] + sum_{j=0}^{k-1} conv_w[d*k + j] * x[b, t-(k-1)+j, d] )
 * Inputs before t = 0 are x_prev[b, k-1+t', d] for t' = t-(k-1)+j < 0 (the k-1 steps that came
 * before), or 0 when x_prev is NULL.  conv_b NULL means 0.
 *   x      : (batch, seqlen, d_inner) io dtype;  x_prev : (batch, k-1, d_inner) io dtype
 *   conv_w : (d_inner, k) f32;  conv_b : (d_inner) f32
 *   u      : (batch, seqlen, d_inner) f64 output, unrounded
 */
int oracle_conv_silu(const void* x, const float* conv_w, const float* conv_b,
                     const void* x_prev, int64_t k, int io_dtype, int64_t batch,
                     int64_t seqlen, int64_t d_inner, double* u) {
  if (!x || !conv_w || !u || k < 1 || batch < 0 || seqlen < 0 || d_inner < 0) return -1;
  if (io_dtype != OR_F32 && io_dtype != OR_BF16) return -1;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t t = 0; t < seqlen; ++t)
      for (int64_t d = 0; d < d_inner; ++d) {
        double acc = conv_b ? (double)conv_b[d] : 0.0;
        for (int64_t j = 0; j < k; ++j) {
          int64_t ts = t - (k - 1) + j; /* time of the input this tap multiplies */
          double xv;
          if (ts >= 0)
            xv = rd(x, (b * seqlen + ts) * d_inner + d, io_dtype);
          else
            xv = x_prev ? rd(x_prev, (b * (k - 1) + (k - 1) + ts) * d_inner + d, io_dtype) : 0.0;
          acc += (double)conv_w[d * k + j] * xv;
        }
        u[(b * seqlen + t) * d_inner + d] = silu(acc);
      }
  return 0;
}

/*
 * Gradients of the prefill by reverse-mode differentiation of the recurrence, in double.  For
 * one row (b, d), with x_t = u, s_t = delta + bias, dt_t = softplus(s_t), e_{t,n} =
 * exp(dt_t a_n), the input gain g_{t,n} = bbar_factor(dt_t, a_n) (dt_t in the first-order form,
 * expm1(dt_t a_n) / a_n under exact ZOH), h_t = e_t h_{t-1} + g_t B_t x_t,
 * y_t = C_t . h_t + D x_t and out_t = y_t silu(z_t), given G_t = dL/d out_t and dL/dh_{L-1}:
 *   gy_t       = G_t silu(z_t);       dz_t = G_t y_t silu'(z_t)
 *   lam_t[n]   = gy_t C_t[n] + e_{t+1,n} lam_{t+1}[n]      (lam_{L-1} also gets dL/dh_{L-1})
 *   ddt_t      = sum_n lam_t[n] (a_n e_{t,n} h_{t-1}[n] + dg/ddt B_t[n] x_t)
 *                  dg/ddt = 1 (first order), e_{t,n} (exact ZOH)
 *   du_t       = gy_t D + sum_n lam_t[n] g_{t,n} B_t[n]
 *   dB_t[n]   += lam_t[n] g_{t,n} x_t          dC_t[n] += gy_t h_t[n]       (summed over d)
 *   dA[d,n]   += sum_t lam_t[n] (dt_t e_{t,n} h_{t-1}[n] + dg/da B_t[n] x_t)
 *                  dg/da = 0 (first order), (dt e - g) / a, or dt^2 / 2 at a = 0 (exact ZOH)
 *   dD[d]     += sum_t gy_t x_t
 *   ddelta_t   = ddt_t softplus'(s_t) = ddt_t sigmoid(s_t)   (ddt_t with softplus off)
 *   dbias[d]  += sum_t ddelta_t;          dh0 = e_0 lam_0
 * The recurrence and the output equation are those of oracle_scan_fwd [P1 Method; P2 output
 * equation and Mamba block]; the derivative rules are the chain rule.
 *   dout : (batch, seqlen, d_inner) f64;  dh_last : (batch, d_inner, d_state) f64 or NULL
 *   du, ddelta, dz : (batch, seqlen, d_inner) f64 (dz ignored without z)
 *   dB, dC : (batch, seqlen, d_state) f64;  dA : (d_inner, d_state);  dD, dbias : (d_inner)
 *   dh0 : (batch, d_inner, d_state) f64 or NULL.  Every output is overwritten.
 * Rows run in parallel (OpenMP, a fixed block of rows per thread); each thread adds the rows'
 * contributions to the summed gradients (dA, dB, dC, dD, dbias) into partial sums of its own,
 * and the partials are added afterwards in thread order, so a given thread count always gives
 * the same bits.
 */

/* d g / d a for the exact-ZOH gain g = expm1(dt a) / a, with e = exp(dt a). */
static double zoh_gain_da(double dt, double a, double e) {
  if (a == 0.0) return 0.5 * dt * dt;
  return (dt * e - expm1(dt * a) / a) / a;
}

/* The reverse pass of one row r = b * d_inner + d; hist ((seqlen + 1) * d_state) and dts
 * (seqlen) are scratch.  Per-element gradients are written, summed ones added to the sA.. sums. */
static void bwd_row(const void* u, const void* delta, const float* A, const void* B,
                    const void* C, const float* D, const void* z, const float* delta_bias,
                    int delta_softplus, const double* h0, int zoh_exact, int io_dtype,
                    int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state, int64_t r,
                    const double* dout, const double* dh_last, double* du, double* ddelta,
                    double* dz, double* dh0, double* hist, double* dts, double* dA, double* dB,
                    double* dC, double* dD, double* dbias) {
  int64_t b = r / d_inner, d = r % d_inner;
  (void)batch;
  /* forward, keeping every state */
  for (int64_t n = 0; n < d_state; ++n) hist[n] = h0 ? h0[r * d_state + n] : 0.0;
  for (int64_t t = 0; t < seqlen; ++t) {
    int64_t e = (b * seqlen + t) * d_inner + d, bc = (b * seqlen + t) * d_state;
    double x = rd(u, e, io_dtype);
    double dt = step_size(rd(delta, e, io_dtype), delta_bias, d, delta_softplus);
    dts[t] = dt;
    for (int64_t n = 0; n < d_state; ++n) {
      double a = (double)A[d * d_state + n];
      hist[(t + 1) * d_state + n] = exp(dt * a) * hist[t * d_state + n] +
                                    bbar_factor(dt, a, zoh_exact) * rd(B, bc + n, io_dtype) * x;
    }
  }
  /* reverse */
  double lam[256], e_next[256];
  for (int64_t n = 0; n < d_state; ++n) {
    lam[n] = dh_last ? dh_last[r * d_state + n] : 0.0;
    e_next[n] = 1.0;
  }
  for (int64_t t = seqlen - 1; t >= 0; --t) {
    int64_t e = (b * seqlen + t) * d_inner + d, bc = (b * seqlen + t) * d_state;
    double x = rd(u, e, io_dtype), dt = dts[t];
    const double* h = &hist[(t + 1) * d_state];
    const double* hp = &hist[t * d_state];
    double y = 0.0;
    for (int64_t n = 0; n < d_state; ++n) y += rd(C, bc + n, io_dtype) * h[n];
    if (D) y += (double)D[d] * x;
    double gy = dout[e];
    if (z) {
      double zv = rd(z, e, io_dtype), sg = 1.0 / (1.0 + exp(-zv));
      gy = dout[e] * zv * sg;
      if (dz) dz[e] = dout[e] * y * sg * (1.0 + zv * (1.0 - sg));
    }
    double ddt = 0.0, dx = D ? gy * (double)D[d] : 0.0;
    for (int64_t n = 0; n < d_state; ++n) {
      double a = (double)A[d * d_state + n];
      double bn = rd(B, bc + n, io_dtype), cn = rd(C, bc + n, io_dtype);
      double et = exp(dt * a);
      double g = bbar_factor(dt, a, zoh_exact);
      double g_dt = zoh_exact ? et : 1.0;
      /* the state's adjoint: from y_t, and from h_{t+1} through e_{t+1} (or dh_last) */
      lam[n] = gy * cn + (t == seqlen - 1 ? lam[n] : e_next[n] * lam[n]);
      ddt += lam[n] * (a * et * hp[n] + g_dt * bn * x);
      dx += lam[n] * g * bn;
      dB[bc + n] += lam[n] * g * x;
      dC[bc + n] += gy * h[n];
      dA[d * d_state + n] += lam[n] * dt * et * hp[n];
      if (zoh_exact) dA[d * d_state + n] += lam[n] * zoh_gain_da(dt, a, et) * bn * x;
      e_next[n] = et;
    }
    dD[d] += gy * x; /* the gradient at D (0 when D is absent) */
    double s = rd(delta, e, io_dtype) + (delta_bias ? (double)delta_bias[d] : 0.0);
    double dd = delta_softplus ? ddt / (1.0 + exp(-s)) : ddt;
    ddelta[e] = dd;
    dbias[d] += dd;
    du[e] = dx;
  }
  if (dh0)
    for (int64_t n = 0; n < d_state; ++n)
      dh0[r * d_state + n] = (seqlen > 0 ? e_next[n] * lam[n] : lam[n]);
}

int oracle_scan_bwd(const void* u, const void* delta, const float* A, const void* B,
                    const void* C, const float* D, const void* z, const float* delta_bias,
                    int delta_softplus, const double* h0, int zoh_exact, int io_dtype,
                    int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                    const double* dout, const double* dh_last, double* du, double* ddelta,
                    double* dz, double* dA, double* dB, double* dC, double* dD, double* dbias,
                    double* dh0, int nthreads) {
  if (!u || !delta || !A || !B || !C || !dout || !du || !ddelta || !dA || !dB || !dC || !dD ||
      !dbias)
    return -1;
  if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state < 1 || d_state > 256) return -1;
  if (io_dtype != OR_F32 && io_dtype != OR_BF16) return -1;
  if (nthreads < 1) nthreads = 1;
  const int64_t nA = d_inner * d_state, nBC = batch * seqlen * d_state;
  const int64_t nsum = nA + 2 * nBC + 2 * d_inner; /* dA | dB | dC | dD | dbias */
  double* part = (double*)calloc((size_t)nthreads * (size_t)(nsum > 0 ? nsum : 1), sizeof(double));
  if (!part) return -1;
  int bad = 0;
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
  {
    int tid = 0;
#ifdef _OPENMP
    tid = omp_get_thread_num();
#endif
    double* p = part + (int64_t)tid * nsum;
    double* hist = (double*)malloc(sizeof(double) * (seqlen + 1) * d_state); /* h_{-1..L-1} */
    double* dts = (double*)malloc(sizeof(double) * (seqlen > 0 ? seqlen : 1));
    if (!hist || !dts) bad = 1;
#pragma omp for schedule(static)
    for (int64_t r = 0; r < batch * d_inner; ++r) {
      if (!hist || !dts) continue;
      bwd_row(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, zoh_exact, io_dtype,
              batch, seqlen, d_inner, d_state, r, dout, dh_last, du, ddelta, dz, dh0, hist, dts,
              p, p + nA, p + nA + nBC, p + nA + 2 * nBC, p + nA + 2 * nBC + d_inner);
    }
    free(hist);
    free(dts);
  }
  /* the summed gradients: partials added in thread order */
  double* outs[5] = {dA, dB, dC, dD, dbias};
  int64_t offs[5] = {0, nA, nA + nBC, nA + 2 * nBC, nA + 2 * nBC + d_inner};
  int64_t lens[5] = {nA, nBC, nBC, d_inner, d_inner};
  for (int k = 0; k < 5; ++k)
    for (int64_t i = 0; i < lens[k]; ++i) {
      double acc = 0.0;
      for (int th = 0; th < nthreads; ++th) acc += part[(int64_t)th * nsum + offs[k] + i];
      outs[k][i] = acc;
    }
  free(part);
  return bad ? -1 : 0;
}

/*
 * Multi-head selective scan with a scalar transition per head (the Mamba-2 form [P2: Mamba-2
 * splits the block into heads like multi-head attention, with B and C shared by groups of heads
 * as in grouped-query attention; P3: the diagonal transition reduced to a scalar times the
 * identity]).  For batch b, head h (group g = h / (nheads / ngroups)), state n, head channel p:
 *   dt_t     = softplus(dt[b,t,h] + dt_bias[h])  (or the raw sum)           [P1 S6]
 *   hs_t[n,p] = exp(dt_t A[h]) hs_{t-1}[n,p] + dt_t B[b,t,g,n] x[b,t,h,p]   [P1 Method]
 *   y_t[p]   = sum_n C[b,t,g,n] hs_t[n,p] + D[h] x[b,t,h,p]                 [P1, P2]
 *   out      = y_t[p] silu(z[b,t,h,p]) when z is given                      [P2 Mamba block]
 *   x, z : (batch, seqlen, nheads, headdim) io dtype;  dt : (batch, seqlen, nheads) io dtype
 *   A, dt_bias, D : (nheads) f32 (dt_bias, D NULL = 0);  B, C : (batch, seqlen, ngroups, d_state)
 *   h0, h_last : (batch, nheads, d_state, headdim) f64 (NULL = zeros / not written)
 *   out : (batch, seqlen, nheads, headdim) f64
 */
int oracle_scan2_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C,
                     const float* D, const void* z, const float* dt_bias, int dt_softplus,
                     const double* h0, int io_dtype, int64_t batch, int64_t seqlen,
                     int64_t nheads, int64_t headdim, int64_t ngroups, int64_t d_state,
                     double* out, double* h_last, int nthreads) {
  if (!x || !dt || !A || !B || !C || !out) return -1;
  if (batch < 0 || seqlen < 0 || nheads < 1 || headdim < 1 || ngroups < 1 || d_state < 1)
    return -1;
  if (nheads % ngroups != 0) return -1;
  if (io_dtype != OR_F32 && io_dtype != OR_BF16) return -1;
  if (nthreads < 1) nthreads = 1;
  const int64_t hpg = nheads / ngroups;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : bad)
  for (int64_t r = 0; r < batch * nheads; ++r) {
    int64_t b = r / nheads, h = r % nheads, g = h / hpg;
    double* hs = (double*)malloc(sizeof(double) * d_state * headdim);
    if (!hs) { bad = 1; continue; }
    for (int64_t i = 0; i < d_state * headdim; ++i) hs[i] = h0 ? h0[r * d_state * headdim + i] : 0.0;
    for (int64_t t = 0; t < seqlen; ++t) {
      double s = rd(dt, (b * seqlen + t) * nheads + h, io_dtype) + (dt_bias ? (double)dt_bias[h] : 0.0);
      double dtv = dt_softplus ? softplus(s) : s;
      double decay = exp(dtv * (double)A[h]);
      int64_t bc = ((b * seqlen + t) * ngroups + g) * d_state;
      int64_t xo = ((b * seqlen + t) * nheads + h) * headdim;
      for (int64_t n = 0; n < d_state; ++n) {
        double bn = dtv * rd(B, bc + n, io_dtype);
        for (int64_t p = 0; p < headdim; ++p)
          hs[n * headdim + p] = decay * hs[n * headdim + p] + bn * rd(x, xo + p, io_dtype);
      }
      for (int64_t p = 0; p < headdim; ++p) {
        double y = 0.0;
        for (int64_t n = 0; n < d_state; ++n) y += rd(C, bc + n, io_dtype) * hs[n * headdim + p];
        double xp = rd(x, xo + p, io_dtype);
        if (D) y += (double)D[h] * xp;
        if (z) y *= silu(rd(z, xo + p, io_dtype));
        out[xo + p] = y;
      }
    }
    if (h_last)
      for (int64_t i = 0; i < d_state * headdim; ++i) h_last[r * d_state * headdim + i] = hs[i];
    free(hs);
  }
  return bad ? -1 : 0;
}

/* Number of threads OpenMP would use by default (for reporting the CPU baseline). */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
