/*
 * ssm_oracle.c -- plain, slow, sequential fp64 CPU oracle for the selective
 * state-space (S6 / Mamba) scan and its single-token decode update.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or helper with the HIP library; the GPU path never calls it.
 *
 * What it computes (all arithmetic in double precision):
 *
 *   for each batch b and channel d, independently, with h[0..N) = 0:
 *     for t = 0 .. L-1:
 *       v      = delta[b,t,d] + (delta_bias ? delta_bias[d] : 0)
 *       dt     = delta_softplus ? softplus(v) : v
 *       for n:   h[n] = exp(dt * A[d,n]) * h[n] + dt * B[b,t,n] * x[b,t,d]
 *       y      = sum_n C[b,t,n] * h[n]  +  (D ? D[d] * x[b,t,d] : 0)
 *       if z:    y = y * silu(z[b,t,d])
 *       out[b,t,d] = y
 *     last_state[b,d,:] = h
 *
 * Sources (page title, section):
 *  - "Mamba 论文精读" (youngju.dev), sec. 2.2 "离散化 (Zero-Order Hold)":
 *    the discretised recurrence h_t = Abar h_{t-1} + Bbar x_t, y_t = C h_t,
 *    with Abar = exp(delta*A).
 *  - same page, sec. 3.3 "Hardware-Aware 算法", the simplified selective_scan
 *    listing: Bbar*x is taken as delta*B*x (not the exact ZOH form), the state
 *    starts at zero, and the state is updated before y_t is read out, so y_t
 *    already sees x_t.  Shapes: x, delta (B,L,D); A (D,N); B, C (B,L,N).
 *  - same page, sec. 3.1: delta = softplus(Linear_delta(x)); sec. 3.4: the
 *    delta projection carries a bias (added before softplus), D is a per-channel
 *    skip parameter and the output is gated by SiLU(z).
 *  - "Mamba的基础知识" (weblog-19d), section on state space models: D is the
 *    direct input-to-output (skip) term of the observation equation.
 *
 * Inputs are read in their storage type (fp32, or bf16 bit patterns) and
 * widened exactly to double; A, D and delta_bias are fp32.
 *
 * The file also holds the depthwise causal convolution that precedes the scan
 * in the Mamba block, and its one-token form (oracle_causal_conv1d,
 * oracle_conv1d_update, below), the backward scan (oracle_scan_bwd), and the
 * Mamba-2 state space dual layer with one scalar A per head and B, C shared by
 * a group of heads (oracle_ssd, "Mamba 论文精读" sec. 4 and 5.2).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

/* Exact widening of one stored element to double.  A bf16 value is the top
 * 16 bits of the fp32 with the same bit pattern, so shifting it up by 16 bits
 * gives that fp32 exactly. */
static double load_elem(const void *p, int dtype, int64_t i) {
  if (dtype == ORACLE_F64) return ((const double *)p)[i];
  if (dtype == ORACLE_F32) return (double)((const float *)p)[i];
  uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* softplus(v) = log(1 + e^v), written in the two overflow-free forms of the
 * same function; no threshold approximation. */
static double softplus(double v) {
  if (v > 0.0) return v + log1p(exp(-v));
  return log1p(exp(v));
}

/* SiLU(z) = z * sigmoid(z) = z / (1 + e^-z). */
static double silu(double z) { return z / (1.0 + exp(-z)); }

/* The definition for one channel (b, d): runs the recurrence over all L steps
 * from the state h (length N, updated in place) and writes y_t to
 * y[t * y_stride_t]. */
/* Bbar for one (d, n), times x: the Delta*B form of the simplified selective_scan
 * ("Mamba 论文精读" sec. 3.3), or the exact zero-order hold of sec. 2.2,
 * Bbar = (Delta A)^-1 (exp(Delta A) - 1) Delta B, which for a diagonal A is
 * expm1(Delta A_n) / A_n * B_n (and Delta B_n in the limit A_n = 0). */
static double bbar_x(int zoh, double dt, double a, double bv, double xt) {
  if (!zoh || a == 0.0) return dt * bv * xt;
  return expm1(dt * a) / a * bv * xt;
}

static void scan_channel(int64_t L, int64_t Dm, int64_t N, int dtype, const void *x, const void *delta,
                         const float *A, const void *B, const void *C, const float *Dskip, const void *z,
                         const float *delta_bias, int delta_softplus, int zoh, int64_t b, int64_t d, double *h,
                         double *y, int64_t y_stride_t) {
  for (int64_t t = 0; t < L; ++t) {
    const int64_t i_td = (b * L + t) * Dm + d;  /* (b,t,d) */
    const int64_t i_tn = (b * L + t) * N;       /* (b,t,0) of B and C */
    double v = load_elem(delta, dtype, i_td) + (delta_bias ? (double)delta_bias[d] : 0.0);
    double dt = delta_softplus ? softplus(v) : v;
    double xt = load_elem(x, dtype, i_td);
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      double abar = exp(dt * (double)A[d * N + n]);
      if (zoh)
        h[n] = abar * h[n] + bbar_x(1, dt, (double)A[d * N + n], load_elem(B, dtype, i_tn + n), xt);
      else
        h[n] = abar * h[n] + dt * load_elem(B, dtype, i_tn + n) * xt;
      acc += load_elem(C, dtype, i_tn + n) * h[n];
    }
    double yt = acc + (Dskip ? (double)Dskip[d] * xt : 0.0);
    if (z) yt *= silu(load_elem(z, dtype, i_td));
    y[t * y_stride_t] = yt;
  }
}

/* Whole scan.  y: (batch, seqlen, dim) doubles.  last_state: (batch, dim,
 * dstate) doubles or NULL.  h0: optional initial state (batch, dim, dstate);
 * NULL means zeros.  Returns 0, or -1 on a bad argument. */
int oracle_scan_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype, const void *x,
                   const void *delta, const float *A, const void *B, const void *C, const float *Dskip,
                   const void *z, const float *delta_bias, int delta_softplus, int zoh, const double *h0, double *y,
                   double *last_state, int nthreads);

int oracle_scan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype, const void *x,
                const void *delta, const float *A, const void *B, const void *C, const float *Dskip,
                const void *z, const float *delta_bias, int delta_softplus, const double *h0, double *y,
                double *last_state, int nthreads) {
  return oracle_scan_ex(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, delta_bias, delta_softplus,
                        0, h0, y, last_state, nthreads);
}

/* oracle_scan with the choice of Bbar: zoh = 0 for Delta*B, 1 for the exact zero-order hold. */
int oracle_scan_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype, const void *x,
                   const void *delta, const float *A, const void *B, const void *C, const float *Dskip,
                   const void *z, const float *delta_bias, int delta_softplus, int zoh, const double *h0, double *y,
                   double *last_state, int nthreads) {
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1 || dstate > 1024) return -1;
  if (!x || !delta || !A || !B || !C || !y) return -1;
  const int64_t nch = batch * dim;
#ifdef _OPENMP
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int64_t ch = 0; ch < nch; ++ch) {
    const int64_t b = ch / dim, d = ch % dim;
    double h[1024];
    for (int64_t n = 0; n < dstate; ++n) h[n] = h0 ? h0[ch * dstate + n] : 0.0;
    scan_channel(seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, delta_bias, delta_softplus, zoh, b, d,
                 h, y + b * seqlen * dim + d, dim);
    if (last_state)
      for (int64_t n = 0; n < dstate; ++n) last_state[ch * dstate + n] = h[n];
  }
  (void)nthreads;
  return 0;
}

/* The same recurrence for a chosen set of channels only (sampling at full
 * size).  sel_b[k], sel_d[k] name channel k.  y_out: (nsel, seqlen);
 * state_out: (nsel, dstate) or NULL.  Starts from zero state. */
int oracle_scan_channels(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype, const void *x,
                         const void *delta, const float *A, const void *B, const void *C, const float *Dskip,
                         const void *z, const float *delta_bias, int delta_softplus, int64_t nsel,
                         const int64_t *sel_b, const int64_t *sel_d, double *y_out, double *state_out,
                         int nthreads) {
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1 || dstate > 1024 || nsel < 0) return -1;
  if (!x || !delta || !A || !B || !C || !y_out || (nsel > 0 && (!sel_b || !sel_d))) return -1;
  for (int64_t k = 0; k < nsel; ++k)
    if (sel_b[k] < 0 || sel_b[k] >= batch || sel_d[k] < 0 || sel_d[k] >= dim) return -1;
#ifdef _OPENMP
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int64_t k = 0; k < nsel; ++k) {
    double h[1024];
    for (int64_t n = 0; n < dstate; ++n) h[n] = 0.0;
    scan_channel(seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, delta_bias, delta_softplus, 0, sel_b[k],
                 sel_d[k], h, y_out + k * seqlen, 1);
    if (state_out)
      for (int64_t n = 0; n < dstate; ++n) state_out[k * dstate + n] = h[n];
  }
  (void)nthreads;
  return 0;
}

/* One decode step for every channel: the recurrence body at a single time
 * step, starting from `state` (batch, dim, dstate) doubles, which is updated
 * in place.  x, delta, z: (batch, dim); B, C: (batch, dstate); y: (batch, dim).
 * ("Mamba 论文精读" sec. 6: inference costs O(1) per token with a fixed-size
 * state and no cache of past inputs.) */
int oracle_state_update_ex(int64_t batch, int64_t dim, int64_t dstate, int dtype, double *state, const void *x,
                           const void *delta, const float *A, const void *B, const void *C, const float *Dskip,
                           const void *z, const float *delta_bias, int delta_softplus, int zoh, double *y);

int oracle_state_update(int64_t batch, int64_t dim, int64_t dstate, int dtype, double *state, const void *x,
                        const void *delta, const float *A, const void *B, const void *C, const float *Dskip,
                        const void *z, const float *delta_bias, int delta_softplus, double *y) {
  return oracle_state_update_ex(batch, dim, dstate, dtype, state, x, delta, A, B, C, Dskip, z, delta_bias,
                                delta_softplus, 0, y);
}

/* oracle_state_update with the choice of Bbar (zoh as in oracle_scan_ex). */
int oracle_state_update_ex(int64_t batch, int64_t dim, int64_t dstate, int dtype, double *state, const void *x,
                           const void *delta, const float *A, const void *B, const void *C, const float *Dskip,
                           const void *z, const float *delta_bias, int delta_softplus, int zoh, double *y) {
  if (batch < 0 || dim < 0 || dstate < 1 || dstate > 1024) return -1;
  if (!state || !x || !delta || !A || !B || !C || !y) return -1;
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t d = 0; d < dim; ++d) {
      const int64_t i_bd = b * dim + d;
      double v = load_elem(delta, dtype, i_bd) + (delta_bias ? (double)delta_bias[d] : 0.0);
      double dt = delta_softplus ? softplus(v) : v;
      double xt = load_elem(x, dtype, i_bd);
      double *h = state + i_bd * dstate;
      double acc = 0.0;
      for (int64_t n = 0; n < dstate; ++n) {
        double abar = exp(dt * (double)A[d * dstate + n]);
        if (zoh)
          h[n] = abar * h[n] + bbar_x(1, dt, (double)A[d * dstate + n], load_elem(B, dtype, b * dstate + n), xt);
        else
          h[n] = abar * h[n] + dt * load_elem(B, dtype, b * dstate + n) * xt;
        acc += load_elem(C, dtype, b * dstate + n) * h[n];
      }
      double yt = acc + (Dskip ? (double)Dskip[d] * xt : 0.0);
      if (z) yt *= silu(load_elem(z, dtype, i_bd));
      y[i_bd] = yt;
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------------
 * Backward pass of the scan: the gradients of L = sum_{b,t,d} dy[b,t,d] *
 * y[b,t,d] with respect to every input, by the adjoint of the recurrence.
 * The forward states are recomputed (the pages' backward recomputes Abar and
 * Bbar instead of storing the O(BLDN) intermediates: "mamba->jamba" sec. 2.3,
 * hardware-aware algorithm).  For one channel, with g_t = dL/dh_t:
 *
 *   y0_t = sum_n C_t[n] h_t[n] + D x_t,  y_t = y0_t * silu(z_t)
 *   dy0_t = dy_t * silu(z_t);   dz_t = dy_t * y0_t * silu'(z_t)
 *   g_t[n] = dy0_t C_t[n] + abar_{t+1}[n] g_{t+1}[n]      (g_L = 0)
 *   dC_t[n] += dy0_t h_t[n];  dD += dy0_t x_t
 *   dB_t[n] += g_t[n] dt_t x_t
 *   dx_t    = dy0_t D + sum_n g_t[n] dt_t B_t[n]
 *   ddt_t   = sum_n g_t[n] (B_t[n] x_t + A[n] abar_t[n] h_{t-1}[n])
 *   dA[n]  += g_t[n] dt_t abar_t[n] h_{t-1}[n]
 *   ddelta_t = ddt_t * (softplus ? sigmoid(delta_t + bias) : 1);  dbias += ddelta_t
 *
 * dy: (batch, L, dim) doubles.  Outputs (doubles, all written): dx, ddelta,
 * dz (batch, L, dim) (dz only when z is given); dB, dC (batch, L, dstate);
 * dA (dim, dstate); dD, ddelta_bias (dim) (only when D / delta_bias are
 * given).  The state starts at zero; last_state is not differentiated.
 * ------------------------------------------------------------------------- */
static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* Exact zero-order hold ("Mamba 论文精读" sec. 2.2), per (d, n) with z = dt A:
 *   u_t = phi B_t x_t,  phi = expm1(z) / A  (dt when A = 0),  dphi/ddt = exp(z) = abar,
 *   dphi/dA = (dt abar - phi) / A = (z expm1(z) + (z - expm1(z))) / A^2  (dt^2 / 2 when A = 0),
 * so the adjoint differs from the Delta B form in these terms only:
 *   dB_t += g phi x_t;  dx_t += g phi B_t;  ddt_t += g abar (B_t x_t + A h_{t-1});
 *   dA += g (dt abar h_{t-1} + B_t x_t dphi/dA). */
int oracle_scan_bwd_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype, const void *x,
                       const void *delta, const float *A, const void *B, const void *C, const float *Dskip,
                       const void *z, const float *delta_bias, int delta_softplus, int zoh, const double *dy,
                       double *dx, double *ddelta, double *dA, double *dB, double *dC, double *dD, double *dz,
                       double *ddelta_bias);
static double zoh_phi(double dt, double a) { return a == 0.0 ? dt : expm1(dt * a) / a; }
static double zoh_dphi_da(double dt, double a) {
  if (a == 0.0) return 0.5 * dt * dt;
  const double zz = dt * a, em = expm1(zz);
  return (zz * em + (zz - em)) / (a * a);
}

int oracle_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype, const void *x,
                    const void *delta, const float *A, const void *B, const void *C, const float *Dskip,
                    const void *z, const float *delta_bias, int delta_softplus, const double *dy, double *dx,
                    double *ddelta, double *dA, double *dB, double *dC, double *dD, double *dz,
                    double *ddelta_bias) {
  return oracle_scan_bwd_ex(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, delta_bias,
                            delta_softplus, 0, dy, dx, ddelta, dA, dB, dC, dD, dz, ddelta_bias);
}

int oracle_scan_bwd_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype, const void *x,
                       const void *delta, const float *A, const void *B, const void *C, const float *Dskip,
                       const void *z, const float *delta_bias, int delta_softplus, int zoh, const double *dy,
                       double *dx, double *ddelta, double *dA, double *dB, double *dC, double *dD, double *dz,
                       double *ddelta_bias) {
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1 || dstate > 1024) return -1;
  if (!x || !delta || !A || !B || !C || !dy || !dx || !ddelta || !dA || !dB || !dC) return -1;
  const int64_t L = seqlen, N = dstate;
  for (int64_t i = 0; i < dim * N; ++i) dA[i] = 0.0;
  for (int64_t i = 0; i < batch * L * N; ++i) dB[i] = dC[i] = 0.0;
  if (dD) for (int64_t d = 0; d < dim; ++d) dD[d] = 0.0;
  if (ddelta_bias) for (int64_t d = 0; d < dim; ++d) ddelta_bias[d] = 0.0;
  double *hs = (double *)malloc(sizeof(double) * (size_t)(L + 1) * (size_t)N);  /* h_{-1}=0 .. h_{L-1} */
  double *g = (double *)malloc(sizeof(double) * (size_t)N);
  if (!hs || !g) { free(hs); free(g); return -1; }
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t d = 0; d < dim; ++d) {
      /* forward: every state, h_t at hs[(t+1)*N] */
      for (int64_t n = 0; n < N; ++n) hs[n] = 0.0;
      for (int64_t t = 0; t < L; ++t) {
        const int64_t i_td = (b * L + t) * dim + d, i_tn = (b * L + t) * N;
        double v = load_elem(delta, dtype, i_td) + (delta_bias ? (double)delta_bias[d] : 0.0);
        double dt = delta_softplus ? softplus(v) : v;
        double xt = load_elem(x, dtype, i_td);
        for (int64_t n = 0; n < N; ++n)
          hs[(t + 1) * N + n] = exp(dt * (double)A[d * N + n]) * hs[t * N + n] +
                                bbar_x(zoh, dt, (double)A[d * N + n], load_elem(B, dtype, i_tn + n), xt);
      }
      /* backward */
      for (int64_t n = 0; n < N; ++n) g[n] = 0.0;
      for (int64_t t = L - 1; t >= 0; --t) {
        const int64_t i_td = (b * L + t) * dim + d, i_tn = (b * L + t) * N;
        double v = load_elem(delta, dtype, i_td) + (delta_bias ? (double)delta_bias[d] : 0.0);
        double dt = delta_softplus ? softplus(v) : v;
        double xt = load_elem(x, dtype, i_td);
        const double *h = hs + (t + 1) * N, *hp = hs + t * N;
        double y0 = Dskip ? (double)Dskip[d] * xt : 0.0;
        for (int64_t n = 0; n < N; ++n) y0 += load_elem(C, dtype, i_tn + n) * h[n];
        double dy0 = dy[i_td];
        if (z) {
          double zt = load_elem(z, dtype, i_td), sg = sigmoid(zt);
          dz[i_td] = dy[i_td] * y0 * (sg + zt * sg * (1.0 - sg));
          dy0 = dy[i_td] * zt * sg;
        }
        double dxt = Dskip ? dy0 * (double)Dskip[d] : 0.0, ddt = 0.0;
        if (dD) dD[d] += dy0 * xt;
        for (int64_t n = 0; n < N; ++n) {
          /* g holds g_{t+1} * abar_{t+1} from the step after; add this step's read-out */
          const double Bn = load_elem(B, dtype, i_tn + n), Cn = load_elem(C, dtype, i_tn + n);
          const double an = (double)A[d * N + n], abar = exp(dt * an);
          g[n] += dy0 * Cn;
          dC[i_tn + n] += dy0 * h[n];
          if (zoh) {
            const double phi = zoh_phi(dt, an);
            dB[i_tn + n] += g[n] * phi * xt;
            dxt += g[n] * phi * Bn;
            ddt += g[n] * abar * (Bn * xt + an * hp[n]);
            dA[d * N + n] += g[n] * (dt * abar * hp[n] + Bn * xt * zoh_dphi_da(dt, an));
          } else {
            dB[i_tn + n] += g[n] * dt * xt;
            dxt += g[n] * dt * Bn;
            ddt += g[n] * (Bn * xt + an * abar * hp[n]);
            dA[d * N + n] += g[n] * dt * abar * hp[n];
          }
          g[n] *= abar; /* carried to step t-1 */
        }
        dx[i_td] = dxt;
        const double dd = delta_softplus ? ddt * sigmoid(v) : ddt;
        ddelta[i_td] = dd;
        if (ddelta_bias) ddelta_bias[d] += dd;
      }
    }
  }
  free(hs);
  free(g);
  return 0;
}

/* ---------------------------------------------------------------------------
 * Mamba-2 state space dual (SSD) layer ("Mamba 论文精读" sec. 4.1: the recurrence
 * h_t = A_t h_{t-1} + B_t x_t, y_t = C_t h_t, dual to a masked structured
 * matrix; sec. 4.2: multi-head; sec. 5.2: the Mamba2 layer with headdim and
 * d_state).  A is one scalar per head, B and C are shared by the heads of a
 * group, and Bbar = dt B as in the selective scan.  For batch b, head h
 * (group g = h / (nheads / ngroups)) and head channel p, from S = h0[b,h,p,:]
 * (zero when h0 is NULL):
 *   dt = softplus(dt[b,t,h] + dt_bias[h])  (or without softplus)
 *   S[p,n] = exp(dt A[h]) S[p,n] + dt x[b,t,h,p] B[b,t,g,n]
 *   y[b,t,h,p] = sum_n C[b,t,g,n] S[p,n] + D[h] x[b,t,h,p];  y *= silu(z[b,t,h,p]) if z
 *   final_state[b,h,p,n] = S
 * x, z, y: (batch, L, nheads, headdim); dt: (batch, L, nheads); B, C: (batch,
 * L, ngroups, dstate); A, D, dt_bias: (nheads) fp32.
 * ------------------------------------------------------------------------- */
int oracle_ssd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups,
               int dtype, const void *x, const void *dt, const float *A, const void *B, const void *C,
               const float *Dskip, const void *z, const float *dt_bias, int dt_softplus, const double *h0,
               double *y, double *final_state, int nthreads) {
  if (batch < 0 || seqlen < 0 || nheads < 1 || headdim < 1 || dstate < 1 || ngroups < 1) return -1;
  if (nheads % ngroups != 0 || !x || !dt || !A || !B || !C || !y) return -1;
  const int64_t H = nheads, P = headdim, N = dstate, G = ngroups, hpg = H / G;
#ifdef _OPENMP
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int64_t bh = 0; bh < batch * H; ++bh) {
    const int64_t b = bh / H, h = bh % H, g = h / hpg;
    double *S = (double *)calloc((size_t)(P * N), sizeof(double));
    if (!S) continue;
    if (h0)
      for (int64_t i = 0; i < P * N; ++i) S[i] = h0[bh * P * N + i];
    for (int64_t t = 0; t < seqlen; ++t) {
      const double v = load_elem(dt, dtype, (b * seqlen + t) * H + h) + (dt_bias ? (double)dt_bias[h] : 0.0);
      const double d = dt_softplus ? softplus(v) : v;
      const double a = exp(d * (double)A[h]);
      const int64_t ibc = ((b * seqlen + t) * G + g) * N;
      for (int64_t p = 0; p < P; ++p) {
        const int64_t ix = ((b * seqlen + t) * H + h) * P + p;
        const double xv = load_elem(x, dtype, ix);
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          S[p * N + n] = a * S[p * N + n] + d * xv * load_elem(B, dtype, ibc + n);
          acc += load_elem(C, dtype, ibc + n) * S[p * N + n];
        }
        double yv = acc + (Dskip ? (double)Dskip[h] * xv : 0.0);
        if (z) yv *= silu(load_elem(z, dtype, ix));
        y[ix] = yv;
      }
    }
    if (final_state)
      for (int64_t i = 0; i < P * N; ++i) final_state[bh * P * N + i] = S[i];
    free(S);
  }
  (void)nthreads;
  return 0;
}

/* ---------------------------------------------------------------------------
 * Depthwise causal convolution that feeds the scan in the Mamba block
 * ("Mamba 论文精读" (youngju.dev), sec. 3.4 "Mamba Block 架构", the MambaBlock
 * listing): a Conv1d with one group per channel, kernel width K and K-1
 * zeros of padding, cut back to the first L outputs, then SiLU.  PyTorch's
 * Conv1d is a cross-correlation, so for channel d of batch row b:
 *
 *   y[t]  = bias[d] + sum_{k=0..K-1} w[d,k] * xin[t - (K-1) + k]
 *   xin[s] = x[b,s,d] for s >= 0; for -(K-1) <= s < 0 it is the initial
 *            state init[b,d,(K-1)+s] (zero without one: the padding)
 *   out[b,t,d]   = silu ? silu(y[t]) : y[t]
 *   final[b,d,j] = xin[L-(K-1)+j], j = 0..K-2  (the last K-1 inputs, oldest first)
 *
 * x, out: (batch, L, dim); w: (dim, K) fp32; bias: (dim) fp32 or NULL;
 * init, final: (batch, dim, K-1) (init in the storage type of x, or NULL;
 * final as doubles, or NULL).  The state layout is a reading: the pages
 * define no convolution state.
 * ------------------------------------------------------------------------- */
int oracle_causal_conv1d(int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int dtype, const void *x,
                         const float *w, const float *bias, const void *init, int apply_silu, double *out,
                         double *final_state) {
  if (batch < 0 || seqlen < 0 || dim < 0 || width < 1 || width > 64) return -1;
  if (!x || !w || !out) return -1;
  const int64_t K = width;
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t d = 0; d < dim; ++d) {
      /* xin[s] for s in [-(K-1), L) */
      for (int64_t t = 0; t < seqlen; ++t) {
        double acc = bias ? (double)bias[d] : 0.0;
        for (int64_t k = 0; k < K; ++k) {
          const int64_t s = t - (K - 1) + k;
          double v;
          if (s >= 0)
            v = load_elem(x, dtype, (b * seqlen + s) * dim + d);
          else
            v = init ? load_elem(init, dtype, (b * dim + d) * (K - 1) + (K - 1) + s) : 0.0;
          acc += (double)w[d * K + k] * v;
        }
        out[(b * seqlen + t) * dim + d] = apply_silu ? silu(acc) : acc;
      }
      if (final_state) {
        for (int64_t j = 0; j < K - 1; ++j) {
          const int64_t s = seqlen - (K - 1) + j;
          double v;
          if (s >= 0)
            v = load_elem(x, dtype, (b * seqlen + s) * dim + d);
          else
            v = init ? load_elem(init, dtype, (b * dim + d) * (K - 1) + (K - 1) + s) : 0.0;
          final_state[(b * dim + d) * (K - 1) + j] = v;
        }
      }
    }
  }
  return 0;
}

/* One decode step of the same convolution: the window is the K-1 stored
 * inputs (oldest first) followed by the new input x[b,d]; then the state
 * drops its oldest input and appends x.  state: (batch, dim, K-1) doubles,
 * updated in place; x, out: (batch, dim). */
int oracle_conv1d_update(int64_t batch, int64_t dim, int64_t width, int dtype, double *state, const void *x,
                         const float *w, const float *bias, int apply_silu, double *out) {
  if (batch < 0 || dim < 0 || width < 1 || width > 64) return -1;
  if (!state || !x || !w || !out) return -1;
  const int64_t K = width;
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t d = 0; d < dim; ++d) {
      double *st = state + (b * dim + d) * (K - 1);
      const double xt = load_elem(x, dtype, b * dim + d);
      double acc = bias ? (double)bias[d] : 0.0;
      for (int64_t k = 0; k < K - 1; ++k) acc += (double)w[d * K + k] * st[k];
      acc += (double)w[d * K + K - 1] * xt;
      for (int64_t k = 0; k + 1 < K - 1; ++k) st[k] = st[k + 1];
      if (K > 1) st[K - 2] = xt;
      out[b * dim + d] = apply_silu ? silu(acc) : acc;
    }
  }
  return 0;
}

/* Scalar entry points so tests can pin the prologue/epilogue functions. */
double oracle_softplus(double v) { return softplus(v); }
double oracle_silu(double z) { return silu(z); }
double oracle_widen(const void *p, int dtype, int64_t i) { return load_elem(p, dtype, i); }

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
