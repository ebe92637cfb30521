/*
 * sscan_oracle.c -- the fp64 CPU oracle for the selective state-space scan.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's
 * cpu_baseline leg load this library. The product path (libsscan and its
 * Python binding) never calls it, and it shares no code, header, table or
 * constant with the HIP kernels.
 *
 * Every function is the plain definition written out as a token loop in
 * double precision: no chunking, no blocking, no reordering. Independent
 * lanes (a batch row and a channel, or a batch row, a head and a head_dim row)
 * run in parallel with OpenMP; each lane's arithmetic is sequential in a fixed
 * order, so results do not depend on the thread count.
 *
 * Sources (the pages, by title and section):
 *  [M1]  "Mamba" (nnterp guide, architectures): the opening paragraph gives,
 *        per channel with a state of state_dim numbers, h = exp(dt*A)*h + dt*B*x
 *        and y = C.h + D*x; section "The values" gives dt = softplus(dt + dt_bias),
 *        decays = dt*A with A per channel and state dimension, one B/C group
 *        shared by every channel, state_input None on a prompt (zeros), and
 *        state_output the state after the last token.
 *  [TT]  "Mamba" (tokentrails lineage), step "Selectivity" (A-bar = exp(dt A))
 *        and section "Code" (A = -exp(A_log), the token loop, and the gate
 *        y * silu(z) before out_proj).
 *  [FM]  "Falcon-Mamba" (nnterp encyclopedia), section "Where the norms sit":
 *        weightless RMS norms on B and C (b * rsqrt(mean(b^2) + eps)) before
 *        the scan; section "The block, in order": the gate after the scan.
 *  [M2]  "Mamba-2" (nnterp encyclopedia), section "The mixer's values": one
 *        scalar decay per head and token (betas = softplus(dt + dt_bias),
 *        decays = betas * A), groups served by repeat_interleave; section
 *        "The block, in order": y = ssd(...) + D*x then the gate; section
 *        "The state": the state after every token, the last one equals
 *        state_output; section "The hidden attention".
 *
 * Parity status: every function here is pinned by the CPU tests (hand cases,
 * the time-invariant closed form, the hidden-attention form, split-sequence
 * and state invariants, the RMS-of-one property); see tests/test_oracle_pins.py.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_MAX_N 1024

/* softplus(v) = log(1 + e^v), in the overflow-free form max(v,0) + log1p(e^-|v|).
 * softplus(-inf) = 0 exactly, which makes a -inf step raw value a zero step. */
static double softplus(double v) { return fmax(v, 0.0) + log1p(exp(-fabs(v))); }

/* silu(z) = z * sigmoid(z) = z / (1 + e^-z) */
static double silu(double z) { return z / (1.0 + exp(-z)); }

int oracle_abi_version(void) { return 1; }

/* Threads an OpenMP loop of the oracle uses (for reporting the CPU baseline). */
int oracle_threads(void) { return omp_get_max_threads(); }

/* Sets the threads of the oracle's later loops on the calling thread (for timing the
 * CPU baseline on one core); the arithmetic of each lane does not depend on it. */
void oracle_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}

/* Weightless RMS norm of every [state_dim] vector of a [rows, state_dim] array
 * ([FM] "Where the norms sit"): out = v / sqrt(mean(v^2) + eps). */
static void rms_norm_rows(int64_t rows, int64_t n, const double* in, double eps, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const double* v = in + r * n;
    double ss = 0.0;
    for (int64_t k = 0; k < n; ++k) ss += v[k] * v[k];
    double inv = 1.0 / sqrt(ss / (double)n + eps);
    for (int64_t k = 0; k < n; ++k) out[r * n + k] = v[k] * inv;
  }
}

/*
 * Mamba-1 selective scan ([M1], [TT], [FM]).
 *   x, dt_raw, z : [batch, seqlen, channels]      (z may be NULL: no gate)
 *   dt_bias, D   : [channels]
 *   A_log        : [channels, state_dim]           (A = -exp(A_log))
 *   B, C         : [batch, seqlen, ngroups, state_dim]; channel c reads group
 *                  c / (channels / ngroups)
 *   bc_eps       : > 0 applies the weightless RMS norm to B and C first
 *   h0           : [batch, channels, state_dim] or NULL (zeros)
 *   y            : [batch, seqlen, channels]
 *   h_out        : [batch, channels, state_dim]
 *   states       : [batch, seqlen, channels, state_dim] or NULL
 * Returns 0, or -1 for an invalid shape.
 */
int oracle_mamba1(int64_t batch, int64_t seqlen, int64_t channels, int64_t state_dim, int64_t ngroups,
                  const double* x, const double* dt_raw, const double* dt_bias, const double* A_log,
                  const double* B, const double* C, const double* D, const double* z, double bc_eps,
                  const double* h0, double* y, double* h_out, double* states) {
  if (batch < 0 || seqlen < 0 || channels <= 0 || state_dim <= 0 || state_dim > ORACLE_MAX_N ||
      ngroups <= 0 || channels % ngroups != 0)
    return -1;
  const int64_t L = seqlen, Dc = channels, N = state_dim, G = ngroups;
  const int64_t per_group = Dc / G;

  /* The norms act on B and C as x_proj produced them, before the scan reads them. */
  const double* Bs = B;
  const double* Cs = C;
  double* nb = NULL;
  double* nc = NULL;
  if (bc_eps > 0.0 && batch * L > 0) {
    nb = (double*)malloc(sizeof(double) * (size_t)(batch * L * G * N));
    nc = (double*)malloc(sizeof(double) * (size_t)(batch * L * G * N));
    if (!nb || !nc) { free(nb); free(nc); return -2; }
    rms_norm_rows(batch * L * G, N, B, bc_eps, nb);
    rms_norm_rows(batch * L * G, N, C, bc_eps, nc);
    Bs = nb;
    Cs = nc;
  }

#pragma omp parallel for schedule(static)
  for (int64_t lane = 0; lane < batch * Dc; ++lane) {
    const int64_t b = lane / Dc, c = lane % Dc, g = c / per_group;
    double h[ORACLE_MAX_N], A[ORACLE_MAX_N];
    for (int64_t n = 0; n < N; ++n) {
      A[n] = -exp(A_log[c * N + n]);
      h[n] = h0 ? h0[(b * Dc + c) * N + n] : 0.0;
    }
    for (int64_t t = 0; t < L; ++t) {
      const int64_t bt = b * L + t;
      const double xv = x[bt * Dc + c];
      const double dt = softplus(dt_raw[bt * Dc + c] + dt_bias[c]);
      const double* Bt = Bs + (bt * G + g) * N;
      const double* Ct = Cs + (bt * G + g) * N;
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        h[n] = exp(dt * A[n]) * h[n] + dt * Bt[n] * xv;
        acc += Ct[n] * h[n];
      }
      double yv = acc + D[c] * xv;
      if (z) yv *= silu(z[bt * Dc + c]);
      y[bt * Dc + c] = yv;
      if (states)
        for (int64_t n = 0; n < N; ++n) states[(bt * Dc + c) * N + n] = h[n];
    }
    for (int64_t n = 0; n < N; ++n) h_out[(b * Dc + c) * N + n] = h[n];
  }
  free(nb);
  free(nc);
  return 0;
}

/*
 * Mamba-2 (SSD) scan ([M2]): the same recurrence with one scalar decay per head
 * and token, and a [head_dim, state_dim] state per head. Written separately
 * from oracle_mamba1 so that "SSD equals Mamba-1 with A tied per head" compares
 * two code paths.
 *   x, z    : [batch, seqlen, nheads, head_dim]   (z may be NULL)
 *   dt_raw  : [batch, seqlen, nheads]
 *   dt_bias, A_log, D : [nheads]
 *   B, C    : [batch, seqlen, ngroups, state_dim]; head h reads group h / (nheads / ngroups)
 *   h0, h_out : [batch, nheads, head_dim, state_dim]  (h0 may be NULL)
 *   y       : [batch, seqlen, nheads, head_dim]
 *   states  : [batch, seqlen, nheads, head_dim, state_dim] or NULL
 */
int oracle_ssd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t head_dim, int64_t state_dim,
               int64_t ngroups, const double* x, const double* dt_raw, const double* dt_bias,
               const double* A_log, const double* B, const double* C, const double* D, const double* z,
               const double* h0, double* y, double* h_out, double* states) {
  if (batch < 0 || seqlen < 0 || nheads <= 0 || head_dim <= 0 || state_dim <= 0 ||
      state_dim > ORACLE_MAX_N || ngroups <= 0 || nheads % ngroups != 0)
    return -1;
  const int64_t L = seqlen, H = nheads, P = head_dim, N = state_dim, G = ngroups;
  const int64_t heads_per_group = H / G;
#pragma omp parallel for schedule(static)
  for (int64_t lane = 0; lane < batch * H * P; ++lane) {
    const int64_t b = lane / (H * P), hd = (lane / P) % H, p = lane % P;
    const int64_t g = hd / heads_per_group;
    const double A = -exp(A_log[hd]);
    double s[ORACLE_MAX_N];
    for (int64_t n = 0; n < N; ++n) s[n] = h0 ? h0[((b * H + hd) * P + p) * N + n] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
      const int64_t bt = b * L + t;
      const double dt = softplus(dt_raw[bt * H + hd] + dt_bias[hd]);
      const double decay = exp(dt * A);
      const double xv = x[(bt * H + hd) * P + p];
      const double* Bt = B + (bt * G + g) * N;
      const double* Ct = C + (bt * G + g) * N;
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        s[n] = decay * s[n] + dt * Bt[n] * xv;
        acc += Ct[n] * s[n];
      }
      double yv = acc + D[hd] * xv;
      if (z) yv *= silu(z[(bt * H + hd) * P + p]);
      y[(bt * H + hd) * P + p] = yv;
      if (states)
        for (int64_t n = 0; n < N; ++n) states[((bt * H + hd) * P + p) * N + n] = s[n];
    }
    for (int64_t n = 0; n < N; ++n) h_out[((b * H + hd) * P + p) * N + n] = s[n];
  }
  return 0;
}

/*
 * The hidden attention of the SSD scan ([M2] "The hidden attention"): per head
 * the scan is a causal linear map over tokens, y_t = sum_s alpha[t, s] x_s + D x_t
 * (before the gate), with
 *     alpha[t, s] = (C_t . B_s) * exp(decays_{s+1} + ... + decays_t) * betas_s,  s <= t,
 * and 0 for s > t; betas = softplus(dt_raw + dt_bias), decays = betas * A,
 * A = -exp(A_log) ([M2] "The mixer's values"). The decay sum is formed directly
 * for each pair (no difference of running sums).
 *   dt_raw  : [batch, seqlen, nheads];  dt_bias, A_log : [nheads]
 *   B, C    : [batch, seqlen, ngroups, state_dim]; head h reads group h / (nheads / ngroups)
 *   alpha   : [batch, seqlen (query t), seqlen (key s), nheads]
 */
int oracle_ssd_attention(int64_t batch, int64_t seqlen, int64_t nheads, int64_t state_dim, int64_t ngroups,
                         const double* dt_raw, const double* dt_bias, const double* A_log, const double* B,
                         const double* C, double* alpha) {
  if (batch < 0 || seqlen < 0 || nheads <= 0 || state_dim <= 0 || ngroups <= 0 || nheads % ngroups != 0)
    return -1;
  const int64_t L = seqlen, H = nheads, N = state_dim, G = ngroups;
  const int64_t heads_per_group = H / G;
#pragma omp parallel for schedule(static)
  for (int64_t row = 0; row < batch * L; ++row) {
    const int64_t b = row / L, t = row % L;
    for (int64_t s = 0; s < L; ++s) {
      for (int64_t h = 0; h < H; ++h) {
        double v = 0.0;
        if (s <= t) {
          const int64_t g = h / heads_per_group;
          const double A = -exp(A_log[h]);
          const double* Ct = C + ((b * L + t) * G + g) * N;
          const double* Bs = B + ((b * L + s) * G + g) * N;
          double cb = 0.0;
          for (int64_t n = 0; n < N; ++n) cb += Ct[n] * Bs[n];
          double dsum = 0.0;  /* decays_{s+1} + ... + decays_t */
          for (int64_t k = s + 1; k <= t; ++k) dsum += softplus(dt_raw[(b * L + k) * H + h] + dt_bias[h]) * A;
          const double beta_s = softplus(dt_raw[(b * L + s) * H + h] + dt_bias[h]);
          v = cb * exp(dsum) * beta_s;
        }
        alpha[((b * L + t) * L + s) * H + h] = v;
      }
    }
  }
  return 0;
}

/*
 * Causal depthwise conv1d of width W followed by silu, the step in front of the
 * scan ("Mamba-2", section "The block, in order": x, B, C = silu(conv1d(xBC)),
 * causal, width 4; "Mamba" tokentrails section "Code": depthwise, width 4).
 * Output token t reads inputs t-W+1 .. t; positions before the call come from
 * conv_state (the W-1 previous inputs, oldest first) or are zero.
 *   x, out      : [batch, seqlen, channels]
 *   weight      : [channels, W];  bias : [channels] or NULL
 *   conv_state  : [batch, channels, W-1] or NULL (zeros)
 *   state_out   : [batch, channels, W-1] or NULL: the last W-1 inputs
 */
int oracle_conv1d_silu(int64_t batch, int64_t seqlen, int64_t channels, int64_t width,
                       const double* x, const double* weight, const double* bias,
                       const double* conv_state, double* out, double* state_out) {
  if (batch < 0 || seqlen < 0 || channels <= 0 || width <= 0 || width > 64) return -1;
  const int64_t L = seqlen, Dc = channels, W = width;
#pragma omp parallel for schedule(static)
  for (int64_t lane = 0; lane < batch * Dc; ++lane) {
    const int64_t b = lane / Dc, c = lane % Dc;
    double hist[64];                  /* the inputs at positions t-W+1 .. t-1 */
    for (int64_t k = 0; k < W - 1; ++k) hist[k] = conv_state ? conv_state[(b * Dc + c) * (W - 1) + k] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
      const double xt = x[(b * L + t) * Dc + c];
      double acc = bias ? bias[c] : 0.0;
      for (int64_t k = 0; k < W - 1; ++k) acc += weight[c * W + k] * hist[k];
      acc += weight[c * W + (W - 1)] * xt;
      out[(b * L + t) * Dc + c] = silu(acc);
      for (int64_t k = 0; k + 1 < W - 1; ++k) hist[k] = hist[k + 1];
      if (W > 1) hist[W - 2] = xt;
    }
    if (state_out)
      for (int64_t k = 0; k < W - 1; ++k) state_out[(b * Dc + c) * (W - 1) + k] = hist[k];
  }
  return 0;
}

/*
 * Gated RMS norm after the SSD ("Mamba-2", section "The block, in order" and
 * the note under it): multiply y by silu(z), then normalize over the mixer's
 * whole width and scale by the norm's weight:
 *   g = y * silu(z);  out = g / sqrt(mean(g^2) + eps) * weight
 *   y, z, out : [rows, width];  weight : [width]
 */
int oracle_gated_rmsnorm(int64_t rows, int64_t width, const double* y, const double* z,
                         const double* weight, double eps, double* out) {
  if (rows < 0 || width <= 0) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double ss = 0.0;
    for (int64_t k = 0; k < width; ++k) {
      double g = y[r * width + k] * silu(z[r * width + k]);
      out[r * width + k] = g;
      ss += g * g;
    }
    double inv = 1.0 / sqrt(ss / (double)width + eps);
    for (int64_t k = 0; k < width; ++k) out[r * width + k] = out[r * width + k] * inv * weight[k];
  }
  return 0;
}
