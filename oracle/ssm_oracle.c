/*
 * Plain fp64 CPU oracle for the selective scan (S6) and its decode step.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests, the smoke check and the bench's CPU
 * baseline may call this code. It shares nothing with the HIP path: no
 * kernels, headers, helpers or constants.
 *
 * What it computes, per (batch row b, channel d), strictly in token order:
 *
 *   h[n] = state_in[b,d,n]  (or 0)                               initial state
 *   for t = 0 .. L-1:
 *     dA[n]  = exp(delta[b,t,d] * A[d,n])                        A-bar, exp-Euler rule
 *     dBx[n] = delta[b,t,d] * Bt[b,t,n] * x[b,t,d]               B-bar = delta*B
 *     h[n]   = dA[n] * h[n] + dBx[n]                             recurrence
 *     y      = sum_n Ct[b,t,n] * h[n]  (+ Dskip[d] * x[b,t,d])    readout, skip
 *     y      = y * z * sigmoid(z)      (when z is given)         silu gate
 *     out[b,t,d] = y
 *   state_out[b,d,:] = h
 *
 * Sources (the web pages on Mamba this method comes from):
 *  - discretisation A-bar = exp(delta*A) and the first-order input rule
 *    B-bar = delta*B: "Notas sobre Mamba", section "Preliminares" (the remark
 *    after the discrete recurrence) and section "Recorrência trapezoidal"
 *    (the exponential-Euler update); the Mamba-2/SSD production blog post,
 *    section "Como o Mamba-1 alcançou complexidade linear" (the two S6
 *    equations, with the D skip).
 *  - time-varying recurrence and readout y_t = C_t^T h_t with the readout
 *    taken on the updated state: "Notas sobre Mamba", section "O mecanismo
 *    de seleção (S6)".
 *  - the silu(z) gate multiplying the SSM output: "Notas sobre Mamba",
 *    section "O bloco Mamba" (flowchart); silu(z) = z * sigmoid(z).
 *  - the single-token step on a stored state: the blog post's
 *    SelectiveSSM.forward_step listing (taken as a description of what is
 *    computed) and "Notas sobre Mamba", section "Preliminares" (recurrent
 *    mode with a constant-size state).
 *
 * The step size may also be given before its activation: delta is then
 * softplus(delta_raw + dt_bias[d]), the pre-activation being a per-token
 * projection and dt_bias a per-channel parameter ("Notas sobre Mamba",
 * section "O mecanismo de seleção (S6)": delta_t as the softplus of a linear
 * map of x_t plus a bias; the blog post's forward_step listing applies the
 * same softplus to its projected delta). oracle_softplus_bias computes that
 * activation; the scan and the step then run on its result unchanged.
 *
 * The exponential-trapezoidal variant (oracle_scan_trap, oracle_step_trap)
 * replaces the input term of the recurrence by a blend of the previous and
 * the current token's input, with a per-token weight lam in [0, 1] ("Notas
 * sobre Mamba", section "Recorrência trapezoidal", the generalised
 * exponential-trapezoidal rule and its coefficients alpha, beta, gamma);
 * lam = 1 gives the exponential-Euler scan above back.
 *
 * oracle_ssd is the Mamba-2 state space dual (SSD) layer: the same recurrence
 * with the transition restricted to a scalar per head times the identity, so
 * each head keeps a (P, N) state updated by an outer product ("Mamba-2 e
 * State Space Duality (SSD)"; "Notas sobre Mamba", section "A forma dual:
 * atenção mascarada", where the scalar transition a_t I and the recurrent
 * form of the dual are given).
 *
 * oracle_scan_bwd is the gradient of the scan (reverse mode, by hand): the
 * pages give the forward pass and say that the states are recomputed rather
 * than stored for the backward ("Notas sobre Mamba", section "A varredura
 * paralela ciente do hardware"); the gradient itself is the chain rule applied
 * to the recurrence above, written out below.
 *
 * Everything is float64 and uses libm exp()/log1p(); no fast-math, no
 * reordering of the token loop. OpenMP only splits independent (b, d) rows
 * across threads.
 */
#include <math.h>
#include <stdlib.h>
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX3(a, b, c, B_, C_) (((int64_t)(a) * (B_) + (b)) * (C_) + (c))

/* Returns the number of threads the parallel loops will use. */
int oracle_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) return nthreads;
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/*
 * Full selective scan over L tokens.
 *   x, delta, z, y : (batch, L, D)   z may be NULL (no gate)
 *   A              : (D, N)
 *   Bt, Ct         : (batch, L, N)
 *   Dskip          : (D) or NULL (no skip term)
 *   state_in       : (batch, D, N) or NULL (zero state)
 *   state_out      : (batch, D, N) or NULL
 * Returns 0, or -1 on a bad size.
 */
int oracle_scan(int64_t batch, int64_t L, int64_t D, int64_t N,
                const double *x, const double *delta, const double *A,
                const double *Bt, const double *Ct, const double *Dskip,
                const double *z, const double *state_in, double *state_out,
                double *y, int nthreads)
{
    if (batch < 0 || L < 0 || D < 0 || N < 1 || N > 4096) return -1;
    int64_t rows = batch * D;
    int nt = oracle_threads(nthreads);
    (void)nt;
#pragma omp parallel for schedule(dynamic, 4) num_threads(nt)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / D, d = r % D;
        double h[4096];
        for (int64_t n = 0; n < N; ++n)
            h[n] = state_in ? state_in[IDX3(b, d, n, D, N)] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            double dt = delta[IDX3(b, t, d, L, D)];
            double u = x[IDX3(b, t, d, L, D)];
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double dA = exp(dt * A[d * N + n]);
                double dBx = dt * Bt[IDX3(b, t, n, L, N)] * u;
                h[n] = dA * h[n] + dBx;
                acc += Ct[IDX3(b, t, n, L, N)] * h[n];
            }
            if (Dskip) acc += Dskip[d] * u;
            if (z) {
                double g = z[IDX3(b, t, d, L, D)];
                acc *= g / (1.0 + exp(-g));
            }
            y[IDX3(b, t, d, L, D)] = acc;
        }
        if (state_out)
            for (int64_t n = 0; n < N; ++n) state_out[IDX3(b, d, n, D, N)] = h[n];
    }
    return 0;
}

/*
 * Step-size activation: out[r, d] = softplus(raw[r, d] + bias[d]) for the
 * `rows` rows of D channels of a (rows, D) array; bias may be NULL (zero).
 * softplus(u) = log(1 + exp(u)), evaluated as max(u, 0) + log1p(exp(-|u|)).
 */
int oracle_softplus_bias(int64_t rows, int64_t D, const double *raw, const double *bias, double *out)
{
    if (rows < 0 || D < 0) return -1;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t d = 0; d < D; ++d) {
            double u = raw[r * D + d] + (bias ? bias[d] : 0.0);
            out[r * D + d] = (u > 0.0 ? u : 0.0) + log1p(exp(-fabs(u)));
        }
    return 0;
}

/*
 * The x branch of the Mamba block ahead of the scan: a short causal
 * convolution over the tokens, separately per channel, then SiLU ("Notas
 * sobre Mamba", section "O bloco Mamba": the projection, a short depthwise
 * convolution that takes in local context, SiLU, then S6; the Mamba-2 layer
 * configuration on the SSD production blog post gives its width, d_conv = 4).
 * Per (b, t, d), with taps w[d, 0..3] (tap 3 on the token itself) and bias
 * cb[d]:
 *   u   = cb[d] + sum_{j=0..3} w[d, j] * xr(b, t - 3 + j, d)
 *   out = u / (1 + exp(-u))                                       SiLU
 * where xr is x for tokens 0..L-1 and, before token 0, the raw x of the
 * three tokens before the call (state[b, d, 0..2], oldest first) or zero.
 * cb and state may be NULL.
 */
int oracle_conv_silu(int64_t batch, int64_t L, int64_t D, const double *x, const double *w, const double *cb,
                     const double *state, double *out)
{
    if (batch < 0 || L < 0 || D < 0) return -1;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t d = 0; d < D; ++d)
            for (int64_t t = 0; t < L; ++t) {
                double u = cb ? cb[d] : 0.0;
                for (int64_t j = 0; j < 4; ++j) {
                    int64_t s = t - 3 + j;
                    double v;
                    if (s >= 0) v = x[IDX3(b, s, d, L, D)];
                    else v = state ? state[IDX3(b, d, s + 3, D, 3)] : 0.0;
                    u += w[d * 4 + j] * v;
                }
                out[IDX3(b, t, d, L, D)] = u / (1.0 + exp(-u));
            }
    return 0;
}

/*
 * Gradient of oracle_conv_silu for a loss whose gradient with respect to its
 * output is gout (batch, L, D), by the chain rule (reverse mode, by hand).
 * With u and the window xr as in oracle_conv_silu and
 *   du[t]     = gout[t] * sigmoid(u[t]) * (1 + u[t] * (1 - sigmoid(u[t])))    (SiLU')
 * the gradients are
 *   gx[s]     = sum_j w[d, j] * du[s + 3 - j]     over tokens s + 3 - j in 0..L-1
 *   gw[d, j]  = sum_{b, t} du[t] * xr(b, t - 3 + j, d)
 *   gb[d]     = sum_{b, t} du[t]
 *   gstate[b, d, k] (the raw x of token k - 3) = sum_j w[d, j] * du[k - j], k - j >= 0
 * gw and gb are overwritten (not accumulated); gb, state and gstate may be
 * NULL.
 */
int oracle_conv_silu_bwd(int64_t batch, int64_t L, int64_t D, const double *x, const double *w, const double *cb,
                         const double *state, const double *gout, double *gx, double *gw, double *gb,
                         double *gstate)
{
    if (batch < 0 || L < 0 || D < 0) return -1;
    double *du = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    if (!du) return -1;
    for (int64_t d = 0; d < D; ++d) {
        for (int64_t j = 0; j < 4; ++j) gw[d * 4 + j] = 0.0;
        if (gb) gb[d] = 0.0;
    }
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t d = 0; d < D; ++d) {
            for (int64_t t = 0; t < L; ++t) {
                double u = cb ? cb[d] : 0.0;
                for (int64_t j = 0; j < 4; ++j) {
                    int64_t s = t - 3 + j;
                    double v;
                    if (s >= 0) v = x[IDX3(b, s, d, L, D)];
                    else v = state ? state[IDX3(b, d, s + 3, D, 3)] : 0.0;
                    u += w[d * 4 + j] * v;
                }
                double sg = 1.0 / (1.0 + exp(-u));
                du[t] = gout[IDX3(b, t, d, L, D)] * sg * (1.0 + u * (1.0 - sg));
                for (int64_t j = 0; j < 4; ++j) {
                    int64_t s = t - 3 + j;
                    double v;
                    if (s >= 0) v = x[IDX3(b, s, d, L, D)];
                    else v = state ? state[IDX3(b, d, s + 3, D, 3)] : 0.0;
                    gw[d * 4 + j] += du[t] * v;
                }
                if (gb) gb[d] += du[t];
            }
            for (int64_t s = 0; s < L; ++s) {
                double g = 0.0;
                for (int64_t j = 0; j < 4; ++j) {
                    int64_t t = s + 3 - j;
                    if (t < L) g += w[d * 4 + j] * du[t];
                }
                gx[IDX3(b, s, d, L, D)] = g;
            }
            if (gstate)
                for (int64_t k = 0; k < 3; ++k) {
                    double g = 0.0;
                    for (int64_t j = 0; j <= k; ++j)
                        if (k - j < L) g += w[d * 4 + j] * du[k - j];
                    gstate[IDX3(b, d, k, D, 3)] = g;
                }
        }
    free(du);
    return 0;
}

/*
 * Gradient of oracle_scan_trap for the loss sum(dy * y) + sum(dstate *
 * state_out), by the chain rule through its recurrence (reverse mode, by
 * hand). With G_t the gradient of h_t (from the readout of token t and from
 * h_{t+1} = alpha_{t+1} h_t + ...):
 *   G_t      = Ct[t] ds_t + alpha_{t+1} G_{t+1},        ds_t = dy_t silu(z_t)
 *   dv_t     = gamma_t G_t + beta_{t+1} G_{t+1}          (v_t feeds h_t and h_{t+1})
 *   ddelta_t = sum_n G_t (A alpha (h_{t-1} + (1 - lam) delta v_{t-1})
 *                         + (1 - lam) alpha v_{t-1} + lam v_t)
 *   dlam_t   = sum_n G_t delta (v_t - alpha v_{t-1})
 *   dA       = sum_t G_t delta alpha (h_{t-1} + (1 - lam) delta v_{t-1})
 *   dx_t     = sum_n dv_t Bt[t] (+ Dskip ds_t), dBt[t] = sum_d dv_t x_t
 * and dv_{-1} = beta_0 G_0 for the token before the first: dx_prev =
 * sum_n dv_{-1} B_prev, dB_prev = sum_d dv_{-1} x_prev (written only when
 * x_prev and B_prev are given). dstate_in = alpha_0 G_0.
 * Outputs (all written): dx, ddelta, dlam (batch, L, D); dA (D, N); dBt, dCt
 * (batch, L, N); dDskip (D) when Dskip; dz when z; dx_prev (batch, D) and
 * dB_prev (batch, N) when x_prev and B_prev; dstate_in (batch, D, N).
 */
int oracle_scan_bwd_trap(int64_t batch, int64_t L, int64_t D, int64_t N,
                         const double *x, const double *delta, const double *lam, const double *A,
                         const double *Bt, const double *Ct, const double *Dskip, const double *z,
                         const double *x_prev, const double *B_prev, const double *state_in,
                         const double *dy, const double *dstate,
                         double *dx, double *ddelta, double *dlam, double *dA, double *dBt, double *dCt,
                         double *dDskip, double *dz, double *dx_prev, double *dB_prev, double *dstate_in)
{
    if (batch < 0 || L < 0 || D < 0 || N < 1 || N > 4096) return -1;
    const int prev = x_prev && B_prev;
    double *H = (double *)malloc((size_t)((L + 1) * N) * sizeof(double));  /* H[(t + 1) N + n] = h_t */
    if (!H) return -1;
    for (int64_t i = 0; i < D * N; ++i) dA[i] = 0.0;
    for (int64_t i = 0; i < batch * L * N; ++i) dBt[i] = dCt[i] = 0.0;
    if (Dskip)
        for (int64_t d = 0; d < D; ++d) dDskip[d] = 0.0;
    if (prev)
        for (int64_t i = 0; i < batch * N; ++i) dB_prev[i] = 0.0;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t d = 0; d < D; ++d) {
            /* the input of token t - 1 (token -1: the earlier token, or none) */
#define VPREV(t, n) ((t) > 0 ? Bt[IDX3(b, (t) - 1, n, L, N)] * x[IDX3(b, (t) - 1, d, L, D)] \
                             : (prev ? B_prev[b * N + (n)] * x_prev[b * D + d] : 0.0))
            for (int64_t n = 0; n < N; ++n) H[n] = state_in ? state_in[IDX3(b, d, n, D, N)] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                double dt = delta[IDX3(b, t, d, L, D)], lm = lam[IDX3(b, t, d, L, D)], u = x[IDX3(b, t, d, L, D)];
                for (int64_t n = 0; n < N; ++n) {
                    double alpha = exp(dt * A[d * N + n]);
                    H[(t + 1) * N + n] = alpha * H[t * N + n] + (1.0 - lm) * dt * alpha * VPREV(t, n)
                                         + lm * dt * Bt[IDX3(b, t, n, L, N)] * u;
                }
            }
            double G[4096], Gb[4096];  /* G_t; beta_{t+1} G_{t+1} */
            for (int64_t n = 0; n < N; ++n) {
                G[n] = dstate ? dstate[IDX3(b, d, n, D, N)] : 0.0;
                Gb[n] = 0.0;
            }
            for (int64_t t = L - 1; t >= 0; --t) {
                int64_t r = IDX3(b, t, d, L, D);
                double dt = delta[r], lm = lam[r], u = x[r];
                double sum = 0.0;
                for (int64_t n = 0; n < N; ++n) sum += Ct[IDX3(b, t, n, L, N)] * H[(t + 1) * N + n];
                if (Dskip) sum += Dskip[d] * u;
                double gate = 1.0, dgate = 0.0;
                if (z) {
                    double zz = z[r], sg = 1.0 / (1.0 + exp(-zz));
                    gate = zz * sg;
                    dgate = sg * (1.0 + zz * (1.0 - sg));
                    dz[r] = dy[r] * sum * dgate;
                }
                double ds = dy[r] * gate;
                double gx = Dskip ? ds * Dskip[d] : 0.0;
                if (Dskip) dDskip[d] += ds * u;
                double gd = 0.0, gl = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    int64_t bn = IDX3(b, t, n, L, N);
                    G[n] += Ct[bn] * ds;
                    dCt[bn] += ds * H[(t + 1) * N + n];
                    double alpha = exp(dt * A[d * N + n]);
                    double v = Bt[bn] * u, vp = VPREV(t, n);
                    double p = H[t * N + n] + (1.0 - lm) * dt * vp;
                    double dv = lm * dt * G[n] + Gb[n];
                    gx += dv * Bt[bn];
                    dBt[bn] += dv * u;
                    gd += G[n] * (A[d * N + n] * alpha * p + (1.0 - lm) * alpha * vp + lm * v);
                    gl += G[n] * dt * (v - alpha * vp);
                    dA[d * N + n] += G[n] * dt * alpha * p;
                    Gb[n] = (1.0 - lm) * dt * alpha * G[n];
                    G[n] *= alpha;
                }
                ddelta[r] = gd;
                dlam[r] = gl;
                dx[r] = gx;
            }
            if (prev) {
                double gp = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    gp += Gb[n] * B_prev[b * N + n];
                    dB_prev[b * N + n] += Gb[n] * x_prev[b * D + d];
                }
                dx_prev[b * D + d] = gp;
            }
            for (int64_t n = 0; n < N; ++n) dstate_in[IDX3(b, d, n, D, N)] = G[n];
#undef VPREV
        }
    free(H);
    return 0;
}

/*
 * Gradient through the step-size activation: with u = raw[r, d] + bias[d] and
 * delta = softplus(u), d delta / d u = sigmoid(u) = 1 / (1 + exp(-u)), so for
 * the gradient g of delta (rows, D):
 *   graw[r, d] = g[r, d] * sigmoid(u)
 *   gbias[d]   = sum over r of graw[r, d]          (gbias may be NULL)
 * bias may be NULL (zero).
 */
int oracle_softplus_grad(int64_t rows, int64_t D, const double *raw, const double *bias, const double *g,
                         double *graw, double *gbias)
{
    if (rows < 0 || D < 0) return -1;
    if (gbias)
        for (int64_t d = 0; d < D; ++d) gbias[d] = 0.0;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t d = 0; d < D; ++d) {
            double u = raw[r * D + d] + (bias ? bias[d] : 0.0);
            double v = g[r * D + d] / (1.0 + exp(-u));
            graw[r * D + d] = v;
            if (gbias) gbias[d] += v;
        }
    return 0;
}

/*
 * One decode step: the loop body above with a single token, on a stored state
 * that is updated in place.
 *   x, delta, z, y : (batch, D)       z may be NULL
 *   A              : (D, N)
 *   Bt, Ct         : (batch, N)
 *   Dskip          : (D) or NULL
 *   state          : (batch, D, N)    read and overwritten
 */
int oracle_step(int64_t batch, int64_t D, int64_t N,
                const double *x, const double *delta, const double *A,
                const double *Bt, const double *Ct, const double *Dskip,
                const double *z, double *state, double *y, int nthreads)
{
    if (batch < 0 || D < 0 || N < 1) return -1;
    int64_t rows = batch * D;
    int nt = oracle_threads(nthreads);
    (void)nt;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / D, d = r % D;
        double dt = delta[r];
        double u = x[r];
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            double *hn = &state[r * N + n];
            double dA = exp(dt * A[d * N + n]);
            double dBx = dt * Bt[b * N + n] * u;
            *hn = dA * *hn + dBx;
            acc += Ct[b * N + n] * *hn;
        }
        if (Dskip) acc += Dskip[d] * u;
        if (z) {
            double g = z[r];
            acc *= g / (1.0 + exp(-g));
        }
        y[r] = acc;
    }
    return 0;
}

/*
 * Exponential-trapezoidal scan over L tokens. Per (b, d), with the input of
 * token t written v_t[n] = Bt[b,t,n] * x[b,t,d]:
 *
 *   alpha[n] = exp(delta_t * A[d,n])
 *   beta[n]  = (1 - lam_t) * delta_t * alpha[n]
 *   gamma    = lam_t * delta_t
 *   h[n]     = alpha[n] * h[n] + beta[n] * v_{t-1}[n] + gamma * v_t[n]
 *
 * with delta_t = delta[b,t,d] and lam_t = lam[b,t,d]. The input before token
 * 0 is v_{-1}[n] = B_prev[b,n] * x_prev[b,d] when both are given (the last
 * token of an earlier call on the same sequence), else 0. Readout, skip,
 * gate and the final state are those of oracle_scan.
 *   lam            : (batch, L, D)
 *   x_prev         : (batch, D) or NULL
 *   B_prev         : (batch, N) or NULL
 */
int oracle_scan_trap(int64_t batch, int64_t L, int64_t D, int64_t N,
                     const double *x, const double *delta, const double *lam, const double *A,
                     const double *Bt, const double *Ct, const double *Dskip,
                     const double *z, const double *x_prev, const double *B_prev,
                     const double *state_in, double *state_out, double *y, int nthreads)
{
    if (batch < 0 || L < 0 || D < 0 || N < 1 || N > 4096) return -1;
    int64_t rows = batch * D;
    int nt = oracle_threads(nthreads);
    (void)nt;
#pragma omp parallel for schedule(dynamic, 4) num_threads(nt)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / D, d = r % D;
        double h[4096], vprev[4096];
        for (int64_t n = 0; n < N; ++n) {
            h[n] = state_in ? state_in[IDX3(b, d, n, D, N)] : 0.0;
            vprev[n] = (x_prev && B_prev) ? B_prev[b * N + n] * x_prev[b * D + d] : 0.0;
        }
        for (int64_t t = 0; t < L; ++t) {
            double dt = delta[IDX3(b, t, d, L, D)];
            double lm = lam[IDX3(b, t, d, L, D)];
            double u = x[IDX3(b, t, d, L, D)];
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double alpha = exp(dt * A[d * N + n]);
                double beta = (1.0 - lm) * dt * alpha;
                double gamma = lm * dt;
                double v = Bt[IDX3(b, t, n, L, N)] * u;
                h[n] = alpha * h[n] + beta * vprev[n] + gamma * v;
                vprev[n] = v;
                acc += Ct[IDX3(b, t, n, L, N)] * h[n];
            }
            if (Dskip) acc += Dskip[d] * u;
            if (z) {
                double g = z[IDX3(b, t, d, L, D)];
                acc *= g / (1.0 + exp(-g));
            }
            y[IDX3(b, t, d, L, D)] = acc;
        }
        if (state_out)
            for (int64_t n = 0; n < N; ++n) state_out[IDX3(b, d, n, D, N)] = h[n];
    }
    return 0;
}

/*
 * One decode step of the exponential-trapezoidal scan on a stored state,
 * updated in place; x_prev (batch, D) and B_prev (batch, N) are the previous
 * token's x and Bt (NULL = none, as at the start of a sequence).
 */
int oracle_step_trap(int64_t batch, int64_t D, int64_t N,
                     const double *x, const double *delta, const double *lam, const double *A,
                     const double *Bt, const double *Ct, const double *Dskip,
                     const double *z, const double *x_prev, const double *B_prev,
                     double *state, double *y, int nthreads)
{
    if (batch < 0 || D < 0 || N < 1) return -1;
    int64_t rows = batch * D;
    int nt = oracle_threads(nthreads);
    (void)nt;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / D, d = r % D;
        double dt = delta[r], lm = lam[r];
        double u = x[r];
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            double *hn = &state[r * N + n];
            double alpha = exp(dt * A[d * N + n]);
            double beta = (1.0 - lm) * dt * alpha;
            double gamma = lm * dt;
            double vp = (x_prev && B_prev) ? B_prev[b * N + n] * x_prev[r] : 0.0;
            *hn = alpha * *hn + beta * vp + gamma * Bt[b * N + n] * u;
            acc += Ct[b * N + n] * *hn;
        }
        if (Dskip) acc += Dskip[d] * u;
        if (z) {
            double g = z[r];
            acc *= g / (1.0 + exp(-g));
        }
        y[r] = acc;
    }
    return 0;
}

/*
 * Mamba-2 SSD layer: per (batch row b, head h), with the scalar transition
 * a_t = exp(delta[b,t,h] * A[h]) and group g = h / (H / G) of Bt and Ct:
 *
 *   S[p][n] = state_in[b,h,p,n]  (or 0)
 *   for t = 0 .. L-1:
 *     S[p][n] = a_t * S[p][n] + delta[b,t,h] * x[b,t,h,p] * Bt[b,t,g,n]
 *     y[b,t,h,p] = sum_n Ct[b,t,g,n] * S[p][n]  (+ Dskip[h] * x[b,t,h,p])
 *   state_out[b,h,:,:] = S
 *
 *   x, y           : (batch, L, H, P)
 *   delta          : (batch, L, H)      step after its activation
 *   A              : (H)                one scalar per head
 *   Bt, Ct         : (batch, L, G, N)   G groups, each shared by H / G heads
 *   Dskip          : (H) or NULL
 *   state_in/_out  : (batch, H, P, N) or NULL
 * The input term is delta * B_t * x_t, the first-order rule of the S6 scan
 * this layer restricts. Returns 0, or -1 on a bad size.
 */
int oracle_ssd(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
               const double *x, const double *delta, const double *A, const double *Bt, const double *Ct,
               const double *Dskip, const double *state_in, double *state_out, double *y, int nthreads)
{
    if (batch < 0 || L < 0 || H < 1 || P < 1 || G < 1 || N < 1 || H % G != 0 || P * N > (1 << 20)) return -1;
    int64_t rows = batch * H;
    int nt = oracle_threads(nthreads);
    (void)nt;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / H, h = r % H, g = h / (H / G);
        double *S = (double *)malloc((size_t)(P * N) * sizeof(double));
        for (int64_t i = 0; i < P * N; ++i) S[i] = state_in ? state_in[r * P * N + i] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            double dt = delta[(b * L + t) * H + h];
            double a = exp(dt * A[h]);
            const double *xt = &x[((b * L + t) * H + h) * P];
            const double *Bg = &Bt[((b * L + t) * G + g) * N];
            const double *Cg = &Ct[((b * L + t) * G + g) * N];
            double *yt = &y[((b * L + t) * H + h) * P];
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    S[p * N + n] = a * S[p * N + n] + dt * xt[p] * Bg[n];
                    acc += Cg[n] * S[p * N + n];
                }
                if (Dskip) acc += Dskip[h] * xt[p];
                yt[p] = acc;
            }
        }
        if (state_out)
            for (int64_t i = 0; i < P * N; ++i) state_out[r * P * N + i] = S[i];
        free(S);
    }
    return 0;
}

/*
 * Gradient of oracle_scan (all gates and options as there) for the loss
 *   sum_{b,t,d} dy[b,t,d] * y[b,t,d]  +  sum_{b,d,n} dstate[b,d,n] * state_out[b,d,n]
 * (dstate may be NULL = 0). Writes the gradient with respect to every input:
 *   dx, ddelta, dz      : (batch, L, D)     (dz only when z is given)
 *   dA                  : (D, N)
 *   dBt, dCt            : (batch, L, N)
 *   dDskip              : (D)              (only when Dskip is given)
 *   dstate_in           : (batch, D, N)    (may be NULL)
 * Per (b, d), with a_t[n] = exp(delta_t A[n]), s_t = sum_n C_t[n] h_t[n] + D x_t,
 * g(z) = z sigmoid(z) and ds_t = dy_t g(z_t):
 *   forward:  h_t = a_t h_{t-1} + delta_t B_t x_t          (kept for every t)
 *   backward: G = dstate (or 0); for t = L-1 .. 0:
 *     G[n]    += C_t[n] ds_t                  (G is now dLoss/dh_t)
 *     dC_t[n] += ds_t h_t[n];  dD += ds_t x_t;  dx_t = ds_t D
 *     dz_t     = dy_t s_t g'(z_t)
 *     ddelta_t = sum_n G[n] (A[n] a_t[n] h_{t-1}[n] + B_t[n] x_t)
 *     dA[n]   += G[n] delta_t a_t[n] h_{t-1}[n]
 *     dB_t[n] += G[n] delta_t x_t;  dx_t += sum_n G[n] delta_t B_t[n]
 *     G[n]     = a_t[n] G[n]                  (dLoss/dh_{t-1} so far)
 *   dstate_in = G.
 * Single-threaded (dA, dB, dC and dD sum over rows). Returns 0, or -1 on a
 * bad size or when memory runs out.
 */
int oracle_scan_bwd(int64_t batch, int64_t L, int64_t D, int64_t N,
                    const double *x, const double *delta, const double *A,
                    const double *Bt, const double *Ct, const double *Dskip,
                    const double *z, const double *state_in, const double *dy, const double *dstate,
                    double *dx, double *ddelta, double *dA, double *dBt, double *dCt, double *dDskip,
                    double *dz, double *dstate_in)
{
    if (batch < 0 || L < 0 || D < 0 || N < 1 || N > 4096) return -1;
    double *H = (double *)malloc((size_t)((L + 1) * N) * sizeof(double));  /* H[(t + 1) N + n] = h_t */
    if (!H) return -1;
    for (int64_t i = 0; i < D * N; ++i) dA[i] = 0.0;
    for (int64_t i = 0; i < batch * L * N; ++i) dBt[i] = dCt[i] = 0.0;
    if (dDskip)
        for (int64_t d = 0; d < D; ++d) dDskip[d] = 0.0;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t d = 0; d < D; ++d) {
            for (int64_t n = 0; n < N; ++n) H[n] = state_in ? state_in[IDX3(b, d, n, D, N)] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                double dt = delta[IDX3(b, t, d, L, D)], u = x[IDX3(b, t, d, L, D)];
                for (int64_t n = 0; n < N; ++n)
                    H[(t + 1) * N + n] = exp(dt * A[d * N + n]) * H[t * N + n] + dt * Bt[IDX3(b, t, n, L, N)] * u;
            }
            double G[4096];
            for (int64_t n = 0; n < N; ++n) G[n] = dstate ? dstate[IDX3(b, d, n, D, N)] : 0.0;
            for (int64_t t = L - 1; t >= 0; --t) {
                int64_t r = IDX3(b, t, d, L, D);
                double dt = delta[r], u = x[r];
                double sum = 0.0;
                for (int64_t n = 0; n < N; ++n) sum += Ct[IDX3(b, t, n, L, N)] * H[(t + 1) * N + n];
                if (Dskip) sum += Dskip[d] * u;
                double gate = 1.0, dgate = 0.0;
                if (z) {
                    double zz = z[r], sg = 1.0 / (1.0 + exp(-zz));
                    gate = zz * sg;
                    dgate = sg * (1.0 + zz * (1.0 - sg));
                    dz[r] = dy[r] * sum * dgate;
                }
                double ds = dy[r] * gate;
                double gx = Dskip ? ds * Dskip[d] : 0.0;
                if (dDskip) dDskip[d] += ds * u;
                double gd = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    int64_t bn = IDX3(b, t, n, L, N);
                    G[n] += Ct[bn] * ds;
                    dCt[bn] += ds * H[(t + 1) * N + n];
                    double a = exp(dt * A[d * N + n]);
                    double hp = H[t * N + n];
                    gd += G[n] * (A[d * N + n] * a * hp + Bt[bn] * u);
                    dA[d * N + n] += G[n] * dt * a * hp;
                    dBt[bn] += G[n] * dt * u;
                    gx += G[n] * dt * Bt[bn];
                    G[n] *= a;
                }
                ddelta[r] = gd;
                dx[r] = gx;
            }
            if (dstate_in)
                for (int64_t n = 0; n < N; ++n) dstate_in[IDX3(b, d, n, D, N)] = G[n];
        }
    free(H);
    return 0;
}
