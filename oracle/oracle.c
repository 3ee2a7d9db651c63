/*
 * oracle.c - fp64 CPU oracle for the Mamba S6 selective scan, its decode update and backward, the
 * causal convolution, and the Mamba-2 (SSD) scan.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load this
 * file's library: only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it. It shares no code, header, table or helper with the HIP kernels.
 *
 * What it computes is the plain definition of the method, in the order the pages give it,
 * with no blocking, fusion or reordering:
 *
 *   step size      D_t   = softplus(delta_raw_t + bias)            (or the raw sum, flag off)
 *   discretise     Abar  = exp(D_t * a_n)                          (zero-order hold decay)
 *                  Bbar  = D_t * b_{t,n}                           (Euler input gain, default)
 *                       or (exp(D_t a_n) - 1) / a_n * b_{t,n}      (exact zero-order hold)
 *   recurrence     h_t   = Abar h_{t-1} + Bbar x_t,   h_{-1} = 0
 *   readout        y_t   = sum_n c_{t,n} h_{t,n}  +  D x_t
 *   gate           out_t = y_t * z_t * sigmoid(z_t)
 *
 * and, for Mamba-2 (a scalar decay per head, a state of P x N numbers per head):
 *
 *   SSD scan       H_t = exp(a_t) H_{t-1} + x_t b_t^T,   y_t = H_t c_t
 *
 * Sources (page titles and sections):
 *  - "Module 19: State-Space Models (Mamba)", sections "The Math: The State-Space Recurrence"
 *    (ZOH formulas, the Euler limit b -> Delta*B, the small-a fallback) and "Selectivity" /
 *    "Code: A Selective SSM (S6)" (Delta, B, C per token; A = -exp(A_log); softplus).
 *  - "Beyond attention with Mamba, state space models and hybrids", section 3 "Selectivity"
 *    (the selective recurrence h_t = exp(D_t a) h_{t-1} + D_t b_t x_t, y_t = c_t^T h_t),
 *    section 4 "The Mamba block" (Mixer.forward: softplus step, decay and write, scan_loop,
 *    skip u*D, gate by SiLU(z); the bias of dt_proj sits inside the softplus) and
 *    section 7 "Generation with a state of fixed size" (mixer_step: the one-token update) and
 *    section 8 "Mamba-2: the same model as attention" (the step-by-step loop of the SSD scan).
 *
 * Every tensor is read as fp64 (bf16 and fp32 inputs convert exactly), every result is fp64.
 * Rows (batch, channel) are independent; threads split the rows, so the result is bitwise
 * identical for any thread count. Built with gcc without fast-math and with contraction off.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

/* softplus(r) = log(1 + e^r). Written as max(r, 0) + log1p(e^{-|r|}): the same function, in a
 * form whose exp never overflows and whose log1p keeps full relative accuracy when e^r is tiny. */
double oracle_softplus(double r) {
    double pos = r > 0.0 ? r : 0.0;
    return pos + log1p(exp(-fabs(r)));
}

/* SiLU(z) = z * sigmoid(z) = z / (1 + e^{-z}). */
double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

/* Discretised input gain for one (token, state): Euler D*b, or the exact zero-order hold
 * (e^{D a} - 1)/a * b with the a = 0 limit D*b ("Module 19", The Math: the small-a fallback).
 * expm1 is the accurate evaluation of e^{D a} - 1. */
static double input_gain(double dt, double a, double b, int zoh) {
    if (!zoh || a == 0.0) return dt * b;
    return expm1(dt * a) / a * b;
}

typedef struct {
    const double *u, *delta, *A, *B, *C, *D, *z, *delta_bias;
    int softplus_flag, zoh_flag;
    int64_t nb, nd, L, N;
    double *out, *last_state;
    int64_t row_begin, row_end;
    int status;
} scan_job;

/* One (batch, channel) row at a time, t ascending, n ascending: the sequential loop. */
static void *scan_rows(void *arg) {
    scan_job *j = (scan_job *)arg;
    const int64_t nd = j->nd, L = j->L, N = j->N;
    double *h = (double *)malloc((size_t)N * sizeof(double));
    if (!h) { j->status = ORACLE_ENOMEM; return NULL; }
    for (int64_t row = j->row_begin; row < j->row_end; ++row) {
        const int64_t b = row / nd, d = row % nd;
        const double *u_row = j->u + row * L;
        const double *dr_row = j->delta + row * L;
        const double *z_row = j->z ? j->z + row * L : NULL;
        double *out_row = j->out + row * L;
        const double *a_row = j->A + d * N;
        const double bias = j->delta_bias ? j->delta_bias[d] : 0.0;
        const double skip = j->D ? j->D[d] : 0.0;
        for (int64_t n = 0; n < N; ++n) h[n] = 0.0; /* h_{-1} = 0 */
        for (int64_t t = 0; t < L; ++t) {
            const double r = dr_row[t] + bias;
            const double dt = j->softplus_flag ? oracle_softplus(r) : r;
            const double x = u_row[t];
            const double *b_tok = j->B + (b * L + t) * N;
            const double *c_tok = j->C + (b * L + t) * N;
            for (int64_t n = 0; n < N; ++n) {
                const double abar = exp(dt * a_row[n]);
                const double bbar = input_gain(dt, a_row[n], b_tok[n], j->zoh_flag);
                h[n] = abar * h[n] + bbar * x;
            }
            double y = 0.0;
            for (int64_t n = 0; n < N; ++n) y += c_tok[n] * h[n];
            if (j->D) y += skip * x;
            if (z_row) y *= oracle_silu(z_row[t]);
            out_row[t] = y;
        }
        if (j->last_state)
            for (int64_t n = 0; n < N; ++n) j->last_state[row * N + n] = h[n];
    }
    free(h);
    j->status = ORACLE_OK;
    return NULL;
}

static int resolve_threads(int nthreads, int64_t rows) {
    if (nthreads <= 0) {
        long c = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = c > 0 ? (int)c : 1;
    }
    if ((int64_t)nthreads > rows) nthreads = (int)(rows > 0 ? rows : 1);
    return nthreads;
}

/*
 * Selective scan over a whole sequence.
 *   u, delta, z, out : [nb, nd, L]   (L fastest)
 *   B, C             : [nb, L, N]
 *   A                : [nd, N]
 *   D, delta_bias    : [nd]
 *   last_state       : [nb, nd, N]
 * D, z, delta_bias and last_state may be NULL (no skip, no gate, zero bias, not written).
 * nthreads <= 0 uses every online core. Returns 0, or a negative code on bad arguments.
 */
int oracle_scan_fwd(const double *u, const double *delta, const double *A, const double *B,
                    const double *C, const double *D, const double *z, const double *delta_bias,
                    int softplus_flag, int zoh_flag, int64_t nb, int64_t nd, int64_t L, int64_t N,
                    double *out, double *last_state, int nthreads) {
    if (!u || !delta || !A || !B || !C || !out) return ORACLE_EINVAL;
    if (nb < 1 || nd < 1 || L < 1 || N < 1) return ORACLE_EINVAL;
    const int64_t rows = nb * nd;
    nthreads = resolve_threads(nthreads, rows);
    scan_job *jobs = (scan_job *)calloc((size_t)nthreads, sizeof(scan_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) { free(jobs); free(tids); return ORACLE_ENOMEM; }
    for (int i = 0; i < nthreads; ++i) {
        scan_job *j = &jobs[i];
        j->u = u; j->delta = delta; j->A = A; j->B = B; j->C = C; j->D = D; j->z = z;
        j->delta_bias = delta_bias; j->softplus_flag = softplus_flag; j->zoh_flag = zoh_flag;
        j->nb = nb; j->nd = nd; j->L = L; j->N = N; j->out = out; j->last_state = last_state;
        j->row_begin = rows * i / nthreads;
        j->row_end = rows * (i + 1) / nthreads;
        j->status = ORACLE_EINVAL;
    }
    int status = ORACLE_OK;
    if (nthreads == 1) {
        scan_rows(&jobs[0]);
    } else {
        int started = 0;
        for (int i = 0; i < nthreads; ++i, ++started)
            if (pthread_create(&tids[i], NULL, scan_rows, &jobs[i]) != 0) break;
        for (int i = started; i < nthreads; ++i) scan_rows(&jobs[i]); /* run what did not start */
        for (int i = 0; i < started; ++i) pthread_join(tids[i], NULL);
    }
    for (int i = 0; i < nthreads; ++i)
        if (jobs[i].status != ORACLE_OK) status = jobs[i].status;
    free(jobs);
    free(tids);
    return status;
}

/*
 * One decode step: the recurrence for a single token, with the state carried by the caller
 * ("Beyond attention with Mamba ...", section 7, mixer_step: step = softplus(.), then
 * h = exp(step a) h + step b u and y = (h c).sum + u D, gated by SiLU of the gate branch).
 *   state            : [nb, nd, N], read and updated in place
 *   x, delta, z, out : [nb, nd]
 *   B, C             : [nb, N]
 *   A                : [nd, N];  D : [nd]
 * The step size is always softplus(delta) with no bias. D and z may be NULL.
 */
int oracle_state_update(double *state, const double *x, const double *delta, const double *A,
                        const double *B, const double *C, const double *D, const double *z,
                        int zoh_flag, int64_t nb, int64_t nd, int64_t N, double *out) {
    if (!state || !x || !delta || !A || !B || !C || !out) return ORACLE_EINVAL;
    if (nb < 1 || nd < 1 || N < 1) return ORACLE_EINVAL;
    for (int64_t b = 0; b < nb; ++b) {
        for (int64_t d = 0; d < nd; ++d) {
            const int64_t row = b * nd + d;
            double *h = state + row * N;
            const double dt = oracle_softplus(delta[row]);
            const double xv = x[row];
            for (int64_t n = 0; n < N; ++n) {
                const double a = A[d * N + n];
                const double abar = exp(dt * a);
                const double bbar = input_gain(dt, a, B[b * N + n], zoh_flag);
                h[n] = abar * h[n] + bbar * xv;
            }
            double y = 0.0;
            for (int64_t n = 0; n < N; ++n) y += C[b * N + n] * h[n];
            if (D) y += D[d] * xv;
            if (z) y *= oracle_silu(z[row]);
            out[row] = y;
        }
    }
    return ORACLE_OK;
}

/*
 * Causal depthwise convolution of width K, then SiLU ("Module 19: State-Space Models (Mamba)",
 * "The Causal Convolution" and "The Math: Six Stages"; "Beyond attention with Mamba, state space
 * models and hybrids", section 4, the Mixer's conv1d with padding K-1 cropped to L):
 *   pre[b,d,t] = bias[d] + sum_{k=0}^{K-1} w[d,k] * x[b,d,t-(K-1)+k]     (x at t < 0 is 0)
 *   out[b,d,t] = silu_flag ? SiLU(pre) : pre
 * Each channel uses its own K taps; channels never mix; output t reads only x up to t.
 *   x, out : [nb, nd, L];  w : [nd, K];  bias : [nd] or NULL.
 */
int oracle_causal_conv1d(const double *x, const double *w, const double *bias, int silu_flag,
                         int64_t nb, int64_t nd, int64_t L, int64_t K, double *out) {
    if (!x || !w || !out) return ORACLE_EINVAL;
    if (nb < 1 || nd < 1 || L < 1 || K < 1) return ORACLE_EINVAL;
    for (int64_t b = 0; b < nb; ++b) {
        for (int64_t d = 0; d < nd; ++d) {
            const double *xr = x + (b * nd + d) * L;
            double *orow = out + (b * nd + d) * L;
            for (int64_t t = 0; t < L; ++t) {
                double pre = bias ? bias[d] : 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const int64_t s = t - (K - 1) + k;
                    if (s >= 0) pre += w[d * K + k] * xr[s];
                }
                orow[t] = silu_flag ? oracle_silu(pre) : pre;
            }
        }
    }
    return ORACLE_OK;
}

/*
 * One decode step of the convolution ("Beyond attention with Mamba, state space models and
 * hybrids", section 7, mixer_step): the window of the last K inputs shifts by one, the new input
 * enters at the end, and the output is the window's dot product with the taps plus the bias:
 *   window[b,d,:] <- (window[b,d,1:], x[b,d]);   out[b,d] = act(bias[d] + sum_k w[d,k] window[b,d,k])
 * Starting from a zero window, the steps reproduce oracle_causal_conv1d token by token.
 *   window : [nb, nd, K] (updated in place);  x, out : [nb, nd];  w : [nd, K];  bias : [nd] or NULL.
 */
int oracle_conv_window_update(double *window, const double *x, const double *w, const double *bias,
                              int silu_flag, int64_t nb, int64_t nd, int64_t K, double *out) {
    if (!window || !x || !w || !out) return ORACLE_EINVAL;
    if (nb < 1 || nd < 1 || K < 1) return ORACLE_EINVAL;
    for (int64_t b = 0; b < nb; ++b) {
        for (int64_t d = 0; d < nd; ++d) {
            double *win = window + (b * nd + d) * K;
            for (int64_t k = 0; k + 1 < K; ++k) win[k] = win[k + 1];
            win[K - 1] = x[b * nd + d];
            double pre = bias ? bias[d] : 0.0;
            for (int64_t k = 0; k < K; ++k) pre += w[d * K + k] * win[k];
            out[b * nd + d] = silu_flag ? oracle_silu(pre) : pre;
        }
    }
    return ORACLE_OK;
}

/*
 * Backward of oracle_scan_fwd (Euler input gain): given dout = dL/dout, the gradients of L with
 * respect to every input, by the adjoint of the recurrence run backwards in time. With
 * h_t = a_t h_{t-1} + Delta_t B_t u_t (a_t = exp(Delta_t A)), y_t = sum_n C_t h_t + D u_t,
 * out_t = y_t SiLU(z_t) and dy_t = dout_t SiLU(z_t), the adjoint of h_t is
 *   lambda_t = C_t dy_t + a_{t+1} lambda_{t+1}        (lambda after the last token is 0)
 * and each term of the forward pass contributes its partial derivative:
 *   dh_{t-1} via a_t:    dA += lambda_t h_{t-1} a_t Delta_t,  dDelta_t += lambda_t h_{t-1} a_t A
 *   write Delta B u:     dDelta_t += lambda_t B_t u_t,  dB_t += lambda_t Delta_t u_t,  du_t += lambda_t Delta_t B_t
 *   readout, skip, gate: dC_t += dy_t h_t,  dD += dy_t u_t,  du_t += D dy_t,  dz_t = dout_t y_t SiLU'(z_t)
 *   step:                ddelta_t = dDelta_t softplus'(r_t) (r_t = delta_t + bias; 1 without softplus),
 *                        dbias += ddelta_t
 * ("Beyond attention with Mamba, state space models and hybrids", section 6 notes that the fused
 * kernel recomputes the states for the backward pass rather than storing them; the oracle keeps
 * them, per row, for plainness.) dB and dC sum over the channels of a batch row, dA, dD and dbias
 * over batch rows and tokens. Gradients of absent optional inputs (NULL) are not written.
 *   du, ddelta, dz : [nb, nd, L];  dA : [nd, N];  dB, dC : [nb, L, N];  dD, ddelta_bias : [nd].
 */
int oracle_scan_bwd(const double *u, const double *delta, const double *A, const double *B,
                    const double *C, const double *D, const double *z, const double *delta_bias,
                    int softplus_flag, const double *dout, int64_t nb, int64_t nd, int64_t L, int64_t N,
                    double *du, double *ddelta, double *dA, double *dB, double *dC, double *dD,
                    double *dz, double *ddelta_bias) {
    if (!u || !delta || !A || !B || !C || !dout || !du || !ddelta || !dA || !dB || !dC) return ORACLE_EINVAL;
    if (nb < 1 || nd < 1 || L < 1 || N < 1) return ORACLE_EINVAL;
    double *h = (double *)malloc((size_t)(L * N) * sizeof(double));
    double *lam = (double *)malloc((size_t)N * sizeof(double));
    if (!h || !lam) {
        free(h);
        free(lam);
        return ORACLE_ENOMEM;
    }
    memset(dA, 0, (size_t)(nd * N) * sizeof(double));
    memset(dB, 0, (size_t)(nb * L * N) * sizeof(double));
    memset(dC, 0, (size_t)(nb * L * N) * sizeof(double));
    if (dD) memset(dD, 0, (size_t)nd * sizeof(double));
    if (ddelta_bias) memset(ddelta_bias, 0, (size_t)nd * sizeof(double));
    for (int64_t b = 0; b < nb; ++b) {
        for (int64_t d = 0; d < nd; ++d) {
            const int64_t row = (b * nd + d) * L;
            const double bias = delta_bias ? delta_bias[d] : 0.0;
            const double *a_row = A + d * N;
            /* forward, keeping every state of the row */
            for (int64_t t = 0; t < L; ++t) {
                const double r = delta[row + t] + bias;
                const double dt = softplus_flag ? oracle_softplus(r) : r;
                const double *bt = B + (b * L + t) * N;
                for (int64_t n = 0; n < N; ++n) {
                    const double prev = t > 0 ? h[(t - 1) * N + n] : 0.0;
                    h[t * N + n] = exp(a_row[n] * dt) * prev + dt * bt[n] * u[row + t];
                }
            }
            /* backward */
            for (int64_t n = 0; n < N; ++n) lam[n] = 0.0;  /* holds a_{t+1} lambda_{t+1} */
            for (int64_t t = L - 1; t >= 0; --t) {
                const double r = delta[row + t] + bias;
                const double dt = softplus_flag ? oracle_softplus(r) : r;
                const double *bt = B + (b * L + t) * N;
                const double *ct = C + (b * L + t) * N;
                const double ut = u[row + t];
                double y = 0.0;
                for (int64_t n = 0; n < N; ++n) y += ct[n] * h[t * N + n];
                if (D) y += D[d] * ut;
                const double g = z ? oracle_silu(z[row + t]) : 1.0;
                const double dy = dout[row + t] * g;
                if (dz) {
                    const double zt = z[row + t];
                    const double sg = 1.0 / (1.0 + exp(-zt));
                    dz[row + t] = dout[row + t] * y * sg * (1.0 + zt * (1.0 - sg));
                }
                double du_t = D ? D[d] * dy : 0.0;
                if (dD) dD[d] += dy * ut;
                double ddt = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double l = lam[n] + ct[n] * dy;
                    const double a = exp(a_row[n] * dt);
                    const double hp = t > 0 ? h[(t - 1) * N + n] : 0.0;
                    dC[(b * L + t) * N + n] += dy * h[t * N + n];
                    ddt += l * (hp * a * a_row[n] + bt[n] * ut);
                    du_t += l * dt * bt[n];
                    dA[d * N + n] += l * hp * a * dt;
                    dB[(b * L + t) * N + n] += l * dt * ut;
                    lam[n] = a * l;
                }
                du[row + t] = du_t;
                const double dr = softplus_flag ? ddt / (1.0 + exp(-r)) : ddt;
                ddelta[row + t] = dr;
                if (ddelta_bias) ddelta_bias[d] += dr;
            }
        }
    }
    free(h);
    free(lam);
    return ORACLE_OK;
}

/*
 * Mamba-2's scan with a scalar decay per head ("Beyond attention with Mamba, state space models and
 * hybrids", section 8, Mamba-2: the same model as attention; its step-by-step loop, the definition
 * the chunked form is checked against). For every batch row b and head h, with a state H of P x N
 * numbers that starts at zero, token by token:
 *   H <- exp(a[b,t,h]) H + x[b,t,h,:] b[b,t,g,:]^T        (an outer product; g = h / (heads / groups))
 *   y[b,t,h,p] = sum_n H[p,n] c[b,t,g,n]                  (n ascending)
 * x: [nb, L, heads, P], the stream already multiplied by its step; a: [nb, L, heads], the step times
 * the head's A; b, c: [nb, L, groups, N], each group shared by heads / groups consecutive heads;
 * y: [nb, L, heads, P]; final_state: [nb, heads, P, N], the state after the last token, or NULL.
 */
typedef struct {
    const double *x, *a, *b, *c;
    int64_t nb, L, heads, P, N, groups;
    double *y, *final_state;
    int64_t row_begin, row_end;
    int status;
} ssd_job;

static void *ssd_rows(void *arg) {
    ssd_job *j = (ssd_job *)arg;
    const int64_t L = j->L, H = j->heads, P = j->P, N = j->N, G = j->groups;
    double *st = (double *)calloc((size_t)(P * N), sizeof(double));
    if (!st) {
        j->status = ORACLE_ENOMEM;
        return NULL;
    }
    for (int64_t row = j->row_begin; row < j->row_end; ++row) {
        const int64_t b = row / H, h = row % H, g = h / (H / G);
        memset(st, 0, (size_t)(P * N) * sizeof(double));
        for (int64_t t = 0; t < L; ++t) {
            const double decay = exp(j->a[(b * L + t) * H + h]);
            const double *xt = j->x + ((b * L + t) * H + h) * P;
            const double *bt = j->b + ((b * L + t) * G + g) * N;
            const double *ct = j->c + ((b * L + t) * G + g) * N;
            double *yt = j->y + ((b * L + t) * H + h) * P;
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    st[p * N + n] = decay * st[p * N + n] + xt[p] * bt[n];
                    acc += st[p * N + n] * ct[n];
                }
                yt[p] = acc;
            }
        }
        if (j->final_state) memcpy(j->final_state + (b * H + h) * P * N, st, (size_t)(P * N) * sizeof(double));
    }
    free(st);
    j->status = ORACLE_OK;
    return NULL;
}

int oracle_ssd_scan(const double *x, const double *a, const double *b, const double *c, int64_t nb, int64_t L,
                    int64_t heads, int64_t P, int64_t N, int64_t groups, double *y, double *final_state,
                    int nthreads) {
    if (!x || !a || !b || !c || !y) return ORACLE_EINVAL;
    if (nb < 1 || L < 1 || heads < 1 || P < 1 || N < 1 || groups < 1 || heads % groups != 0) return ORACLE_EINVAL;
    const int64_t rows = nb * heads;
    nthreads = resolve_threads(nthreads, rows);
    ssd_job *jobs = (ssd_job *)calloc((size_t)nthreads, sizeof(ssd_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) { free(jobs); free(tids); return ORACLE_ENOMEM; }
    for (int i = 0; i < nthreads; ++i) {
        ssd_job *j = &jobs[i];
        j->x = x; j->a = a; j->b = b; j->c = c;
        j->nb = nb; j->L = L; j->heads = heads; j->P = P; j->N = N; j->groups = groups;
        j->y = y; j->final_state = final_state;
        j->row_begin = rows * i / nthreads;
        j->row_end = rows * (i + 1) / nthreads;
        j->status = ORACLE_EINVAL;
    }
    int status = ORACLE_OK;
    if (nthreads == 1) {
        ssd_rows(&jobs[0]);
    } else {
        int started = 0;
        for (int i = 0; i < nthreads; ++i, ++started)
            if (pthread_create(&tids[i], NULL, ssd_rows, &jobs[i]) != 0) break;
        for (int i = started; i < nthreads; ++i) ssd_rows(&jobs[i]);
        for (int i = 0; i < started; ++i) pthread_join(tids[i], NULL);
    }
    for (int i = 0; i < nthreads; ++i)
        if (jobs[i].status != ORACLE_OK) status = jobs[i].status;
    free(jobs);
    free(tids);
    return status;
}

int oracle_abi_version(void) { return 3; }
