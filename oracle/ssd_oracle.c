/*
 * Float64 token-by-token oracle for the chunked SSD scan (and, at the end of
 * this file, for the Mamba-1 selective scan and the Mamba-3 trapezoid).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the bench's CPU
 * baseline leg do. It shares no code with the HIP path.
 *
 * What it computes (for every batch b and head h, group g = h / (H/G)):
 *
 *   S = init_state[b,h]  (P x N, or zero)
 *   for t = 0 .. T-1:
 *     if theta: every N-axis pair (2k, 2k+1) of S is turned by the plane
 *               rotation R(theta[b,t,h,k]) = [[cos, -sin], [sin, cos]]
 *     S = exp(da[b,t,h]) * S + sum_r x[b,t,r,h,:] (outer) B[b,t,r,g,:]
 *     y[b,t,r,h,p] = sum_n C[b,t,r,g,n] * S[p,n] + D[h] * x[b,t,r,h,p]
 *   final_state[b,h] = S
 *
 * Sources (cited by page title and section):
 *  - "SSM Selective Scan" (LeetGPU challenge write-up), problem statement:
 *    the selective-scan recurrence h_t = Abar_t h_{t-1} + Bbar_t u_t,
 *    y_t = C_t . h_t + skip * u_t, with a zero starting state. Here the decay
 *    is one scalar per head (Mamba-2), Abar = exp(da), and x already carries
 *    the input scaling (dt enters only through da).
 *  - burn-mamba "mamba3/ssd/serial.rs", ssd_serial and k1..k5: the multi-rank
 *    (MIMO) form. The R writes of one step are summed into the state under a
 *    single decay, and every rank's read at step t sees all R writes of step t
 *    (the K5 mask keeps the full R x R diagonal block).
 *  - "mamba3/scan.py", module docstring ("THE TRICK"): the rotated recurrence
 *    h_t = alpha_t R(theta_t) h_{t-1} + S_t (trapezoid weights beta=0,
 *    gamma=1); rotate_by gives the pair convention (even = c*a - s*b,
 *    odd = s*a + c*b). final_state is the physical state h_{T-1}.
 *
 * Inputs x, B, C are read at their stored precision (fp32, or bf16 decoded
 * exactly; the tests may also hand in float64); da, D, theta, init_state are
 * fp32. All arithmetic is double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_IN_F32 0
#define ORACLE_IN_BF16 1
#define ORACLE_IN_F64 2

typedef struct {
    int64_t batch, T, H, P, N, G, R;
    int in_dtype;
    const void *x, *B, *C;
    const float *da, *D, *init_state, *theta;
} oracle_problem;

/* Exact widening of one stored input element to double. */
static double load_elem(const void *base, int64_t i, int dtype) {
    if (dtype == ORACLE_IN_F32) return (double)((const float *)base)[i];
    if (dtype == ORACLE_IN_F64) return ((const double *)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* One (b, h) slice: y_out is [T][R][P], fin_out is [P][N], S is P*N scratch. */
static void run_slice(const oracle_problem *pr, int64_t b, int64_t h,
                      double *y_out, double *fin_out, double *S) {
    const int64_t T = pr->T, H = pr->H, P = pr->P, N = pr->N, G = pr->G, R = pr->R;
    const int64_t g = h / (H / G);

    if (pr->init_state) {
        const float *h0 = pr->init_state + (b * H + h) * P * N;
        for (int64_t i = 0; i < P * N; ++i) S[i] = (double)h0[i];
    } else {
        memset(S, 0, sizeof(double) * (size_t)(P * N));
    }

    for (int64_t t = 0; t < T; ++t) {
        /* rotation of the carried state, pair (2k, 2k+1) by theta[b,t,h,k] */
        if (pr->theta) {
            const float *th = pr->theta + ((b * T + t) * H + h) * (N / 2);
            for (int64_t k = 0; k < N / 2; ++k) {
                double c = cos((double)th[k]), s = sin((double)th[k]);
                for (int64_t p = 0; p < P; ++p) {
                    double a0 = S[p * N + 2 * k], a1 = S[p * N + 2 * k + 1];
                    S[p * N + 2 * k] = c * a0 - s * a1;
                    S[p * N + 2 * k + 1] = s * a0 + c * a1;
                }
            }
        }
        /* decay, then the R rank-one writes of step t */
        double a = exp((double)pr->da[(b * T + t) * H + h]);
        for (int64_t i = 0; i < P * N; ++i) S[i] *= a;
        for (int64_t r = 0; r < R; ++r) {
            int64_t xrow = (((b * T + t) * R + r) * H + h) * P;
            int64_t brow = (((b * T + t) * R + r) * G + g) * N;
            for (int64_t p = 0; p < P; ++p) {
                double xv = load_elem(pr->x, xrow + p, pr->in_dtype);
                for (int64_t n = 0; n < N; ++n)
                    S[p * N + n] += xv * load_elem(pr->B, brow + n, pr->in_dtype);
            }
        }
        /* every rank reads the state after all writes of step t */
        for (int64_t r = 0; r < R; ++r) {
            int64_t xrow = (((b * T + t) * R + r) * H + h) * P;
            int64_t crow = (((b * T + t) * R + r) * G + g) * N;
            double dh = pr->D ? (double)pr->D[h] : 0.0;
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n)
                    acc += load_elem(pr->C, crow + n, pr->in_dtype) * S[p * N + n];
                acc += dh * load_elem(pr->x, xrow + p, pr->in_dtype);
                y_out[(t * R + r) * P + p] = acc;
            }
        }
    }
    memcpy(fin_out, S, sizeof(double) * (size_t)(P * N));
}

/*
 * Runs the recurrence on the selected (b, h) slices.
 *   bh_list: n_bh indices bh = b*H + h (NULL: every slice, in bh order).
 *   y_sel:   [n_bh][T][R][P] doubles (may be NULL to skip y).
 *   fin_sel: [n_bh][P][N] doubles.
 *   nthreads <= 0 uses the OpenMP default.
 * Returns 0, or a negative code for a bad argument.
 */
int ssd_oracle_f64(int64_t batch, int64_t T, int64_t H, int64_t P, int64_t N,
                   int64_t G, int64_t R, int in_dtype,
                   const void *x, const float *da, const void *B, const void *C,
                   const float *D, const float *init_state, const float *theta,
                   const int64_t *bh_list, int64_t n_bh,
                   double *y_sel, double *fin_sel, int nthreads) {
    if (batch < 1 || T < 1 || H < 1 || P < 1 || N < 1 || G < 1 || R < 1) return -1;
    if (H % G != 0) return -2;
    if (theta && (N % 2)) return -3;
    if (in_dtype != ORACLE_IN_F32 && in_dtype != ORACLE_IN_BF16 && in_dtype != ORACLE_IN_F64)
        return -4;
    if (!x || !da || !B || !C || !fin_sel) return -5;
    if (!bh_list) n_bh = batch * H;
    for (int64_t i = 0; bh_list && i < n_bh; ++i)
        if (bh_list[i] < 0 || bh_list[i] >= batch * H) return -6;

    oracle_problem pr = {batch, T, H, P, N, G, R, in_dtype, x, B, C, da, D, init_state, theta};
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)(P * N));
        double *ytmp = y_sel ? NULL : (double *)malloc(sizeof(double) * (size_t)(T * R * P));
        int ok = S && (y_sel || ytmp);
        if (!ok) {
#pragma omp atomic write
            err = -7;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_bh; ++i) {
            if (!ok) continue;
            int64_t bh = bh_list ? bh_list[i] : i;
            double *yo = y_sel ? y_sel + i * T * R * P : ytmp;
            run_slice(&pr, bh / H, bh % H, yo, fin_sel + i * P * N, S);
        }
        free(S);
        free(ytmp);
    }
    return err;
}

/* Number of threads an OpenMP parallel region would use (for reporting). */
int ssd_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Mamba-1 selective scan with a per-(channel, state) decay, as the "SSM
 * Selective Scan" page states it (problem statement): for every batch b,
 * channel d and state index n, from a zero state,
 *
 *   Abar = exp(delta[b,t,d] * A[d,n]),   Bbar = delta[b,t,d] * B[b,t,n]
 *   h[n] = Abar * h[n] + Bbar * u[b,t,d]
 *   y[b,t,d] = sum_n C[b,t,n] * h[n] + skip[d] * u[b,t,d]
 *
 * Channels share B and C and have their own rows of A. Inputs are fp32,
 * widened to double; y is double.
 *   y:       [batch][T][Dm] doubles, or the selected channels only:
 *   bd_list: n_bd indices bd = b*Dm + d (NULL: every channel, y in [b][T][Dm]);
 *            with a list, y is [n_bd][T].
 * Returns 0, or a negative code for a bad argument.
 */
int selective_scan_f64(int64_t batch, int64_t T, int64_t Dm, int64_t N,
                       const float *u, const float *delta, const float *A, const float *B,
                       const float *C, const float *skip, const int64_t *bd_list, int64_t n_bd,
                       double *y, int nthreads) {
    if (batch < 1 || T < 1 || Dm < 1 || N < 1) return -1;
    if (!u || !delta || !A || !B || !C || !skip || !y) return -5;
    if (!bd_list) n_bd = batch * Dm;
    for (int64_t i = 0; bd_list && i < n_bd; ++i)
        if (bd_list[i] < 0 || bd_list[i] >= batch * Dm) return -6;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *h = (double *)malloc(sizeof(double) * (size_t)N);
        if (!h) {
#pragma omp atomic write
            err = -7;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_bd; ++i) {
            if (!h) continue;
            const int64_t bd = bd_list ? bd_list[i] : i;
            const int64_t b = bd / Dm, d = bd % Dm;
            for (int64_t n = 0; n < N; ++n) h[n] = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const int64_t row = b * T + t;
                const double dl = (double)delta[row * Dm + d], ut = (double)u[row * Dm + d];
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double abar = exp(dl * (double)A[d * N + n]);
                    const double bbar = dl * (double)B[row * N + n];
                    h[n] = abar * h[n] + bbar * ut;
                    acc += (double)C[row * N + n] * h[n];
                }
                acc += (double)skip[d] * ut;
                if (bd_list)
                    y[i * T + t] = acc;
                else
                    y[row * Dm + d] = acc;
            }
        }
        free(h);
    }
    return err;
}

/*
 * Mamba-3 trapezoid (two-write) recurrence in the physical frame, for every
 * batch b and head h (group g = h / (H/G)):
 *
 *   W_t  = sum_r x[b,t,r,h,:] (outer) B[b,t,r,g,:]            (P x N)
 *   W_-1 = sum_r prev_x[b,r,h,:] (outer) prev_B[b,r,g,:]       (zero if absent)
 *   h_t  = R(theta[b,t,h]) (exp(da[b,t,h]) h_{t-1} + beta[b,t,h] W_{t-1})
 *          + gamma[b,t,h] W_t
 *   y[b,t,r,h,p] = sum_n C[b,t,r,g,n] h_t[p,n]
 *   h_-1 = init_state[b,h] (or zero); final_state[b,h] = h_{T-1}
 *
 * Sources (cited by page title and section):
 *  - "mamba3/scan.py", module docstring: h_t = alpha_t R(theta_t) h_{t-1}
 *    + beta_t S_{t-1} + gamma_t S_t; and scan_forward, whose comment (citing
 *    the Mamba-3 paper's eq. 11) turns the beta write by the previous step's
 *    cumulative angle. In the physical frame that makes the beta write part
 *    of what step t rotates, as written above. The docstring's literal form
 *    (beta write not rotated at step t) is the other reading; this file
 *    follows the code and eq. 11.
 *  - burn-mamba "mamba3/moments.rs", module documentation and
 *    build_moments_input: the beta stream is the previous token's x and
 *    rotated B scaled by the current beta; its first element comes from the
 *    cache's previous-token entries (prev_x, prev_B here); the initial state
 *    enters once.
 * No skip term (the Mamba-3 scan has none). x, B, C, prev_x, prev_B at their
 * stored precision; the rest fp32; double arithmetic.
 */
static void run_trap_slice(const oracle_problem *pr, const float *beta, const float *gamma,
                           const void *prev_x, const void *prev_B, int64_t b, int64_t h,
                           double *y_out, double *fin_out, double *S, double *Wp, double *Wc) {
    const int64_t T = pr->T, H = pr->H, P = pr->P, N = pr->N, G = pr->G, R = pr->R;
    const int64_t g = h / (H / G);

    if (pr->init_state) {
        const float *h0 = pr->init_state + (b * H + h) * P * N;
        for (int64_t i = 0; i < P * N; ++i) S[i] = (double)h0[i];
    } else {
        memset(S, 0, sizeof(double) * (size_t)(P * N));
    }
    memset(Wp, 0, sizeof(double) * (size_t)(P * N));
    if (prev_x && prev_B) {
        for (int64_t r = 0; r < R; ++r) {
            int64_t xrow = ((b * R + r) * H + h) * P, brow = ((b * R + r) * G + g) * N;
            for (int64_t p = 0; p < P; ++p) {
                double xv = load_elem(prev_x, xrow + p, pr->in_dtype);
                for (int64_t n = 0; n < N; ++n)
                    Wp[p * N + n] += xv * load_elem(prev_B, brow + n, pr->in_dtype);
            }
        }
    }
    for (int64_t t = 0; t < T; ++t) {
        const int64_t sh = (b * T + t) * H + h;
        /* this step's write W_t */
        memset(Wc, 0, sizeof(double) * (size_t)(P * N));
        for (int64_t r = 0; r < R; ++r) {
            int64_t xrow = (((b * T + t) * R + r) * H + h) * P;
            int64_t brow = (((b * T + t) * R + r) * G + g) * N;
            for (int64_t p = 0; p < P; ++p) {
                double xv = load_elem(pr->x, xrow + p, pr->in_dtype);
                for (int64_t n = 0; n < N; ++n)
                    Wc[p * N + n] += xv * load_elem(pr->B, brow + n, pr->in_dtype);
            }
        }
        /* decayed state plus the previous step's write, then the rotation */
        const double a = exp((double)pr->da[sh]), be = (double)beta[sh], ga = (double)gamma[sh];
        for (int64_t i = 0; i < P * N; ++i) S[i] = a * S[i] + be * Wp[i];
        if (pr->theta) {
            const float *th = pr->theta + sh * (N / 2);
            for (int64_t k = 0; k < N / 2; ++k) {
                const double cs = cos((double)th[k]), sn = sin((double)th[k]);
                for (int64_t p = 0; p < P; ++p) {
                    double *pair = S + p * N + 2 * k;
                    const double ev = pair[0], od = pair[1];
                    pair[0] = cs * ev - sn * od;
                    pair[1] = sn * ev + cs * od;
                }
            }
        }
        for (int64_t i = 0; i < P * N; ++i) S[i] += ga * Wc[i];
        /* every rank reads the state after both writes of step t */
        for (int64_t r = 0; r < R; ++r) {
            int64_t crow = (((b * T + t) * R + r) * G + g) * N;
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n)
                    acc += load_elem(pr->C, crow + n, pr->in_dtype) * S[p * N + n];
                y_out[(t * R + r) * P + p] = acc;
            }
        }
        memcpy(Wp, Wc, sizeof(double) * (size_t)(P * N));
    }
    memcpy(fin_out, S, sizeof(double) * (size_t)(P * N));
}

/*
 * Runs the trapezoid recurrence on the selected (b, h) slices; arguments as
 * ssd_oracle_f64 (no D), plus beta, gamma [b,T,H] fp32 and the optional
 * previous-token entries prev_x [b,R,H,P], prev_B [b,R,G,N] (both or neither).
 */
int trapezoid_f64(int64_t batch, int64_t T, int64_t H, int64_t P, int64_t N,
                  int64_t G, int64_t R, int in_dtype,
                  const void *x, const float *da, const void *B, const void *C,
                  const float *beta, const float *gamma, const void *prev_x, const void *prev_B,
                  const float *init_state, const float *theta,
                  const int64_t *bh_list, int64_t n_bh,
                  double *y_sel, double *fin_sel, int nthreads) {
    if (batch < 1 || T < 1 || H < 1 || P < 1 || N < 1 || G < 1 || R < 1) return -1;
    if (H % G != 0) return -2;
    if (theta && (N % 2)) return -3;
    if (in_dtype != ORACLE_IN_F32 && in_dtype != ORACLE_IN_BF16 && in_dtype != ORACLE_IN_F64)
        return -4;
    if (!x || !da || !B || !C || !beta || !gamma || !fin_sel || !y_sel) return -5;
    if ((prev_x == NULL) != (prev_B == NULL)) return -5;
    if (!bh_list) n_bh = batch * H;
    for (int64_t i = 0; bh_list && i < n_bh; ++i)
        if (bh_list[i] < 0 || bh_list[i] >= batch * H) return -6;

    oracle_problem pr = {batch, T, H, P, N, G, R, in_dtype, x, B, C, da, NULL, init_state, theta};
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *buf = (double *)malloc(sizeof(double) * (size_t)(3 * P * N));
        if (!buf) {
#pragma omp atomic write
            err = -7;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_bh; ++i) {
            if (!buf) continue;
            int64_t bh = bh_list ? bh_list[i] : i;
            run_trap_slice(&pr, beta, gamma, prev_x, prev_B, bh / H, bh % H,
                           y_sel + i * T * R * P, fin_sel + i * P * N, buf, buf + P * N, buf + 2 * P * N);
        }
        free(buf);
    }
    return err;
}

/*
 * Physical-frame state moments, burn-mamba "mamba3/moments.rs": module
 * documentation (the per-token physical state c_t, steps 1-4: states,
 * de-rotation to the physical frame, plain real m2/m1 sums masked to
 * valid_len) and state_moments_phys (raw sums, count = valid_len * P).
 * For every (b, h), with h_t the physical state after step t of the
 * trapezoid recurrence of trapezoid_f64 (or, when beta and gamma are NULL,
 * of the single-write recurrence: beta = 0, gamma = 1, no previous token):
 *
 *   m2[b,h][n][n'] = sum_{t < valid_len} sum_p h_t[p][n] h_t[p][n']
 *   m1[b,h][n]     = sum_{t < valid_len} sum_p h_t[p][n]
 *
 * The moments see the states only; y and C play no part. Tokens at
 * t >= valid_len still step the state but are not counted.
 *   m2_sel: [n_bh][N][N], m1_sel: [n_bh][N] doubles.
 */
static void run_moments_slice(const oracle_problem *pr, const float *beta, const float *gamma,
                              const void *prev_x, const void *prev_B, int64_t valid_len,
                              int64_t b, int64_t h, double *m2, double *m1,
                              double *st, double *wlast, double *wnow) {
    const int64_t T = pr->T, H = pr->H, P = pr->P, N = pr->N, G = pr->G, R = pr->R;
    const int64_t g = h / (H / G);
    const int64_t PN = P * N;

    for (int64_t i = 0; i < PN; ++i)
        st[i] = pr->init_state ? (double)pr->init_state[(b * H + h) * PN + i] : 0.0;
    for (int64_t i = 0; i < PN; ++i) wlast[i] = 0.0;
    if (beta && prev_x && prev_B) {
        for (int64_t r = 0; r < R; ++r)
            for (int64_t p = 0; p < P; ++p) {
                const double xe = load_elem(prev_x, ((b * R + r) * H + h) * P + p, pr->in_dtype);
                for (int64_t n = 0; n < N; ++n)
                    wlast[p * N + n] += xe * load_elem(prev_B, ((b * R + r) * G + g) * N + n, pr->in_dtype);
            }
    }
    for (int64_t i = 0; i < N * N; ++i) m2[i] = 0.0;
    for (int64_t n = 0; n < N; ++n) m1[n] = 0.0;

    for (int64_t t = 0; t < T; ++t) {
        const int64_t row = (b * T + t) * H + h;
        /* this step's rank-R write */
        for (int64_t i = 0; i < PN; ++i) wnow[i] = 0.0;
        for (int64_t r = 0; r < R; ++r)
            for (int64_t p = 0; p < P; ++p) {
                const double xe = load_elem(pr->x, (((b * T + t) * R + r) * H + h) * P + p, pr->in_dtype);
                for (int64_t n = 0; n < N; ++n)
                    wnow[p * N + n] += xe * load_elem(pr->B, (((b * T + t) * R + r) * G + g) * N + n, pr->in_dtype);
            }
        const double dec = exp((double)pr->da[row]);
        const double wb = beta ? (double)beta[row] : 0.0, wg = gamma ? (double)gamma[row] : 1.0;
        /* decay and the previous step's write, the turn of step t, this step's write */
        for (int64_t i = 0; i < PN; ++i) st[i] = dec * st[i] + wb * wlast[i];
        if (pr->theta) {
            for (int64_t k = 0; k < N / 2; ++k) {
                const double ang = (double)pr->theta[row * (N / 2) + k];
                const double co = cos(ang), si = sin(ang);
                for (int64_t p = 0; p < P; ++p) {
                    const double e0 = st[p * N + 2 * k], e1 = st[p * N + 2 * k + 1];
                    st[p * N + 2 * k] = co * e0 - si * e1;
                    st[p * N + 2 * k + 1] = si * e0 + co * e1;
                }
            }
        }
        for (int64_t i = 0; i < PN; ++i) st[i] += wg * wnow[i];
        for (int64_t i = 0; i < PN; ++i) wlast[i] = wnow[i];
        /* the sums, over the tokens inside valid_len */
        if (t < valid_len) {
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n) {
                    const double hv = st[p * N + n];
                    m1[n] += hv;
                    for (int64_t n2 = 0; n2 < N; ++n2) m2[n * N + n2] += hv * st[p * N + n2];
                }
        }
    }
}

/*
 * Runs the moments on the selected (b, h) slices; arguments as
 * trapezoid_f64 without C and y (beta and gamma both NULL for the
 * single-write recurrence, when prev_x and prev_B are ignored), plus
 * valid_len in 1..T.
 */
int state_moments_f64(int64_t batch, int64_t T, int64_t H, int64_t P, int64_t N,
                      int64_t G, int64_t R, int in_dtype,
                      const void *x, const float *da, const void *B,
                      const float *beta, const float *gamma, const void *prev_x, const void *prev_B,
                      const float *init_state, const float *theta, int64_t valid_len,
                      const int64_t *bh_list, int64_t n_bh,
                      double *m2_sel, double *m1_sel, int nthreads) {
    if (batch < 1 || T < 1 || H < 1 || P < 1 || N < 1 || G < 1 || R < 1) return -1;
    if (H % G != 0) return -2;
    if (theta && (N % 2)) return -3;
    if (in_dtype != ORACLE_IN_F32 && in_dtype != ORACLE_IN_BF16 && in_dtype != ORACLE_IN_F64)
        return -4;
    if (!x || !da || !B || !m2_sel || !m1_sel) return -5;
    if ((beta == NULL) != (gamma == NULL) || (prev_x == NULL) != (prev_B == NULL)) return -5;
    if (valid_len < 1 || valid_len > T) return -8;
    if (!bh_list) n_bh = batch * H;
    for (int64_t i = 0; bh_list && i < n_bh; ++i)
        if (bh_list[i] < 0 || bh_list[i] >= batch * H) return -6;

    oracle_problem pr = {batch, T, H, P, N, G, R, in_dtype, x, B, NULL, da, NULL, init_state, theta};
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *work = (double *)malloc(sizeof(double) * (size_t)(3 * P * N));
        if (!work) {
#pragma omp atomic write
            err = -7;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_bh; ++i) {
            if (!work) continue;
            const int64_t bh = bh_list ? bh_list[i] : i;
            run_moments_slice(&pr, beta, gamma, prev_x, prev_B, valid_len, bh / H, bh % H,
                              m2_sel + i * N * N, m1_sel + i * N, work, work + P * N, work + 2 * P * N);
        }
        free(work);
    }
    return err;
}

/*
 * Gradients of the scan of ssd_oracle_f64 (reverse mode, written out for the
 * token recurrence). "mamba3/scan.py", verify(): the backward is checked
 * against the recurrence at float64; burn-mamba "mamba3/moments.rs", module
 * documentation: the recompute discipline, here the plain form that keeps
 * every state of a slice. With S_t the state after step t (S_-1 = init or 0),
 * U_t = R(theta_t) S_{t-1} and a_t = exp(da_t), so S_t = a_t U_t + W_t,
 * and G the gradient of the loss with respect to S_t, going backwards from
 * G = dfinal:
 *
 *   G      += sum_r dy[t,r] (outer) C[t,r]          (y_t reads S_t)
 *   dC[t,r][n] += sum_p dy[t,r][p] S_t[p][n]        (summed over the heads of a group)
 *   dx[t,r][p]  = sum_n G[p][n] B[t,r][n] + D dy[t,r][p]
 *   dB[t,r][n] += sum_p G[p][n] x[t,r][p]           (summed over the heads of a group)
 *   dD         += sum_{r,p} dy[t,r][p] x[t,r][p]
 *   dda[t]      = a_t sum_{p,n} G[p][n] U_t[p][n]
 *   dtheta[t,k] = a_t sum_p (G[p][2k+1] U_t[p][2k] - G[p][2k] U_t[p][2k+1])
 *   G           = a_t R(theta_t)^T G               (gradient with respect to S_{t-1})
 *
 * and dinit = G at the end. dy is fp32 [b,T,R,H,P]; dfinal fp32 [b,H,P,N] or
 * NULL (zero). Outputs are double: dx [b,T,R,H,P], dda [b,T,H],
 * dB and dC [b,T,R,G,N], dtheta [b,T,H,N/2] (when theta), dinit [b,H,P,N],
 * dD [H] (when D). Parallel over (batch, group) pairs; each keeps the T + 1
 * states of one head at a time.
 */
static void backward_head(const oracle_problem *pr, const float *dy, const float *dfinal,
                          int64_t b, int64_t h, double *st_all, double *G, double *U,
                          double *dx, double *dda, double *dB, double *dC, double *dth,
                          double *dinit, double *dD_h) {
    const int64_t T = pr->T, H = pr->H, P = pr->P, N = pr->N, G_ = pr->G, R = pr->R;
    const int64_t g = h / (H / G_);
    const int64_t PN = P * N;
    /* forward, keeping S_-1 .. S_{T-1} */
    double *s0 = st_all;
    for (int64_t i = 0; i < PN; ++i)
        s0[i] = pr->init_state ? (double)pr->init_state[(b * H + h) * PN + i] : 0.0;
    for (int64_t t = 0; t < T; ++t) {
        const double *sp = st_all + t * PN;
        double *sn = st_all + (t + 1) * PN;
        const int64_t row = (b * T + t) * H + h;
        for (int64_t i = 0; i < PN; ++i) sn[i] = sp[i];
        if (pr->theta) {
            for (int64_t k = 0; k < N / 2; ++k) {
                const double ang = (double)pr->theta[row * (N / 2) + k], co = cos(ang), si = sin(ang);
                for (int64_t p = 0; p < P; ++p) {
                    const double u0 = sp[p * N + 2 * k], u1 = sp[p * N + 2 * k + 1];
                    sn[p * N + 2 * k] = co * u0 - si * u1;
                    sn[p * N + 2 * k + 1] = si * u0 + co * u1;
                }
            }
        }
        const double at = exp((double)pr->da[row]);
        for (int64_t i = 0; i < PN; ++i) sn[i] *= at;
        for (int64_t r = 0; r < R; ++r)
            for (int64_t p = 0; p < P; ++p) {
                const double xe = load_elem(pr->x, (((b * T + t) * R + r) * H + h) * P + p, pr->in_dtype);
                for (int64_t n = 0; n < N; ++n)
                    sn[p * N + n] += xe * load_elem(pr->B, (((b * T + t) * R + r) * G_ + g) * N + n, pr->in_dtype);
            }
    }
    /* backward */
    for (int64_t i = 0; i < PN; ++i) G[i] = dfinal ? (double)dfinal[(b * H + h) * PN + i] : 0.0;
    const double dh = pr->D ? (double)pr->D[h] : 0.0;
    for (int64_t t = T - 1; t >= 0; --t) {
        const double *sc = st_all + (t + 1) * PN, *sp = st_all + t * PN;
        const int64_t row = (b * T + t) * H + h;
        for (int64_t r = 0; r < R; ++r) {
            const int64_t yrow = (((b * T + t) * R + r) * H + h) * P;
            const int64_t crow = (((b * T + t) * R + r) * G_ + g) * N;
            for (int64_t p = 0; p < P; ++p) {
                const double dyv = (double)dy[yrow + p];
                for (int64_t n = 0; n < N; ++n) {
                    G[p * N + n] += dyv * load_elem(pr->C, crow + n, pr->in_dtype);
                    dC[crow + n] += dyv * sc[p * N + n];
                }
            }
        }
        for (int64_t r = 0; r < R; ++r) {
            const int64_t xrow = (((b * T + t) * R + r) * H + h) * P;
            const int64_t brow = (((b * T + t) * R + r) * G_ + g) * N;
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                const double xe = load_elem(pr->x, xrow + p, pr->in_dtype);
                for (int64_t n = 0; n < N; ++n) {
                    acc += G[p * N + n] * load_elem(pr->B, brow + n, pr->in_dtype);
                    dB[brow + n] += G[p * N + n] * xe;
                }
                const double dyv = (double)dy[xrow + p];
                dx[xrow + p] = acc + dh * dyv;
                *dD_h += dyv * xe;
            }
        }
        /* U_t = R(theta_t) S_{t-1} */
        for (int64_t i = 0; i < PN; ++i) U[i] = sp[i];
        if (pr->theta) {
            for (int64_t k = 0; k < N / 2; ++k) {
                const double ang = (double)pr->theta[row * (N / 2) + k], co = cos(ang), si = sin(ang);
                for (int64_t p = 0; p < P; ++p) {
                    const double u0 = sp[p * N + 2 * k], u1 = sp[p * N + 2 * k + 1];
                    U[p * N + 2 * k] = co * u0 - si * u1;
                    U[p * N + 2 * k + 1] = si * u0 + co * u1;
                }
            }
        }
        const double at = exp((double)pr->da[row]);
        double acc = 0.0;
        for (int64_t i = 0; i < PN; ++i) acc += G[i] * U[i];
        dda[row] = at * acc;
        if (pr->theta) {
            for (int64_t k = 0; k < N / 2; ++k) {
                double tk = 0.0;
                for (int64_t p = 0; p < P; ++p)
                    tk += G[p * N + 2 * k + 1] * U[p * N + 2 * k] - G[p * N + 2 * k] * U[p * N + 2 * k + 1];
                dth[row * (N / 2) + k] = at * tk;
            }
        }
        /* G <- a_t R(theta_t)^T G */
        if (pr->theta) {
            for (int64_t k = 0; k < N / 2; ++k) {
                const double ang = (double)pr->theta[row * (N / 2) + k], co = cos(ang), si = sin(ang);
                for (int64_t p = 0; p < P; ++p) {
                    const double g0 = G[p * N + 2 * k], g1 = G[p * N + 2 * k + 1];
                    G[p * N + 2 * k] = co * g0 + si * g1;
                    G[p * N + 2 * k + 1] = -si * g0 + co * g1;
                }
            }
        }
        for (int64_t i = 0; i < PN; ++i) G[i] *= at;
    }
    for (int64_t i = 0; i < PN; ++i) dinit[(b * H + h) * PN + i] = G[i];
}

int ssd_backward_f64(int64_t batch, int64_t T, int64_t H, int64_t P, int64_t N,
                     int64_t G, int64_t R, int in_dtype,
                     const void *x, const float *da, const void *B, const void *C,
                     const float *D, const float *init_state, const float *theta,
                     const float *dy, const float *dfinal,
                     double *dx, double *dda, double *dB, double *dC, double *dtheta,
                     double *dinit, double *dD, int nthreads) {
    if (batch < 1 || T < 1 || H < 1 || P < 1 || N < 1 || G < 1 || R < 1) return -1;
    if (H % G != 0) return -2;
    if (theta && (N % 2)) return -3;
    if (in_dtype != ORACLE_IN_F32 && in_dtype != ORACLE_IN_BF16 && in_dtype != ORACLE_IN_F64)
        return -4;
    if (!x || !da || !B || !C || !dy || !dx || !dda || !dB || !dC || !dinit) return -5;
    if ((theta && !dtheta) || (D && !dD)) return -5;
    oracle_problem pr = {batch, T, H, P, N, G, R, in_dtype, x, B, C, da, D, init_state, theta};
    for (int64_t i = 0; i < batch * T * R * G * N; ++i) dB[i] = dC[i] = 0.0;
    if (dD)
        for (int64_t h = 0; h < H; ++h) dD[h] = 0.0;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    double *dDpart = (double *)calloc((size_t)(batch * H), sizeof(double));
    if (!dDpart) return -7;
#pragma omp parallel
    {
        double *work = (double *)malloc(sizeof(double) * (size_t)((T + 3) * P * N));
        if (!work) {
#pragma omp atomic write
            err = -7;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t bg = 0; bg < batch * G; ++bg) {
            if (!work) continue;
            const int64_t b = bg / G, g = bg % G;
            for (int64_t h = g * (H / G); h < (g + 1) * (H / G); ++h)
                backward_head(&pr, dy, dfinal, b, h, work + 2 * P * N, work, work + P * N, dx, dda, dB,
                              dC, dtheta, dinit, dDpart + b * H + h);
        }
        free(work);
    }
    if (dD)
        for (int64_t b = 0; b < batch; ++b)
            for (int64_t h = 0; h < H; ++h) dD[h] += dDpart[b * H + h];
    free(dDpart);
    return err;
}
