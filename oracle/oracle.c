/*
 * oracle.c -- plain, serial-in-time FP64 CPU reference for the SAMU complex
 * diagonal scan and the RG-LRU real gated scan, forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library.  It is slow on purpose: one token at a time, in FP64, following
 * the equations of the pages in their own order and notation.  Threads only
 * split recurrences that are independent by definition (one complex mode, one
 * real channel).
 *
 * Sources (page titles as published):
 *   [SAMU-GPU]  "SAMU 与 RG-LRU 的 H800 训练性能对比", section 05 "SAMU 在 GPU
 *               上如何运行": controller equations, the per-token special
 *               functions, the mode transition lambda, the recurrence, and the
 *               backward relations for the state, c-bar/d-bar and p-bar/r-bar.
 *   [SAMU-GPU]  section 04 "RG-LRU 在 GPU 上如何运行": gates, retention a_t,
 *               normalized write, recurrence, reset semantics, backward and
 *               the alpha-gradient reduction.
 *   [PROTOCOL]  "Griffin 第 4、5 节 H800 对照协议", "RG-LRU 的固定方程": reset
 *               at a segment start cuts the old state and drops the
 *               normalization multiplier of that token.
 *
 * Every input and result is FP64.  The Python wrapper widens the BF16 and
 * FP32 bit patterns the GPU receives exactly (BF16 -> FP32 -> FP64), so both
 * sides read the same numbers; finite-difference checks pass FP64 directly.
 *
 * Readings where the pages leave a step open (each also listed in the design
 * notes of the repository):
 *   - state index: z_t = lambda_t z_{t-1} + b_t, the output of token t is z_t;
 *   - visible output y_t = z_t (Re, Im interleaved), no write normalization
 *     for SAMU (no SAMU equation has one);
 *   - drive layout b[..., m, 0] = Re, b[..., m, 1] = Im;
 *   - selector x_sel has D entries, x~ = [x_sel; 1] has D+1, and the
 *     direction norm runs over all D+1 entries;
 *   - M = D/2 in the 1/sqrt(M) scaling;
 *   - complex cotangents are dL/dRe + i dL/dIm;
 *   - the square-root derivative of the RG-LRU write normalization is capped
 *     at 1000 (1/(2 sqrt(u)) with u clamped below at 2.5e-7).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* Lower clamp of u = 1 - a^2 inside the square-root derivative. */
#define RGLRU_SQRT_GRAD_UMIN 2.5e-7


int oracle_max_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }

/* ------------------------------------------------------------------------ */
/* SAMU controller ([SAMU-GPU] section 05, first four display equations).     */
/*   x~_t = [x_sel_t; 1],  w^ = w / ||w||_2                                  */
/*   p_t = tanh(x~_t . w^_phi),  r_t = tanh(x~_t . w^_r),  q = r / (1 + r^2) */
/*   d_t = tanh(a_phi)/sqrt(M) p_t,  c_t = tanh(a_r)/sqrt(M) q(r_t)          */
/*   E_t = exp(c_t), C_t = cos d_t, S_t = sin d_t (once per token)           */
/* ------------------------------------------------------------------------ */
static void unit_direction(int n, const double *w, double *w_hat, double *norm)
{
    double s = 0.0;
    for (int j = 0; j < n; ++j) s += w[j] * w[j];
    *norm = sqrt(s);
    for (int j = 0; j < n; ++j) w_hat[j] = w[j] / *norm;
}

void oracle_samu_controller(int B, int L, int D, const double *x_sel,
                            const double *w_phi, const double *w_r,
                            double a_phi, double a_r,
                            double *p, double *r, double *d, double *c,
                            double *E, double *C, double *S)
{
    const int M = D / 2;
    double *wh_phi = malloc(sizeof(double) * (D + 1));
    double *wh_r = malloc(sizeof(double) * (D + 1));
    double n_phi, n_r;
    unit_direction(D + 1, w_phi, wh_phi, &n_phi);
    unit_direction(D + 1, w_r, wh_r, &n_r);
    const double amp_phi = tanh(a_phi) / sqrt(M);
    const double amp_r = tanh(a_r) / sqrt(M);

    #pragma omp parallel for schedule(static)
    for (long bt = 0; bt < (long)B * L; ++bt) {
        const double *xr = x_sel + bt * D;
        double u_phi = wh_phi[D];          /* the appended constant 1 */
        double u_r = wh_r[D];
        for (int j = 0; j < D; ++j) {
            double x = xr[j];
            u_phi += x * wh_phi[j];
            u_r += x * wh_r[j];
        }
        double pt = tanh(u_phi), rt = tanh(u_r);
        double qt = rt / (1.0 + rt * rt);
        double dt = amp_phi * pt, ct = amp_r * qt;
        p[bt] = pt; r[bt] = rt; d[bt] = dt; c[bt] = ct;
        E[bt] = exp(ct); C[bt] = cos(dt); S[bt] = sin(dt);
    }
    free(wh_phi);
    free(wh_r);
}

/* lambda_{t,m} = exp(-nu_m E_t) [(cos th C - sin th S) + i (sin th C + cos th S)] */
static inline void samu_lambda(double nu, double cth, double sth,
                               double Et, double Ct, double St,
                               double *lr, double *li)
{
    double rho = exp(-nu * Et);
    *lr = rho * (cth * Ct - sth * St);
    *li = rho * (sth * Ct + cth * St);
}

/* ------------------------------------------------------------------------ */
/* SAMU forward: z_{t,m} = lambda_{t,m} z_{t-1,m} + b_{t,m}; y_t = z_t.       */
/* y is [B,L,M,2] (Re, Im); z_final is [B,M,2]; p, r are [B,L].               */
/* ------------------------------------------------------------------------ */
void oracle_samu_fwd(int B, int L, int D, const double *x_sel, const double *b,
                     const double *w_phi, const double *w_r, double a_phi, double a_r,
                     const double *nu, const double *theta, const double *z0,
                     double *y, double *z_final, double *p_out, double *r_out)
{
    const int M = D / 2;
    const long BL = (long)B * L;
    double *p = malloc(sizeof(double) * BL), *r = malloc(sizeof(double) * BL);
    double *d = malloc(sizeof(double) * BL), *c = malloc(sizeof(double) * BL);
    double *E = malloc(sizeof(double) * BL), *C = malloc(sizeof(double) * BL);
    double *S = malloc(sizeof(double) * BL);
    oracle_samu_controller(B, L, D, x_sel, w_phi, w_r, a_phi, a_r, p, r, d, c, E, C, S);

    #pragma omp parallel for schedule(static) collapse(2)
    for (int bb = 0; bb < B; ++bb) {
        for (int m = 0; m < M; ++m) {
            const double nu_m = nu[m];
            const double cth = cos(theta[m]), sth = sin(theta[m]);
            double zr = 0.0, zi = 0.0;
            if (z0) {
                zr = z0[((long)bb * M + m) * 2 + 0];
                zi = z0[((long)bb * M + m) * 2 + 1];
            }
            for (int t = 0; t < L; ++t) {
                const long bt = (long)bb * L + t;
                double lr, li;
                samu_lambda(nu_m, cth, sth, E[bt], C[bt], S[bt], &lr, &li);
                const long o = (bt * M + m) * 2;
                double br = b[o], bi = b[o + 1];
                double nr = lr * zr - li * zi + br;
                double ni = lr * zi + li * zr + bi;
                zr = nr; zi = ni;
                y[o] = zr; y[o + 1] = zi;
            }
            if (z_final) {
                z_final[((long)bb * M + m) * 2 + 0] = zr;
                z_final[((long)bb * M + m) * 2 + 1] = zi;
            }
        }
    }
    if (p_out) memcpy(p_out, p, sizeof(double) * BL);
    if (r_out) memcpy(r_out, r, sizeof(double) * BL);
    free(p); free(r); free(d); free(c); free(E); free(C); free(S);
}

/* ------------------------------------------------------------------------ */
/* SAMU backward: exact adjoint of the forward above.                         */
/*   state:  z-bar_{t-1} += conj(lambda_t) z-bar_t,  b-bar_t = z-bar_t         */
/*   with gamma = conj(lambda_t) g_t conj(z_{t-1}) for g_t = total z-bar_t:    */
/*     d nu_m += -E_t Re gamma,  d theta_m += Im gamma,                        */
/*     c-bar_t += -nu_m E_t Re gamma,  d-bar_t += Im gamma  (summed over m)    */
/*   controller: p-bar = d-bar tanh(a_phi)/sqrt(M),                            */
/*               r-bar = c-bar tanh(a_r)/sqrt(M) (1 - r^2)/(1 + r^2)^2         */
/* dx_sel [B,L,D]; db [B,L,M,2]; dz0 [B,M,2] (may be NULL); dw_* [D+1];        */
/* da_* scalars; dnu, dtheta [M].                                              */
/* ------------------------------------------------------------------------ */
void oracle_samu_bwd(int B, int L, int D, const double *x_sel, const double *b,
                     const double *w_phi, const double *w_r, double a_phi, double a_r,
                     const double *nu, const double *theta, const double *z0,
                     const double *dy, const double *dz_final,
                     double *dx_sel, double *db, double *dz0,
                     double *dw_phi, double *dw_r, double *da_phi, double *da_r,
                     double *dnu, double *dtheta)
{
    const int M = D / 2;
    const long BL = (long)B * L;
    double *p = malloc(sizeof(double) * BL), *r = malloc(sizeof(double) * BL);
    double *d = malloc(sizeof(double) * BL), *c = malloc(sizeof(double) * BL);
    double *E = malloc(sizeof(double) * BL), *C = malloc(sizeof(double) * BL);
    double *S = malloc(sizeof(double) * BL);
    oracle_samu_controller(B, L, D, x_sel, w_phi, w_r, a_phi, a_r, p, r, d, c, E, C, S);

    const int T = omp_get_max_threads();
    /* per-thread partial sums of c-bar_t and d-bar_t over the modes it owns */
    double *cbar_t = calloc((size_t)T * BL, sizeof(double));
    double *dbar_t = calloc((size_t)T * BL, sizeof(double));

    #pragma omp parallel
    {
        const int tid = omp_get_thread_num();
        double *zh = malloc(sizeof(double) * 2 * ((size_t)L + 1)); /* z_0..z_L */
        double *cb = cbar_t + (size_t)tid * BL, *dbr = dbar_t + (size_t)tid * BL;
        #pragma omp for schedule(static)
        for (int m = 0; m < M; ++m) {
            const double nu_m = nu[m];
            const double cth = cos(theta[m]), sth = sin(theta[m]);
            double gnu = 0.0, gth = 0.0;
            for (int bb = 0; bb < B; ++bb) {
                /* replay the forward recurrence, keeping every state */
                double zr = 0.0, zi = 0.0;
                if (z0) {
                    zr = z0[((long)bb * M + m) * 2 + 0];
                    zi = z0[((long)bb * M + m) * 2 + 1];
                }
                zh[0] = zr; zh[1] = zi;
                for (int t = 0; t < L; ++t) {
                    const long bt = (long)bb * L + t;
                    double lr, li;
                    samu_lambda(nu_m, cth, sth, E[bt], C[bt], S[bt], &lr, &li);
                    const long o = (bt * M + m) * 2;
                    double br = b[o], bi = b[o + 1];
                    double nr = lr * zr - li * zi + br;
                    double ni = lr * zi + li * zr + bi;
                    zr = nr; zi = ni;
                    zh[2 * (t + 1)] = zr; zh[2 * (t + 1) + 1] = zi;
                }
                /* reverse adjoint */
                double kr = 0.0, ki = 0.0;   /* z-bar arriving from token t+1 */
                if (dz_final) {
                    kr = dz_final[((long)bb * M + m) * 2 + 0];
                    ki = dz_final[((long)bb * M + m) * 2 + 1];
                }
                for (int t = L - 1; t >= 0; --t) {
                    const long bt = (long)bb * L + t;
                    const long o = (bt * M + m) * 2;
                    double gr = dy[o] + kr;
                    double gi = dy[o + 1] + ki;
                    db[o] = gr; db[o + 1] = gi;
                    double lr, li;
                    samu_lambda(nu_m, cth, sth, E[bt], C[bt], S[bt], &lr, &li);
                    /* conj(lambda) * g */
                    double hr = lr * gr + li * gi;
                    double hi = lr * gi - li * gr;
                    /* gamma = conj(lambda) g conj(z_{t-1}) */
                    double pr = zh[2 * t], pi = zh[2 * t + 1];
                    double gam_r = hr * pr + hi * pi;
                    double gam_i = hi * pr - hr * pi;
                    gnu += -E[bt] * gam_r;
                    gth += gam_i;
                    cb[bt] += -nu_m * E[bt] * gam_r;
                    dbr[bt] += gam_i;
                    kr = hr; ki = hi;
                }
                if (dz0) {
                    dz0[((long)bb * M + m) * 2 + 0] = kr;
                    dz0[((long)bb * M + m) * 2 + 1] = ki;
                }
            }
            dnu[m] = gnu;
            dtheta[m] = gth;
        }
        free(zh);
    }

    /* c-bar_t, d-bar_t: sum the per-thread partials in thread order */
    double *cbar = calloc(BL, sizeof(double)), *dbar = calloc(BL, sizeof(double));
    for (int k = 0; k < T; ++k)
        for (long i = 0; i < BL; ++i) {
            cbar[i] += cbar_t[(size_t)k * BL + i];
            dbar[i] += dbar_t[(size_t)k * BL + i];
        }
    free(cbar_t); free(dbar_t);

    /* controller backward */
    double *wh_phi = malloc(sizeof(double) * (D + 1));
    double *wh_r = malloc(sizeof(double) * (D + 1));
    double n_phi, n_r;
    unit_direction(D + 1, w_phi, wh_phi, &n_phi);
    unit_direction(D + 1, w_r, wh_r, &n_r);
    const double th_phi = tanh(a_phi), th_r = tanh(a_r);
    const double sM = sqrt(M);
    double *u_phi = malloc(sizeof(double) * BL), *u_r = malloc(sizeof(double) * BL);
    double sum_dp = 0.0, sum_cq = 0.0;
    for (long bt = 0; bt < BL; ++bt) {
        double pt = p[bt], rt = r[bt];
        double qt = rt / (1.0 + rt * rt);
        double pbar = dbar[bt] * th_phi / sM;
        double rbar = cbar[bt] * th_r / sM * (1.0 - rt * rt) / ((1.0 + rt * rt) * (1.0 + rt * rt));
        u_phi[bt] = pbar * (1.0 - pt * pt);
        u_r[bt] = rbar * (1.0 - rt * rt);
        sum_dp += dbar[bt] * pt;
        sum_cq += cbar[bt] * qt;
    }
    *da_phi = (1.0 - th_phi * th_phi) / sM * sum_dp;
    *da_r = (1.0 - th_r * th_r) / sM * sum_cq;

    #pragma omp parallel for schedule(static)
    for (long bt = 0; bt < BL; ++bt)
        for (int j = 0; j < D; ++j)
            dx_sel[bt * D + j] = u_phi[bt] * wh_phi[j] + u_r[bt] * wh_r[j];

    /* g^ = sum_t u-bar_t x~_t, then dw = (g^ - w^ (w^ . g^)) / ||w|| */
    double *g_phi = calloc(D + 1, sizeof(double)), *g_r = calloc(D + 1, sizeof(double));
    #pragma omp parallel for schedule(static)
    for (int j = 0; j <= D; ++j) {
        double sp = 0.0, sr = 0.0;
        for (long bt = 0; bt < BL; ++bt) {
            double x = (j < D) ? (x_sel[bt * D + j]) : 1.0;
            sp += u_phi[bt] * x;
            sr += u_r[bt] * x;
        }
        g_phi[j] = sp; g_r[j] = sr;
    }
    double dot_phi = 0.0, dot_r = 0.0;
    for (int j = 0; j <= D; ++j) { dot_phi += wh_phi[j] * g_phi[j]; dot_r += wh_r[j] * g_r[j]; }
    for (int j = 0; j <= D; ++j) {
        dw_phi[j] = (g_phi[j] - wh_phi[j] * dot_phi) / n_phi;
        dw_r[j] = (g_r[j] - wh_r[j] * dot_r) / n_r;
    }

    free(g_phi); free(g_r); free(u_phi); free(u_r); free(wh_phi); free(wh_r);
    free(cbar); free(dbar);
    free(p); free(r); free(d); free(c); free(E); free(C); free(S);
}

/* ------------------------------------------------------------------------ */
/* RG-LRU ([SAMU-GPU] section 04):                                           */
/*   g^x = sigmoid(l^x), g^a = sigmoid(l^a), a_t = exp(-8 g^a softplus(alpha))*/
/*   b_t = x_t g^x sqrt(max(1 - a_t^2, 0)),  h_t = a_t h_{t-1} + b_t         */
/*   at a segment start (reset flag): a_t = 0 and the multiplier is 1.        */
/* x, lx, la, y: [B,L,D]; alpha [D]; reset [B,L] (NULL = none); h0 [B,D].     */
/* ------------------------------------------------------------------------ */
static inline double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }
static inline double softplus(double v) { return log1p(exp(v)); }

typedef struct { double a, m, gx, ga, x; int rs; } rglru_tok;

static inline rglru_tok rglru_token(double x, double lx, double la, double sp, int rs)
{
    rglru_tok k;
    k.x = x; k.rs = rs;
    k.gx = sigmoid(lx);
    k.ga = sigmoid(la);
    k.a = exp(-8.0 * k.ga * sp);
    double u = 1.0 - k.a * k.a;
    k.m = sqrt(u > 0.0 ? u : 0.0);
    if (rs) { k.a = 0.0; k.m = 1.0; }
    return k;
}

void oracle_rglru_fwd(int B, int L, int D, const double *x, const double *lx,
                      const double *la, const double *alpha, const unsigned char *reset,
                      const double *h0, double *y, double *h_final)
{
    #pragma omp parallel for schedule(static) collapse(2)
    for (int bb = 0; bb < B; ++bb) {
        for (int dd = 0; dd < D; ++dd) {
            const double sp = softplus(alpha[dd]);
            double h = h0 ? h0[(long)bb * D + dd] : 0.0;
            for (int t = 0; t < L; ++t) {
                const long bt = (long)bb * L + t, o = bt * D + dd;
                rglru_tok k = rglru_token(x[o], lx[o],
                                          la[o], sp, reset ? reset[bt] != 0 : 0);
                h = k.a * h + k.x * k.gx * k.m;
                y[o] = h;
            }
            if (h_final) h_final[(long)bb * D + dd] = h;
        }
    }
}

void oracle_rglru_bwd(int B, int L, int D, const double *x, const double *lx,
                      const double *la, const double *alpha, const unsigned char *reset,
                      const double *h0, const double *dy, const double *dh_final,
                      double *dx, double *dlx, double *dla, double *dalpha, double *dh0)
{
    #pragma omp parallel
    {
        double *hh = malloc(sizeof(double) * ((size_t)L + 1)); /* h_0..h_L */
        #pragma omp for schedule(static)
        for (int dd = 0; dd < D; ++dd) {
            const double sp = softplus(alpha[dd]);
            const double dsp = sigmoid(alpha[dd]);   /* d softplus / d alpha */
            double galpha = 0.0;
            for (int bb = 0; bb < B; ++bb) {
                double h = h0 ? h0[(long)bb * D + dd] : 0.0;
                hh[0] = h;
                for (int t = 0; t < L; ++t) {
                    const long bt = (long)bb * L + t, o = bt * D + dd;
                    rglru_tok k = rglru_token(x[o], lx[o],
                                              la[o], sp, reset ? reset[bt] != 0 : 0);
                    h = k.a * h + k.x * k.gx * k.m;
                    hh[t + 1] = h;
                }
                double carry = dh_final ? dh_final[(long)bb * D + dd] : 0.0;
                for (int t = L - 1; t >= 0; --t) {
                    const long bt = (long)bb * L + t, o = bt * D + dd;
                    rglru_tok k = rglru_token(x[o], lx[o],
                                              la[o], sp, reset ? reset[bt] != 0 : 0);
                    double g = dy[o] + carry;
                    dx[o] = g * k.gx * k.m;
                    dlx[o] = g * k.x * k.m * k.gx * (1.0 - k.gx);
                    if (!k.rs) {
                        double u = 1.0 - k.a * k.a;
                        if (u < RGLRU_SQRT_GRAD_UMIN) u = RGLRU_SQRT_GRAD_UMIN;
                        double dm_da = -k.a / sqrt(u);
                        double abar = g * hh[t] + g * k.x * k.gx * dm_da;
                        dla[o] = abar * k.a * (-8.0 * sp) * k.ga * (1.0 - k.ga);
                        galpha += abar * k.a * (-8.0 * k.ga) * dsp;
                    } else {
                        dla[o] = 0.0;
                    }
                    carry = k.a * g;
                }
                if (dh0) dh0[(long)bb * D + dd] = carry;
            }
            dalpha[dd] = galpha;
        }
        free(hh);
    }
}

/* ------------------------------------------------------------------------ */
/* RG-LRU gate projections ([PROTOCOL] "RG-LRU 的固定方程": both gates come   */
/* from 16-block block-diagonal linear layers).  Reading: block i covers     */
/* channels [i Db, (i+1) Db) with Db = D/16, the weight is stored [16, Db,   */
/* Db] as (block, output, input), and each channel has a bias:               */
/*   l[t, i Db + o] = bias[i Db + o] + sum_k W[i][o][k] x[t, i Db + k].      */
/* ------------------------------------------------------------------------ */
void oracle_rglru_gate_proj(int B, int L, int D, const double *x, const double *w,
                            const double *bias, double *out)
{
    const int Db = D / 16;
    const long BL = (long)B * L;
#pragma omp parallel for schedule(static)
    for (long bt = 0; bt < BL; ++bt) {
        for (int i = 0; i < 16; ++i) {
            const double *xb = x + bt * D + (long)i * Db;
            for (int o = 0; o < Db; ++o) {
                const double *wr = w + ((long)i * Db + o) * Db;
                double s = bias[i * Db + o];
                for (int k = 0; k < Db; ++k) s += wr[k] * xb[k];
                out[bt * D + (long)i * Db + o] = s;
            }
        }
    }
}

/* Adjoint of the projection for a cotangent dl of l:                        */
/*   dx[t, i Db + k] += sum_o W[i][o][k] dl[t, i Db + o]    (accumulated),   */
/*   dW[i][o][k] = sum_t dl[t, i Db + o] x[t, i Db + k],  dbias = sum_t dl.  */
void oracle_rglru_gate_proj_bwd(int B, int L, int D, const double *x, const double *w,
                                const double *dl, double *dx, double *dw, double *dbias)
{
    const int Db = D / 16;
    const long BL = (long)B * L;
#pragma omp parallel for schedule(static)
    for (long bt = 0; bt < BL; ++bt) {
        for (int i = 0; i < 16; ++i) {
            for (int k = 0; k < Db; ++k) {
                double s = 0.0;
                for (int o = 0; o < Db; ++o)
                    s += w[((long)i * Db + o) * Db + k] * dl[bt * D + (long)i * Db + o];
                dx[bt * D + (long)i * Db + k] += s;
            }
        }
    }
#pragma omp parallel for schedule(static)
    for (int c = 0; c < D; ++c) {
        const int i = c / Db, o = c - i * Db;
        double sb = 0.0;
        for (long bt = 0; bt < BL; ++bt) sb += dl[bt * D + c];
        dbias[c] = sb;
        for (int k = 0; k < Db; ++k) {
            double s = 0.0;
            for (long bt = 0; bt < BL; ++bt) s += dl[bt * D + c] * x[bt * D + (long)i * Db + k];
            dw[((long)i * Db + o) * Db + k] = s;
        }
    }
}
