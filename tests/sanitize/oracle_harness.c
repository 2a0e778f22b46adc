/* oracle_harness.c -- runs every function of the FP64 oracle on small
 * seeded shapes (ragged lengths, a single token, segment starts everywhere,
 * initial states on and off) for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer, and checks that every output is finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_set_threads(int n);
void oracle_samu_controller(int B, int L, int D, const double *x_sel, const double *w_phi, const double *w_r,
                            double a_phi, double a_r, double *p, double *r, double *d, double *c, double *E,
                            double *C, double *S);
void oracle_samu_fwd(int B, int L, int D, const double *x_sel, const double *b, const double *w_phi,
                     const double *w_r, double a_phi, double a_r, const double *nu, const double *theta,
                     const double *z0, double *y, double *z_final, double *p_out, double *r_out);
void oracle_samu_bwd(int B, int L, int D, const double *x_sel, const double *b, const double *w_phi,
                     const double *w_r, double a_phi, double a_r, const double *nu, const double *theta,
                     const double *z0, const double *dy, const double *dz_final, double *dx_sel, double *db,
                     double *dz0, double *dw_phi, double *dw_r, double *da_phi, double *da_r, double *dnu,
                     double *dtheta);
void oracle_rglru_fwd(int B, int L, int D, const double *x, const double *lx, const double *la,
                      const double *alpha, const uint8_t *reset, const double *h0, double *y, double *h_final);
void oracle_rglru_bwd(int B, int L, int D, const double *x, const double *lx, const double *la,
                      const double *alpha, const uint8_t *reset, const double *h0, const double *dy,
                      const double *dh_final, double *dx, double *dlx, double *dla, double *dalpha, double *dh0);
void oracle_rglru_gate_proj(int B, int L, int D, const double *x, const double *w, const double *bias,
                            double *out);
void oracle_rglru_gate_proj_bwd(int B, int L, int D, const double *x, const double *w, const double *dl,
                                double *dx, double *dw, double *db);

static uint64_t rng = 88172645463325252ull;
static double urand(void) {  /* xorshift64, uniform in (-1, 1) */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static double *vec(size_t n) {
    double *v = malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) v[i] = urand();
    return v;
}
static int finite_all(const double *v, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(v[i])) return 0;
    return 1;
}
#define CHECK(v, n)                                                                 \
    do {                                                                            \
        if (!finite_all((v), (n))) {                                                \
            fprintf(stderr, "non-finite output %s at line %d\n", #v, __LINE__);    \
            return 2;                                                               \
        }                                                                           \
    } while (0)

int main(void) {
    oracle_set_threads(2);
    const int shapes[][3] = {{1, 1, 8}, {2, 5, 8}, {2, 37, 16}, {3, 70, 24}};
    for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
        const int B = shapes[s][0], L = shapes[s][1], D = shapes[s][2], M = D / 2;
        const size_t BL = (size_t)B * L, BLD = BL * D, BM = (size_t)B * M;
        double *x = vec(BLD), *b = vec(BLD), *wp = vec(D + 1), *wr = vec(D + 1), *nu = vec(M), *th = vec(M);
        for (int m = 0; m < M; ++m) nu[m] = 0.01 + fabs(nu[m]);
        double *z0 = vec(2 * BM), *dy = vec(BLD), *dzf = vec(2 * BM);
        double *c7 = malloc(7 * BL * sizeof(double));
        oracle_samu_controller(B, L, D, x, wp, wr, 0.5, -0.7, c7, c7 + BL, c7 + 2 * BL, c7 + 3 * BL, c7 + 4 * BL,
                               c7 + 5 * BL, c7 + 6 * BL);
        CHECK(c7, 7 * BL);
        double *y = malloc(BLD * sizeof(double)), *zf = malloc(2 * BM * sizeof(double));
        for (int use0 = 0; use0 < 2; ++use0) {
            oracle_samu_fwd(B, L, D, x, b, wp, wr, 0.5, -0.7, nu, th, use0 ? z0 : NULL, y, zf, c7, c7 + BL);
            CHECK(y, BLD);
            CHECK(zf, 2 * BM);
        }
        double *dx = malloc(BLD * sizeof(double)), *db = malloc(BLD * sizeof(double)),
               *dz0 = malloc(2 * BM * sizeof(double)), *dwp = malloc((D + 1) * sizeof(double)),
               *dwr = malloc((D + 1) * sizeof(double)), da[2], *dnu = malloc(M * sizeof(double)),
               *dth = malloc(M * sizeof(double));
        for (int usef = 0; usef < 2; ++usef) {
            oracle_samu_bwd(B, L, D, x, b, wp, wr, 0.5, -0.7, nu, th, z0, dy, usef ? dzf : NULL, dx, db, dz0, dwp,
                            dwr, da, da + 1, dnu, dth);
            CHECK(dx, BLD); CHECK(db, BLD); CHECK(dz0, 2 * BM); CHECK(dwp, D + 1); CHECK(dwr, D + 1);
            CHECK(da, 2); CHECK(dnu, M); CHECK(dth, M);
        }
        /* RG-LRU: no resets, some, and every token a segment start */
        double *lx = vec(BLD), *la = vec(BLD), *al = vec(D), *h0 = vec((size_t)B * D), *dhf = vec((size_t)B * D);
        uint8_t *rs = malloc(BL);
        double *hf = malloc((size_t)B * D * sizeof(double)), *dlx = malloc(BLD * sizeof(double)),
               *dla = malloc(BLD * sizeof(double)), *dal = malloc(D * sizeof(double)),
               *dh0 = malloc((size_t)B * D * sizeof(double));
        for (int mode = 0; mode < 3; ++mode) {
            for (size_t i = 0; i < BL; ++i) rs[i] = mode == 2 ? 1 : (mode == 1 && i % 5 == 0);
            oracle_rglru_fwd(B, L, D, x, lx, la, al, mode ? rs : NULL, mode == 1 ? NULL : h0, y, hf);
            CHECK(y, BLD); CHECK(hf, (size_t)B * D);
            oracle_rglru_bwd(B, L, D, x, lx, la, al, mode ? rs : NULL, h0, dy, mode ? dhf : NULL, dx, dlx, dla, dal,
                             dh0);
            CHECK(dx, BLD); CHECK(dlx, BLD); CHECK(dla, BLD); CHECK(dal, D); CHECK(dh0, (size_t)B * D);
        }
        if (D % 16 == 0) {
            const int Db = D / 16;
            double *w = vec((size_t)16 * Db * Db), *bias = vec(D), *dl = vec(BLD), *dw = malloc(16 * Db * Db * sizeof(double)),
                   *dbs = malloc(D * sizeof(double));
            oracle_rglru_gate_proj(B, L, D, x, w, bias, y);
            CHECK(y, BLD);
            for (size_t i = 0; i < BLD; ++i) dx[i] = 0.0;
            oracle_rglru_gate_proj_bwd(B, L, D, x, w, dl, dx, dw, dbs);
            CHECK(dx, BLD); CHECK(dw, (size_t)16 * Db * Db); CHECK(dbs, D);
            free(w); free(bias); free(dl); free(dw); free(dbs);
        }
        free(x); free(b); free(wp); free(wr); free(nu); free(th); free(z0); free(dy); free(dzf); free(c7); free(y);
        free(zf); free(dx); free(db); free(dz0); free(dwp); free(dwr); free(dnu); free(dth); free(lx); free(la);
        free(al); free(h0); free(dhf); free(rs); free(hf); free(dlx); free(dla); free(dal); free(dh0);
    }
    printf("oracle harness: all outputs finite\n");
    return 0;
}
