/*
 * f64 CPU oracle of the binary low-rank (`blr`) linear layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do. It shares no code, header, table or helper with the
 * HIP library.
 *
 * Source: the cortiq-engine page "src/gpu_wgpu/train_mm.rs" (0.8.21), its
 * module doc block (the layer W^ = diag(h) S_U diag(l) S_V^T diag(g) and
 * the forward/backward equations), the `expand` shader (bit convention),
 * `blr_forward` / `blr_backward` (overwrite and accumulate rules), and the
 * f64 host reference inside test `blr_layer_matches_host`, which this file
 * follows step for step, one token at a time.
 *
 * Exact maths in f64; f32 staging and f16 rounding are NOT simulated (the
 * method reaches this result up to the rounding of its staged operands).
 * The loss scale `gscale` cancels exactly in the method and does not appear.
 *
 * Determinism: tokens are cut into fixed blocks of ORACLE_TBLK; each block
 * sums its tokens in order, and block partials are added in block order, so
 * results do not depend on the thread count.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_TBLK 64

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* O1, `expand` shader: S[row][k] = +1 when bit (k mod 32) of word
 * bits[row][k/32] is set, else -1; words per row = ceil(r/32); bits at
 * ranks >= r in the last word are never read. */
void oracle_decode_signs(const uint32_t *bits, int64_t rows, int64_t r, double *S) {
    int64_t W = (r + 31) / 32;
    for (int64_t row = 0; row < rows; ++row)
        for (int64_t k = 0; k < r; ++k) {
            uint32_t word = bits[row * W + k / 32];
            int bit = (int)((word >> (k % 32)) & 1u);
            S[row * r + k] = bit ? 1.0 : -1.0;
        }
}

/* `expand` shader: the f16 planes PL[rows][r] and PLT[r][rows] the GEMMs
 * read. +1 is the f16 pattern 0x3C00, -1 is 0xBC00. Either output may be
 * NULL. */
void oracle_expand_planes(const uint32_t *bits, int64_t rows, int64_t r, uint16_t *pl, uint16_t *plt) {
    int64_t W = (r + 31) / 32;
    for (int64_t row = 0; row < rows; ++row)
        for (int64_t k = 0; k < r; ++k) {
            int bit = (int)((bits[row * W + k / 32] >> (k % 32)) & 1u);
            uint16_t v = bit ? (uint16_t)0x3C00 : (uint16_t)0xBC00;
            if (pl) pl[row * r + k] = v;
            if (plt) plt[k * rows + row] = v;
        }
}

static double *decode_alloc(const uint32_t *bits, int64_t rows, int64_t r) {
    double *S = (double *)malloc((size_t)(rows * r) * sizeof(double));
    if (S) oracle_decode_signs(bits, rows, r, S);
    return S;
}

/* One token of the forward (doc block, forward line):
 *   a[k] = sum_j x[j] g[j] S_V[j][k]
 *   c[i] = sum_k a[k] l[k] S_U[i][k]                                   */
static void token_forward(int64_t d_in, int64_t d_out, int64_t r, const double *xt, const double *SU,
                          const double *SV, const double *l, const double *g, double *a, double *c) {
    for (int64_t k = 0; k < r; ++k) a[k] = 0.0;
    for (int64_t j = 0; j < d_in; ++j) {
        double xg = xt[j] * g[j];
        const double *sv = SV + j * r;
        for (int64_t k = 0; k < r; ++k) a[k] += xg * sv[k];
    }
    for (int64_t i = 0; i < d_out; ++i) {
        const double *su = SU + i * r;
        double s = 0.0;
        for (int64_t k = 0; k < r; ++k) s += a[k] * l[k] * su[k];
        c[i] = s;
    }
}

/* Forward (`blr_forward`; doc block "y += h (.) c").
 * y [M][d_out]: accumulate_y = 0 overwrites with h*c, 1 adds h*c (the page
 * overwrites for path 0 and adds for later paths).
 * a [M][r] and c [M][d_out] (may be NULL) receive the tape. Returns 0, or -1
 * when memory runs out. */
int oracle_blr_forward(int64_t M, int64_t d_in, int64_t d_out, int64_t r, const double *x,
                       const uint32_t *bits_u, const uint32_t *bits_v, const double *h, const double *l,
                       const double *g, double *y, int accumulate_y, double *a_out, double *c_out) {
    double *SU = decode_alloc(bits_u, d_out, r);
    double *SV = decode_alloc(bits_v, d_in, r);
    int bad = (SU == NULL || SV == NULL);
    if (!bad) {
#pragma omp parallel
        {
            double *a = (double *)malloc((size_t)r * sizeof(double));
            double *c = (double *)malloc((size_t)d_out * sizeof(double));
            if (a == NULL || c == NULL) {
#pragma omp atomic write
                bad = 1;
            } else {
#pragma omp for schedule(static)
                for (int64_t t = 0; t < M; ++t) {
                    token_forward(d_in, d_out, r, x + t * d_in, SU, SV, l, g, a, c);
                    for (int64_t i = 0; i < d_out; ++i)
                        y[t * d_out + i] = (accumulate_y ? y[t * d_out + i] : 0.0) + h[i] * c[i];
                    if (a_out) memcpy(a_out + t * r, a, (size_t)r * sizeof(double));
                    if (c_out) memcpy(c_out + t * d_out, c, (size_t)d_out * sizeof(double));
                }
            }
            free(a);
            free(c);
        }
    }
    free(SU);
    free(SV);
    return bad ? -1 : 0;
}

/* Backward (`blr_backward`; doc block, backward lines), recomputing a and c
 * from x (the method keeps them as a tape of the last forward on the same x):
 *   dh[i] += sum_t dy[t][i] c[t][i]
 *   db[k]  = sum_i dy[i] h[i] S_U[i][k]                 (per token)
 *   dl[k] += sum_t a[t][k] db[t][k]
 *   dx'[j] = sum_k db[k] l[k] S_V[j][k]                 (per token)
 *   dg[j] += sum_t x[t][j] dx'[t][j]
 *   dx[t][j] = (accumulate_dx ? dx[t][j] : 0) + g[j] dx'[t][j]
 * dh, dl, dg always accumulate (the caller zeroes them). Returns 0, or -1
 * when memory runs out. */
int oracle_blr_backward(int64_t M, int64_t d_in, int64_t d_out, int64_t r, const double *x, const double *dy,
                        const uint32_t *bits_u, const uint32_t *bits_v, const double *h, const double *l,
                        const double *g, double *dh, double *dl, double *dg, double *dx, int accumulate_dx) {
    int64_t nblk = (M + ORACLE_TBLK - 1) / ORACLE_TBLK;
    double *SU = decode_alloc(bits_u, d_out, r);
    double *SV = decode_alloc(bits_v, d_in, r);
    double *ph = (double *)calloc((size_t)(nblk * d_out), sizeof(double));
    double *pl = (double *)calloc((size_t)(nblk * r), sizeof(double));
    double *pg = (double *)calloc((size_t)(nblk * d_in), sizeof(double));
    int bad = (SU == NULL || SV == NULL || ph == NULL || pl == NULL || pg == NULL);
    if (!bad) {
#pragma omp parallel
        {
            double *a = (double *)malloc((size_t)r * sizeof(double));
            double *c = (double *)malloc((size_t)d_out * sizeof(double));
            double *db = (double *)malloc((size_t)r * sizeof(double));
            double *dxp = (double *)malloc((size_t)d_in * sizeof(double));
            if (a == NULL || c == NULL || db == NULL || dxp == NULL) {
#pragma omp atomic write
                bad = 1;
            } else {
#pragma omp for schedule(static)
                for (int64_t b = 0; b < nblk; ++b) {
                    int64_t t1 = (b + 1) * ORACLE_TBLK < M ? (b + 1) * ORACLE_TBLK : M;
                    for (int64_t t = b * ORACLE_TBLK; t < t1; ++t) {
                        const double *xt = x + t * d_in;
                        const double *dyt = dy + t * d_out;
                        token_forward(d_in, d_out, r, xt, SU, SV, l, g, a, c);
                        for (int64_t i = 0; i < d_out; ++i) ph[b * d_out + i] += dyt[i] * c[i];
                        for (int64_t k = 0; k < r; ++k) db[k] = 0.0;
                        for (int64_t i = 0; i < d_out; ++i) {
                            double dyh = dyt[i] * h[i];
                            const double *su = SU + i * r;
                            for (int64_t k = 0; k < r; ++k) db[k] += dyh * su[k];
                        }
                        for (int64_t k = 0; k < r; ++k) pl[b * r + k] += a[k] * db[k];
                        for (int64_t j = 0; j < d_in; ++j) {
                            const double *sv = SV + j * r;
                            double s = 0.0;
                            for (int64_t k = 0; k < r; ++k) s += db[k] * l[k] * sv[k];
                            dxp[j] = s;
                        }
                        for (int64_t j = 0; j < d_in; ++j) {
                            pg[b * d_in + j] += xt[j] * dxp[j];
                            dx[t * d_in + j] = (accumulate_dx ? dx[t * d_in + j] : 0.0) + g[j] * dxp[j];
                        }
                    }
                }
            }
            free(a);
            free(c);
            free(db);
            free(dxp);
        }
    }
    if (!bad) {
        for (int64_t b = 0; b < nblk; ++b) {
            for (int64_t i = 0; i < d_out; ++i) dh[i] += ph[b * d_out + i];
            for (int64_t k = 0; k < r; ++k) dl[k] += pl[b * r + k];
            for (int64_t j = 0; j < d_in; ++j) dg[j] += pg[b * d_in + j];
        }
    }
    free(SU);
    free(SV);
    free(ph);
    free(pl);
    free(pg);
    return bad ? -1 : 0;
}
