/*
 * f64 CPU oracle of the binary low-rank (`blr`) linear layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do. It shares no code, header, table or helper with the
 * HIP library.
 *
 * Source: the cortiq-engine page "src/gpu_wgpu/train_mm.rs" (0.8.21): the
 * module doc block (the layer W^ = diag(h) S_U diag(l) S_V^T diag(g) and its
 * forward and backward equations), the `expand` shader (bit convention) and
 * `blr_forward` / `blr_backward` (overwrite and accumulate rules).
 *
 * Loop order (this file's own): per token, the forward forms a, then c, then
 * y from the equations; the backward forms db and dx' per token into
 * per-token arrays, and the column sums dh, dl, dg run over the tokens in
 * index order afterwards.
 *
 * Exact maths in f64; f32 staging and f16 rounding are NOT simulated (the
 * method reaches this result up to the rounding of its staged operands).
 * The loss scale `gscale` cancels exactly in the method and does not appear.
 *
 * Determinism: every sum runs in a fixed order (over k, i, j inside a
 * token; over tokens in order for the column sums), so results do not
 * depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

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

/* out[col] += sum over t = 0..M-1 (in order) of P[t][col] Q[t][col]
 * (`colsum_prod` shader). Columns are split over threads in fixed ranges of
 * 64; each thread walks the tokens in order over its range. */
static void colsum_prod(int64_t M, int64_t n, const double *P, const double *Q, double *out) {
    int64_t nch = (n + 63) / 64;
#pragma omp parallel for schedule(static)
    for (int64_t ch = 0; ch < nch; ++ch) {
        int64_t c0 = ch * 64, c1 = c0 + 64 < n ? c0 + 64 : n;
        double acc[64];
        for (int64_t c = c0; c < c1; ++c) acc[c - c0] = 0.0;
        for (int64_t t = 0; t < M; ++t)
            for (int64_t c = c0; c < c1; ++c) acc[c - c0] += P[t * n + c] * Q[t * n + c];
        for (int64_t c = c0; c < c1; ++c) out[c] += acc[c - c0];
    }
}

/* Backward (`blr_backward`; doc block, backward lines), recomputing a and c
 * from x (the method keeps them as a tape of the last forward on the same x):
 *   dh[i] += sum_t dy[t][i] c[t][i]
 *   db[t][k] = sum_i dy[t][i] h[i] S_U[i][k]
 *   dl[k] += sum_t a[t][k] db[t][k]
 *   dx'[t][j] = sum_k db[t][k] l[k] S_V[j][k]
 *   dg[j] += sum_t x[t][j] dx'[t][j]
 *   dx[t][j] = (accumulate_dx ? dx[t][j] : 0) + g[j] dx'[t][j]
 * dh, dl, dg always accumulate (the caller zeroes them). The per-token
 * arrays are formed first (in parallel over tokens), then each column sum
 * runs over the tokens in order (in parallel over columns). Returns 0, or -1
 * when memory runs out. */
int oracle_blr_backward(int64_t M, int64_t d_in, int64_t d_out, int64_t r, const double *x, const double *dy,
                        const uint32_t *bits_u, const uint32_t *bits_v, const double *h, const double *l,
                        const double *g, double *dh, double *dl, double *dg, double *dx, int accumulate_dx) {
    double *SU = decode_alloc(bits_u, d_out, r);
    double *SV = decode_alloc(bits_v, d_in, r);
    double *A = (double *)malloc((size_t)(M * r) * sizeof(double));
    double *C = (double *)malloc((size_t)(M * d_out) * sizeof(double));
    double *DB = (double *)malloc((size_t)(M * r) * sizeof(double));
    double *DXP = (double *)malloc((size_t)(M * d_in) * sizeof(double));
    int bad = (SU == NULL || SV == NULL || A == NULL || C == NULL || DB == NULL || DXP == NULL);
    if (!bad) {
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < M; ++t) {
            const double *dyt = dy + t * d_out;
            double *a = A + t * r, *db = DB + t * r, *dxp = DXP + t * d_in;
            token_forward(d_in, d_out, r, x + t * d_in, SU, SV, l, g, a, C + t * d_out);
            for (int64_t k = 0; k < r; ++k) db[k] = 0.0;
            for (int64_t i = 0; i < d_out; ++i) {
                double dyh = dyt[i] * h[i];
                const double *su = SU + i * r;
                for (int64_t k = 0; k < r; ++k) db[k] += dyh * su[k];
            }
            for (int64_t j = 0; j < d_in; ++j) {
                const double *sv = SV + j * r;
                double s = 0.0;
                for (int64_t k = 0; k < r; ++k) s += db[k] * l[k] * sv[k];
                dxp[j] = s;
            }
            for (int64_t j = 0; j < d_in; ++j)
                dx[t * d_in + j] = (accumulate_dx ? dx[t * d_in + j] : 0.0) + g[j] * dxp[j];
        }
        colsum_prod(M, d_out, dy, C, dh);
        colsum_prod(M, r, A, DB, dl);
        colsum_prod(M, d_in, x, DXP, dg);
    }
    free(SU);
    free(SV);
    free(A);
    free(C);
    free(DB);
    free(DXP);
    return bad ? -1 : 0;
}

/* Sign gradients (page: `blr_backward` with sign state, and the f64 host
 * reference `host_sign_grads` of its tests): the gradients of
 * L = sum_{t,i} dy[t][i] y[t][i] with respect to the entries of S_U and S_V
 * taken as real numbers,
 *   a[t][k] = sum_j x[t][j] g[j] S_V[j][k]
 *   b[t][k] = sum_i dy[t][i] h[i] S_U[i][k]
 *   G_U[i][k] = (accumulate ? G_U[i][k] : 0) + h[i] l[k] sum_t dy[t][i] a[t][k]
 *   G_V[j][k] = (accumulate ? G_V[j][k] : 0) + g[j] l[k] sum_t x[t][j] b[t][k]
 * The per-token arrays a and b are formed first (in parallel over tokens),
 * then each row of G sums over the tokens in order (in parallel over rows).
 * Returns 0, or -1 when memory runs out. */
int oracle_blr_sign_grads(int64_t M, int64_t d_in, int64_t d_out, int64_t r, const double *x, const double *dy,
                          const uint32_t *bits_u, const uint32_t *bits_v, const double *h, const double *l,
                          const double *g, double *gu, double *gv, int accumulate) {
    double *SU = decode_alloc(bits_u, d_out, r);
    double *SV = decode_alloc(bits_v, d_in, r);
    double *A = (double *)malloc((size_t)(M * r) * sizeof(double));
    double *B = (double *)malloc((size_t)(M * r) * sizeof(double));
    int bad = (SU == NULL || SV == NULL || A == NULL || B == NULL);
    if (!bad) {
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < M; ++t) {
            const double *xt = x + t * d_in, *dyt = dy + t * d_out;
            double *a = A + t * r, *b = B + t * r;
            for (int64_t k = 0; k < r; ++k) a[k] = b[k] = 0.0;
            for (int64_t j = 0; j < d_in; ++j) {
                const double xg = xt[j] * g[j];
                const double *sv = SV + j * r;
                for (int64_t k = 0; k < r; ++k) a[k] += xg * sv[k];
            }
            for (int64_t i = 0; i < d_out; ++i) {
                const double dyh = dyt[i] * h[i];
                const double *su = SU + i * r;
                for (int64_t k = 0; k < r; ++k) b[k] += dyh * su[k];
            }
        }
        /* G_U rows then G_V rows: out[row][k] = s[row] l[k] sum_t P[t][row] Q[t][k] */
#pragma omp parallel
        {
            double *acc = (double *)malloc((size_t)r * sizeof(double));
            if (acc == NULL) {
#pragma omp atomic write
                bad = 1;
            } else {
#pragma omp for schedule(static)
                for (int64_t row = 0; row < d_out + d_in; ++row) {
                    const int u = row < d_out;
                    const int64_t i = u ? row : row - d_out;
                    const int64_t n = u ? d_out : d_in;
                    const double *P = u ? dy : x, *Q = u ? A : B;
                    double *out = (u ? gu : gv) + i * r;
                    const double s = u ? h[i] : g[i];
                    for (int64_t k = 0; k < r; ++k) acc[k] = 0.0;
                    for (int64_t t = 0; t < M; ++t) {
                        const double p = P[t * n + i];
                        const double *q = Q + t * r;
                        for (int64_t k = 0; k < r; ++k) acc[k] += p * q[k];
                    }
                    for (int64_t k = 0; k < r; ++k) out[k] = (accumulate ? out[k] : 0.0) + s * l[k] * acc[k];
                }
            }
            free(acc);
        }
    }
    free(SU);
    free(SV);
    free(A);
    free(B);
    return bad ? -1 : 0;
}

/* Sum of squares (page: `sumsq` shader and wrapper, used to check a buffer
 * for non-finite values): sum_i a[i]^2 in f64, in index order. Non-finite
 * inputs propagate (inf or NaN result). */
double oracle_sumsq(const double *a, int64_t n) {
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += a[i] * a[i];
    return s;
}

/* IEEE binary16 bit pattern -> double, exactly (sign, 5-bit exponent with
 * bias 15, 10-bit fraction; subnormals, infinities and NaN included). */
static double f16_to_f64(uint16_t hbits) {
    const int sign = hbits >> 15, e = (hbits >> 10) & 31, f = hbits & 1023;
    double v;
    if (e == 0) v = (double)f / 1024.0 / 16384.0;                  /* f * 2^-24 */
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = (1.0 + (double)f / 1024.0) * ldexp(1.0, e - 15);
    return sign ? -v : v;
}

void oracle_f16_decode(const uint16_t *h, int64_t n, double *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = f16_to_f64(h[i]);
}

/* Dense frozen linear (page: `plane_linear`): y[t][i] = sum_j x[t][j] P[i][j]
 * with P the f16 plane [n][k] taken exactly; the staging scale cancels. */
int oracle_plane_linear(int64_t M, int64_t n, int64_t k, const double *x, const uint16_t *plane, double *y) {
    double *P = (double *)malloc((size_t)(n * k) * sizeof(double));
    if (P == NULL) return -1;
    oracle_f16_decode(plane, n * k, P);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < M; ++t)
        for (int64_t i = 0; i < n; ++i) {
            double s = 0.0;
            for (int64_t j = 0; j < k; ++j) s += x[t * k + j] * P[i * k + j];
            y[t * n + i] = s;
        }
    free(P);
    return 0;
}
