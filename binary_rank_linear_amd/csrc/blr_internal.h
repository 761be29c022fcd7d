// Internal interface between the C ABI (blr_api.hip) and the kernels
// (blr_kernels.hip). Not installed; the public interface is include/blr.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace blr {

// Smallest row tile of the MFMA contraction kernels; the column reductions
// fused into the contractions write one partial row per row tile, so the
// partial buffers are sized for this tile.
constexpr int GEMM_BM_MIN = 64;
// Tokens per partial of the standalone column reduction.
constexpr int COLSUM_ROWS = 64;
// Tokens per row of the dl partial buffer as sized (every producer writes
// one row per 64 tokens, within this).
constexpr int PART_ROWS_MIN = 32;

// Kernel kinds, for per-kernel timing.
enum KernelId {
    K_EXPAND = 0,
    K_TRANSPOSE, // bitmap [rows][r/32] -> [r][rows/32]
    K_GEMM_F1,   // a = (x.g) S_V
    K_GEMM_F2,   // c = (a.l) S_U^T, y (+)= h.c
    K_GEMM_B1,   // db = (dy.h.gs) S_U / gs, partials of dl
    K_GEMM_B2,   // dx' = (db.l.gs) S_V^T / gs, dx (+)= g.dx', partials of dg
    K_COLSUM,    // partials of dh = sum_t dy.c from the stored c tape
    K_GEMM_DH,   // c recomputed as in F2, partials of dh = sum_t dy.c
    K_FINISH,    // sum of partials into dh / dl / dg
    K_GEMM_B1_DH, // B1 with dh fused (c recomputed per column block)
    K_GEMM_SIGNS, // sign gradients G_U, G_V (contractions over tokens)
    K_SUMSQ,      // sum-of-squares partials (finite check)
    K_GEMM_PLANE, // dense frozen f16 linear
    K_SIGNS_REDUCE, // sign gradients: the token ranges' partials summed in order
    K_COUNT
};
const char *kernel_name(int id);

// out[m][n] = (sum_k f16(A[m][k] * colscale[k] * ascale) * S[n][k]) * oscale
// with the +-1 plane S [N][K] given as a bitmap; every [M][N] array below
// has row stride N.
struct GemmArgs {
    const float *A;        // [M][lda] f32
    int64_t lda;
    const float *colscale; // [K]
    float ascale;          // power of two
    const uint32_t *Bbits; // sign bitmap of the plane [N][K]: row n, word k/32, bit k%32 (set = +1)
    const uint16_t *Bplane; // GEMM_PLANE: the f16 plane [N][K] itself (no column scale)
    int64_t M;
    int N, K;
    float oscale;          // power of two (1/ascale)
    float *out;            // [M][N] raw product (F1: tape a, F2: tape c, B1: db)
    float *out2;           // [M][N] out2 (+)= out2col[n] * product (F2: y, B2: dx)
    const float *out2col;
    int out2acc;
    const float *dot_other; // [M][N]: partial[mt][n] = sum_{m in tile} product * other
    float *dot_partial;     // [ceil(M/gemm_tile_rows(kind))][N]
    // B1 with the dh reduction fused (GEMM_B1_DH): c = (a.l) S_U^T is
    // recomputed per column block of dy and dh partials sum dy.c over the tile
    const uint32_t *dh_bits; // bitmap of S_U [K][N/32] (K = d_out, N = r)
    const float *dh_a;       // the a tape [M][N]
    const float *dh_l;       // l [N]
    float *dh_partial;       // [(N/BN) * ceil(M/BM)][K], row nt * ceil(M/BM) + mt
    // A layer of several paths (y = sum_p h_p . c_p); zero for one path.
    // Paths along N (F1, B1: the ranks of all paths side by side): path_n
    // columns per path; the tile of column n0 belongs to path n0 / path_n,
    // whose column scales start at colscale + path * cs_pstride and, for the
    // fused dh role, whose S_U bitmap is dh_bits + path * dh_pstride words
    // with dh_row_words words per row.
    int path_n;
    int64_t cs_pstride, dh_pstride;
    int dh_row_words;
    // Paths along K (GEMM_F2_MP, GEMM_B2_MP: K = paths * path_k): the
    // bitmap of path q is Bbits + q * b_pstride words, rows of path_k / 32
    // words; at the end of each path's ranks the product is scaled by
    // out2col + q * o2_pstride into a running sum (stored at the end), and
    // that path's column partials go to dot_partial + q * dot_pstride.
    int path_k;
    int64_t b_pstride, o2_pstride, dot_pstride;
};

// F2 writes the c tape and y (F2) or y only (F2_NOTAPE); DH repeats F2's
// contraction with the same tiles (so c is bit-identical) and sums dy.c.
enum GemmKind {
    GEMM_F1 = 0, GEMM_F2, GEMM_F2_NOTAPE, GEMM_B1, GEMM_B2, GEMM_DH, GEMM_B1_DH, GEMM_PLANE,
    GEMM_F2_MP,  // y (+)= sum_p h_p . c_p over paths along K (no c tape)
    GEMM_B2_MP   // dx (+)= sum_p g_p . dx'_p, partials of dg_p per path
};
// Most paths of one layer the fused launches serve.
constexpr int MAX_PATHS = 4;
// At most this many 64 x 256 tiles (half the CUs) leave the chip half idle
// or worse: F1, B1 and the fused B1_DH then take 128-column tiles.
constexpr int64_t SMALL_GRID = 128;
// GEMM_B1_DH tiles for M tokens and P paths of r ranks: rank columns and
// token rows per workgroup (0 where the fused launch does not serve r). The
// dh partials of a path have ceil(M / b1dh_tile_rows(r)) * (r /
// b1dh_cols(M, r, P)) rows, at most 4 * ceil(M / 64); the dl partials
// ceil(M / b1dh_tile_rows(r)).
int b1dh_cols(int64_t M, int64_t r, int64_t P);
int b1dh_tile_rows(int64_t r);

// Sign-plane expansion jobs (one bitmap each; pl and/or plt may be null).
struct ExpandJob {
    const uint32_t *bits;  // [rows][ceil(r/32)]
    int64_t rows, r;
    uint16_t *pl;   // f16 [rows][r]
    uint16_t *plt;  // f16 [r][rows]
};
struct ExpandJobs {
    ExpandJob job[2];
    int count;
};

// Column-sum finishing jobs: out[n] += sum_p partial[p][n].
struct FinishJob {
    const float *partial;
    int64_t nparts;
    int N;
    float *out;
};
struct FinishJobs {
    FinishJob job[2 * MAX_PATHS + 1];
    int blocks_before[2 * MAX_PATHS + 1];
    int count;
};

// Token-contraction jobs for the sign gradients:
//   out[m][n] (+)= (sum_t f16(A[t][m] acol[m] ascale) f16(B[t][n] bcol[n] bscale)) oscale
// A [T][lda] and B [T][ldb] row-major (columns Mo and No used); out
// [Mo][No]; Mo, No multiples of 128.
struct TnJob {
    const float *A;
    const float *acol;
    float ascale;
    const float *B;
    const float *bcol;
    float bscale;
    int Mo, No;
    float oscale;
    float *out;
    int acc;
    int tiles_before;  // filled by the launcher
    int64_t lda, ldb;  // row strides of A and B (elements)
    int64_t elems_before;  // filled by the launcher: sum of Mo * No of the jobs before
};
struct TnJobs {
    TnJob job[2 * MAX_PATHS];
    int count;
    int64_t T;
    // Partial sums of token ranges 1 .. splits-1 (range 0 writes out itself):
    // part[(s - 1) * part_stride + elems_before + m * No + n], with
    // part_stride = sum over jobs of Mo * No. Needed when sign_splits() > 1.
    float *part;
};
// Token ranges of the sign-gradient contraction on its 256 x 256 tiles:
// enough ranges (each at least 512 tokens) to give about 256 workgroups over
// `tiles256` output tiles, 1 when the tiles alone fill the GPU. Only shapes
// whose output sizes are all multiples of 256 take those tiles (and ranges).
int sign_splits(int64_t tiles256, int64_t T);

// Launchers: enqueue on `s`, return the launch error (hipSuccess if none).
hipError_t launch_gemm_tn(TnJobs jobs, hipStream_t s);
hipError_t launch_sumsq(const float *a, int64_t n, float *partials, int nparts, hipStream_t s);
hipError_t launch_expand(const ExpandJobs &jobs, hipStream_t s);
// out [r][rows/32]: bit (i % 32) of word i / 32 in row k is rank k of row i
// of bits [rows][r/32] (rows and r multiples of 32); for paths > 1, bits
// holds that many such bitmaps back to back and out their transposes.
hipError_t launch_transpose_bits(const uint32_t *bits, int64_t rows, int64_t r, uint32_t *out, hipStream_t s,
                                 int paths = 1);
hipError_t launch_gemm(GemmKind kind, const GemmArgs &a, hipStream_t s);
int gemm_tile_rows(GemmKind kind);
hipError_t launch_colsum(const float *A, const float *B, int64_t M, int N, float *partial, hipStream_t s);
hipError_t launch_finish(FinishJobs jobs, hipStream_t s);

// Profiling hooks around each launch (no-ops unless enabled).
void prof_begin(int id, hipStream_t s);
void prof_end(hipStream_t s);

}  // namespace blr
