// HIP kernels of the binary low-rank (`blr`) layer for CDNA4 (gfx950).
//
// The computation follows the layer of the cortiq-engine page
// "src/gpu_wgpu/train_mm.rs" (module doc block; `expand`, `cvt_col`,
// `colsum_prod`, `scale_acc` shaders; the GEMM contract of `mm`). The
// page's separate staging and scaling passes are fused here: the f32 -> f16
// staging of the activation operand happens in the contraction's load
// prologue, the diag(h) / diag(g) scaling, the 1/gscale and the tapes are
// written in its epilogue, and the dl / dg column reductions are formed in
// the epilogue of the contraction that produces db / dx'.
#include "blr_internal.h"

namespace blr {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// f16 bit patterns of +1 and -1.
constexpr uint32_t F16_ONE = 0x3C00u;
constexpr uint32_t F16_MINUS_ONE = 0xBC00u;

__device__ __forceinline__ uint32_t sign_pair(uint32_t b0, uint32_t b1) {
    // bit set -> +1 (0x3C00), clear -> -1 (0xBC00): flip the sign bit of -1
    return (F16_MINUS_ONE ^ (b0 << 15)) | ((F16_MINUS_ONE ^ (b1 << 15)) << 16);
}

// ---------------------------------------------------------------------------
// Sign expansion (page: `expand` shader). One workgroup decodes a tile of
// 64 rows x 64 ranks: the 128 words go through LDS, then both planes are
// written with 32-byte row segments (the page writes the transposed plane
// one strided half at a time).
constexpr int EXP_TR = 64;
constexpr int EXP_TK = 64;

__global__ __launch_bounds__(256) void expand_signs_kernel(const uint32_t *__restrict__ bits, int64_t rows,
                                                           int64_t r, int64_t W, uint16_t *__restrict__ pl,
                                                           uint16_t *__restrict__ plt) {
    __shared__ uint32_t wb[EXP_TR][2];
    const int t = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.y * EXP_TR;
    const int64_t k0 = (int64_t)blockIdx.x * EXP_TK;
    const int64_t w0 = k0 >> 5;
    if (t < 2 * EXP_TR) {
        const int row = t >> 1, wi = t & 1;
        uint32_t v = 0;
        if (r0 + row < rows && w0 + wi < W) v = bits[(r0 + row) * W + w0 + wi];
        wb[row][wi] = v;
    }
    __syncthreads();
    if (pl != nullptr) {
        const int row = t >> 2, seg = t & 3;
        const int64_t grow = r0 + row;
        const int64_t kb = k0 + seg * 16;
        if (grow < rows && kb < r) {
            const uint32_t word = wb[row][seg >> 1] >> ((seg & 1) * 16);
            uint32_t d[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) d[q] = sign_pair((word >> (2 * q)) & 1u, (word >> (2 * q + 1)) & 1u);
            uint16_t *dst = pl + grow * r + kb;
            if (kb + 16 <= r && (r & 7) == 0) {
                reinterpret_cast<uint4 *>(dst)[0] = make_uint4(d[0], d[1], d[2], d[3]);
                reinterpret_cast<uint4 *>(dst)[1] = make_uint4(d[4], d[5], d[6], d[7]);
            } else {
                for (int e = 0; e < 16 && kb + e < r; ++e) dst[e] = (uint16_t)(d[e >> 1] >> ((e & 1) * 16));
            }
        }
    }
    if (plt != nullptr) {
        const int kk = t >> 2, seg = t & 3;
        const int64_t gk = k0 + kk;
        const int64_t rb = r0 + seg * 16;
        if (gk < r && rb < rows) {
            const int wi = kk >> 5, sh = kk & 31;
            uint32_t d[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                d[q] = sign_pair((wb[seg * 16 + 2 * q][wi] >> sh) & 1u, (wb[seg * 16 + 2 * q + 1][wi] >> sh) & 1u);
            uint16_t *dst = plt + gk * rows + rb;
            if (rb + 16 <= rows && (rows & 7) == 0) {
                reinterpret_cast<uint4 *>(dst)[0] = make_uint4(d[0], d[1], d[2], d[3]);
                reinterpret_cast<uint4 *>(dst)[1] = make_uint4(d[4], d[5], d[6], d[7]);
            } else {
                for (int e = 0; e < 16 && rb + e < rows; ++e) dst[e] = (uint16_t)(d[e >> 1] >> ((e & 1) * 16));
            }
        }
    }
}

hipError_t launch_expand(const uint32_t *bits, int64_t rows, int64_t r, uint16_t *pl, uint16_t *plt,
                         hipStream_t s) {
    const int64_t W = (r + 31) / 32;
    dim3 grid((unsigned)((r + EXP_TK - 1) / EXP_TK), (unsigned)((rows + EXP_TR - 1) / EXP_TR));
    prof_begin(K_EXPAND, s);
    hipLaunchKernelGGL(expand_signs_kernel, grid, dim3(256), 0, s, bits, rows, r, W, pl, plt);
    hipError_t e = hipGetLastError();
    prof_end(s);
    return e;
}

// ---------------------------------------------------------------------------
// f16 MFMA contraction with fused staging (page: `cvt_col` feeding `mm`,
// then `scale_acc` / `colsum_prod`):
//   prod[m][n] = (sum_k f16(A[m][k] * colscale[k] * ascale) * B[n][k]) * oscale
// B is an f16 sign plane [N][K]. Each workgroup computes a BM x BN tile with
// WM x WN waves; each wave holds (BM/WM) x (BN/WN) f32 accumulators as
// 32x32 MFMA tiles (v_mfma_f32_32x32x16_f16). The K loop is double
// buffered through LDS: the next tile's global loads are in flight while the
// current tile is multiplied.
//
// MFMA 32x32x16 operand layout: lane l supplies row (l % 32) of A and column
// (l % 32) of B, each with the 8 consecutive k of group (l / 32). The
// accumulator register v of lane l holds row 8*(v/4) + 4*(l/32) + v%4,
// column l % 32.
template <int BM, int BN, int BK, int WM, int WN, bool OUT, bool OUT2, bool DOT>
__global__ __launch_bounds__(WM *WN * 64) void gemm_kernel(GemmArgs p) {
    constexpr int NT = WM * WN * 64;
    constexpr int LDK = BK + 8;  // halves per LDS row (pad: conflict-free 16-byte reads)
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int A_CHUNKS = BM * BK / 4;  // float4 chunks of an A tile
    constexpr int B_CHUNKS = BN * BK / 8;  // 16-byte chunks of a B tile
    constexpr int A_PER = A_CHUNKS / NT, B_PER = B_CHUNKS / NT;
    static_assert(A_CHUNKS % NT == 0 && B_CHUNKS % NT == 0, "tile/thread mismatch");
    static_assert(TM % 32 == 0 && TN % 32 == 0 && BK % 16 == 0, "tile shape");

    __shared__ __attribute__((aligned(16))) _Float16 As[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) _Float16 Bs[2][BN * LDK];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int nk = p.K / BK;
    const int64_t M = p.M;
    const int N = p.N;

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    float4 ar[A_PER];
    uint4 br[B_PER];

    auto gload = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int v = 0; v < A_PER; ++v) {
            const int idx = tid + v * NT;
            const int row = idx / (BK / 4), c4 = idx % (BK / 4);
            const int64_t gm = m0 + row;
            if (gm < M)
                ar[v] = *reinterpret_cast<const float4 *>(p.A + gm * p.lda + k0 + c4 * 4);
            else
                ar[v] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int v = 0; v < B_PER; ++v) {
            const int idx = tid + v * NT;
            const int row = idx / (BK / 8), c8 = idx % (BK / 8);
            br[v] = *reinterpret_cast<const uint4 *>(p.B + (int64_t)(n0 + row) * p.K + k0 + c8 * 8);
        }
    };
    auto sstore = [&](int kt, int buf) {
        const int k0 = kt * BK;
#pragma unroll
        for (int v = 0; v < A_PER; ++v) {
            const int idx = tid + v * NT;
            const int row = idx / (BK / 4), c4 = idx % (BK / 4);
            const float4 cs = *reinterpret_cast<const float4 *>(p.colscale + k0 + c4 * 4);
            half4_t hv;
            hv[0] = (_Float16)(ar[v].x * cs.x * p.ascale);
            hv[1] = (_Float16)(ar[v].y * cs.y * p.ascale);
            hv[2] = (_Float16)(ar[v].z * cs.z * p.ascale);
            hv[3] = (_Float16)(ar[v].w * cs.w * p.ascale);
            *reinterpret_cast<half4_t *>(&As[buf][row * LDK + c4 * 4]) = hv;
        }
#pragma unroll
        for (int v = 0; v < B_PER; ++v) {
            const int idx = tid + v * NT;
            const int row = idx / (BK / 8), c8 = idx % (BK / 8);
            *reinterpret_cast<uint4 *>(&Bs[buf][row * LDK + c8 * 8]) = br[v];
        }
    };
    auto compute = [&](int buf) {
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            half8_t af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const half8_t *>(
                    &As[buf][(wm * TM + i * 32 + (lane & 31)) * LDK + s * 16 + (lane >> 5) * 8]);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = *reinterpret_cast<const half8_t *>(
                    &Bs[buf][(wn * TN + j * 32 + (lane & 31)) * LDK + s * 16 + (lane >> 5) * 8]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
    };

    gload(0);
    sstore(0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        compute(cur);
        if (kt + 1 < nk) sstore(kt + 1, cur ^ 1);
        __syncthreads();
    }

    // Epilogue: products, tapes, scaled outputs and column partials.
    float dotp[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) dotp[j] = 0.0f;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int gn = n0 + wn * TN + j * 32 + (lane & 31);
        const float c2 = OUT2 ? p.out2col[gn] : 0.0f;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int rin = wm * TM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int64_t gm = m0 + rin;
                if (gm < M) {
                    const float val = acc[i][j][v] * p.oscale;
                    const int64_t o = gm * N + gn;
                    if (OUT) p.out[o] = val;
                    if (OUT2) p.out2[o] = (p.out2acc ? p.out2[o] : 0.0f) + val * c2;
                    if (DOT) dotp[j] += val * p.dot_other[o];
                }
            }
        }
    }
    if (DOT) {
        // rows of a column are spread over the two lane halves and the WM
        // waves of a column strip: fold lanes l and l+32, then waves in order
        float *red = reinterpret_cast<float *>(&As[0][0]);  // [WM][BN], K loop is done
#pragma unroll
        for (int j = 0; j < FN; ++j) dotp[j] += __shfl_xor(dotp[j], 32);
        if (lane < 32) {
#pragma unroll
            for (int j = 0; j < FN; ++j) red[wm * BN + wn * TN + j * 32 + lane] = dotp[j];
        }
        __syncthreads();
        for (int c = tid; c < BN; c += NT) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < WM; ++w) s += red[w * BN + c];
            p.dot_partial[(int64_t)blockIdx.y * N + n0 + c] = s;
        }
    }
}

template <int BM, int BN, int BK, int WM, int WN, bool OUT, bool OUT2, bool DOT>
static hipError_t launch_gemm_t(int id, const GemmArgs &a, hipStream_t s) {
    static_assert(BM == GEMM_BM, "partials are laid out per GEMM_BM tile");
    static_assert(WM * BN * 4 <= 2 * BM * (BK + 8) * 2, "reduction buffer fits in the A tiles");
    dim3 grid((unsigned)(a.N / BN), (unsigned)((a.M + BM - 1) / BM));
    prof_begin(id, s);
    hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, WM, WN, OUT, OUT2, DOT>), grid, dim3(WM * WN * 64), 0, s, a);
    hipError_t e = hipGetLastError();
    prof_end(s);
    return e;
}

hipError_t launch_gemm(GemmKind kind, const GemmArgs &a, hipStream_t s) {
    switch (kind) {
        case GEMM_F1: return launch_gemm_t<128, 128, 32, 2, 2, true, false, false>(K_GEMM_F1, a, s);
        case GEMM_F2: return launch_gemm_t<128, 128, 32, 2, 2, true, true, false>(K_GEMM_F2, a, s);
        case GEMM_B1: return launch_gemm_t<128, 128, 32, 2, 2, true, false, true>(K_GEMM_B1, a, s);
        case GEMM_B2: return launch_gemm_t<128, 128, 32, 2, 2, false, true, true>(K_GEMM_B2, a, s);
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Column reduction (page: `colsum_prod`, one thread per column with a serial
// row loop, later two-pass): here each thread owns 4 adjacent columns
// (float4, so a wavefront reads 1 KB contiguous per row) over COLSUM_ROWS
// tokens; partial[chunk][col] is summed in chunk order by finish_kernel.
__global__ __launch_bounds__(256) void colsum_prod_kernel(const float *__restrict__ A, const float *__restrict__ B,
                                                          int64_t M, int N, float *__restrict__ partial) {
    const int col = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (col >= N) return;
    const int64_t t0 = (int64_t)blockIdx.y * COLSUM_ROWS;
    const int64_t t1 = t0 + COLSUM_ROWS < M ? t0 + COLSUM_ROWS : M;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t t = t0; t < t1; ++t) {
        const float4 a = *reinterpret_cast<const float4 *>(A + t * N + col);
        const float4 b = *reinterpret_cast<const float4 *>(B + t * N + col);
        s.x += a.x * b.x;
        s.y += a.y * b.y;
        s.z += a.z * b.z;
        s.w += a.w * b.w;
    }
    *reinterpret_cast<float4 *>(partial + (int64_t)blockIdx.y * N + col) = s;
}

hipError_t launch_colsum(const float *A, const float *B, int64_t M, int N, float *partial, hipStream_t s) {
    dim3 grid((unsigned)((N + 1023) / 1024), (unsigned)((M + COLSUM_ROWS - 1) / COLSUM_ROWS));
    prof_begin(K_COLSUM, s);
    hipLaunchKernelGGL(colsum_prod_kernel, grid, dim3(256), 0, s, A, B, M, N, partial);
    hipError_t e = hipGetLastError();
    prof_end(s);
    return e;
}

// out[n] += sum over parts (in order) of partial[part][n].
__global__ __launch_bounds__(256) void finish_kernel(const float *__restrict__ partial, int64_t nparts, int N,
                                                     float *__restrict__ out) {
    const int col = blockIdx.x * 256 + threadIdx.x;
    if (col >= N) return;
    float s = 0.0f;
    for (int64_t q = 0; q < nparts; ++q) s += partial[q * N + col];
    out[col] = out[col] + s;
}

hipError_t launch_finish(const float *partial, int64_t nparts, int N, float *out, hipStream_t s) {
    prof_begin(K_FINISH, s);
    hipLaunchKernelGGL(finish_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, partial, nparts, N, out);
    hipError_t e = hipGetLastError();
    prof_end(s);
    return e;
}

const char *kernel_name(int id) {
    switch (id) {
        case K_EXPAND: return "expand_signs";
        case K_GEMM_F1: return "gemm_f1_xg_sv";
        case K_GEMM_F2: return "gemm_f2_al_sut";
        case K_GEMM_B1: return "gemm_b1_dyh_su";
        case K_GEMM_B2: return "gemm_b2_dbl_svt";
        case K_COLSUM: return "colsum_dy_c";
        case K_FINISH: return "colsum_finish";
    }
    return "?";
}

}  // namespace blr
