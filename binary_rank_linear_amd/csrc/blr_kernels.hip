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
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

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
// one strided half at a time). One launch serves up to two bitmaps
// (blockIdx.z picks the job).
constexpr int EXP_TR = 64;
constexpr int EXP_TK = 64;

__global__ __launch_bounds__(256) void expand_signs_kernel(ExpandJobs jobs) {
    const ExpandJob &jb = jobs.job[blockIdx.z];
    const int64_t rows = jb.rows, r = jb.r, W = (jb.r + 31) / 32;
    const uint32_t *__restrict__ bits = jb.bits;
    uint16_t *__restrict__ pl = jb.pl;
    uint16_t *__restrict__ plt = jb.plt;
    const int64_t r0 = (int64_t)blockIdx.y * EXP_TR;
    const int64_t k0 = (int64_t)blockIdx.x * EXP_TK;
    if (r0 >= rows || k0 >= r) return;  // this job's grid is smaller than the launch's
    __shared__ uint32_t wb[EXP_TR][2];
    const int t = threadIdx.x;
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

hipError_t launch_expand(const ExpandJobs &jobs, hipStream_t s) {
    int64_t gx = 1, gy = 1;
    for (int j = 0; j < jobs.count; ++j) {
        const int64_t x = (jobs.job[j].r + EXP_TK - 1) / EXP_TK, y = (jobs.job[j].rows + EXP_TR - 1) / EXP_TR;
        gx = x > gx ? x : gx;
        gy = y > gy ? y : gy;
    }
    prof_begin(K_EXPAND, s);
    hipLaunchKernelGGL(expand_signs_kernel, dim3((unsigned)gx, (unsigned)gy, (unsigned)jobs.count), dim3(256), 0, s,
                       jobs);
    hipError_t e = hipGetLastError();
    prof_end(s);
    return e;
}

// ---------------------------------------------------------------------------
// f16 MFMA contraction with fused staging (page: `cvt_col` feeding `mm`,
// then `scale_acc` / `colsum_prod`):
//   prod[m][n] = (sum_k f16(A[m][k] * (colscale[k] * ascale)) * S[n][k]) * oscale
// S is the +-1 plane [N][K], read as its bitmap (one u32 per row per K
// step) and decoded to f16 while staging: the page's expanded f16 planes
// are never materialised. ascale is a power of two, so folding it into
// colscale rounds exactly like the page's (A * col) * scale except where an
// f32 intermediate would overflow.
//
// Wave roles: a workgroup holds WM x WN "MMA" waves and as many "loader"
// waves, so each SIMD runs one of each. Loader waves keep P K-stages of
// global loads in flight in a statically indexed register ring, convert
// the activation stage to f16 with its column scale and write both operand
// tiles to one of two LDS buffers; MMA waves read fragments from the other
// buffer and issue MFMAs (v_mfma_f32_32x32x16_f16, f32 accumulators). One
// barrier per K step swaps the buffers, so the VALU staging of one wave and
// the MFMAs of the other overlap on every SIMD.
//
// Tile order: workgroups are dealt round-robin to the 8 XCDs, each with its
// own L2. The launch index is remapped so that tiles sharing operands run
// on the same XCD (see GM below).
//
// MFMA 32x32x16 operand layout: lane l supplies row (l % 32) of A and column
// (l % 32) of B, each with the 8 consecutive k of group (l / 32). The
// accumulator register v of lane l holds row 8*(v/4) + 4*(l/32) + v%4,
// column l % 32.
constexpr int NUM_XCD = 8;

// Signs of bits 0..15 of `w` (bit j = sign j; set = +1) as 16 f16 values:
// lo = signs 0..7, hi = signs 8..15, two per dword (sign 2q in the low
// half). Both 16-bit lanes of y hold the inverted bits; a packed shift moves
// bit 2q (low lane) and bit 2q+1 (high lane) to the lanes' sign positions,
// and the and-or keeps those sign bits over the pattern of +1.
__device__ __forceinline__ uint32_t sign_dword(uint32_t y, int q, uint32_t sgnmask, uint32_t one16) {
    const u16x2_t sh = {(uint16_t)(15 - 2 * q), (uint16_t)(14 - 2 * q)};
    const u16x2_t t = __builtin_bit_cast(u16x2_t, y) << sh;
    return (__builtin_bit_cast(uint32_t, t) & sgnmask) | one16;
}
// Signs of bits 0..UB-1 of `w` as UB f16 values in UB/8 16-byte groups.
template <int UB>
__device__ __forceinline__ void decode_signs(uint32_t w, uint32_t sgnmask, uint32_t one16, u32x4_t *d) {
#pragma unroll
    for (int h = 0; h < (UB + 15) / 16; ++h) {
        const uint32_t y = (~(w >> (16 * h)) & 0xFFFFu) * 0x10001u;
#pragma unroll
        for (int q = 0; q < (UB < 16 ? UB / 2 : 8); ++q) d[2 * h + q / 4][q % 4] = sign_dword(y, q, sgnmask, one16);
    }
}

// Bitmap transpose: out [r][rows/32] from bits [rows][r/32]; each thread
// assembles one output word from 32 input words (rows 32*jw .. 32*jw+31,
// rank k). Consecutive threads take consecutive ranks, so a wavefront reads
// a few words per row (cache broadcasts).
__global__ __launch_bounds__(256) void transpose_bits_kernel(const uint32_t *__restrict__ bits, int64_t rows,
                                                             int64_t r, uint32_t *__restrict__ out) {
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t rw = rows / 32, W = r / 32;
    if (id >= r * rw) return;
    const int64_t k = id % r, jw = id / r;
    const uint32_t *src = bits + jw * 32 * W + k / 32;
    const int sh = (int)(k % 32);
    uint32_t word = 0;
#pragma unroll 8
    for (int b = 0; b < 32; ++b) word |= ((src[b * W] >> sh) & 1u) << b;
    out[k * rw + jw] = word;
}

hipError_t launch_transpose_bits(const uint32_t *bits, int64_t rows, int64_t r, uint32_t *out, hipStream_t s) {
    const int64_t n = r * (rows / 32);
    prof_begin(K_TRANSPOSE, s);
    hipLaunchKernelGGL(transpose_bits_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, bits, rows, r, out);
    hipError_t e = hipGetLastError();
    prof_end(s);
    return e;
}

template <int BM, int BN, int BK, int WM, int WN, int LW, int P, bool OUT, bool OUT2, bool DOT, int GM>
__global__ __launch_bounds__((1 + LW) * WM *WN * 64) void gemm_kernel(GemmArgs p) {
    constexpr int NW = WM * WN;      // MMA waves; LW * NW loader waves
    constexpr int NTR = LW * NW * 64;  // loader threads
    constexpr int LDK = BK + 8;      // halves per LDS row (pad: conflict-free 16-byte reads)
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int A_CHUNKS = BM * BK / 4;   // float4 chunks of an A tile
    constexpr int UB = BN * BK / NTR;       // signs of a B tile decoded per loader thread
    constexpr int A_PER = A_CHUNKS / NTR;
    constexpr int AROW_STEP = NTR / (BK / 4);
    static_assert(BK == 32, "one bitmap word per plane row per K step");
    static_assert(A_CHUNKS % NTR == 0 && (UB == 8 || UB == 16 || UB == 32), "tile/thread mismatch");
    static_assert(TM % 32 == 0 && TN % 32 == 0 && BK % 16 == 0, "tile shape");
    static_assert(NTR % (BK / 4) == 0, "a loader thread keeps one column group of A");
    static_assert(P % 2 == 0, "LDS buffer index must be static in the unrolled loop");
    // Epilogue staging: each MMA wave writes 32 accumulator rows x TN
    // columns of f32 to its own LDS region; the MMA wave and its first
    // loader partner then read half the rows each as row-contiguous float4. Row
    // stride EPS = TN + 8 floats puts the two half-waves (rows r and r+4) on
    // disjoint banks.
    constexpr int EPS = TN + 8;
    constexpr int LANES_PER_ROW = TN / 4;
    constexpr int ROWS_PER_READ = 64 / LANES_PER_ROW;
    constexpr int RPT = 16 / ROWS_PER_READ;  // row reads per strip per wave
    constexpr int LOOP_BYTES = 2 * (BM + BN) * LDK * 2;
    constexpr int EPI_BYTES = NW * 32 * EPS * 4;
    constexpr int RED_BYTES = DOT ? 2 * WM * BN * 4 : 0;
    constexpr int SMEM = LOOP_BYTES > EPI_BYTES + RED_BYTES ? LOOP_BYTES : EPI_BYTES + RED_BYTES;
    static_assert(64 % LANES_PER_ROW == 0 && 16 % ROWS_PER_READ == 0, "epilogue read shape");

    __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
    _Float16 *As0 = reinterpret_cast<_Float16 *>(smem);
    _Float16 *Bs0 = reinterpret_cast<_Float16 *>(smem + 2 * BM * LDK * 2);
#define BLR_AS(buf) (As0 + (buf) * (BM * LDK))
#define BLR_BS(buf) (Bs0 + (buf) * (BN * LDK))

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave: roles branch on scalars
    const bool loader = wave >= NW;
    const bool partner = loader && wave < 2 * NW;  // loader wave sharing an MMA wave's epilogue rows
    const int rw = loader ? (wave - NW) % NW : wave;  // MMA wave index (a loader's partner)
    const int wm = rw / WN, wn = rw % WN;
    const int N = p.N, K = p.K;
    const int ntn = N / BN;
    const int L = blockIdx.x, G = gridDim.x;
    const int T = (G % NUM_XCD == 0) ? (L % NUM_XCD) * (G / NUM_XCD) + L / NUM_XCD : L;
    // Within an XCD's run of tiles, GM consecutive M tiles share an N tile:
    // the workgroups resident at one time then read a few activation
    // row-blocks and a few plane slices, which fit in the XCD's L2. GM = 1
    // walks the N tiles of one M tile first.
    int mt, nt;
    if (GM == 1) {
        mt = T / ntn;
        nt = T - mt * ntn;
    } else {
        const int mtiles = (int)((p.M + BM - 1) / BM);
        const int grp = T / (GM * ntn), within = T - grp * (GM * ntn);
        const int gsz = (grp + 1) * GM <= mtiles ? GM : mtiles - grp * GM;
        mt = grp * GM + within % gsz;
        nt = within / gsz;
    }
    const int n0 = nt * BN;
    const int64_t m0 = (int64_t)mt * BM;
    const int nk = K / BK;  // a multiple of P (the launcher checks)
    const int64_t M = p.M;

    // Loader operand addressing: a uniform base advanced by the stage, plus
    // a fixed 32-bit byte offset per thread (every operand is below 4 GiB,
    // checked by the caller). Rows past M read row M-1 instead: a row of the
    // product depends on its own A row only, and those rows are never stored
    // or summed.
    const int lt = loader ? tid - NW * 64 : 0;  // loader thread index
    const int c4 = lt % (BK / 4);
    const int arow = lt / (BK / 4);
    uint32_t aoff[A_PER];
#pragma unroll
    for (int v = 0; v < A_PER; ++v) {
        int64_t gm = m0 + arow + v * AROW_STEP;
        gm = gm < M ? gm : M - 1;
        aoff[v] = (uint32_t)((gm * p.lda + c4 * 4) * 4);
    }
    // B unit of this loader thread: plane row brow, signs bpart*UB ..
    // bpart*UB + UB-1 of the K step's word
    const int brow = lt / (32 / UB), bpart = lt % (32 / UB);
    const uint32_t boff = (uint32_t)((int64_t)(n0 + brow) * (K / 32) * 4);
    const int bofs = brow * LDK + bpart * UB;
    const int bsh = bpart * UB;
    // f16 sign patterns held in VGPRs so the decode's and-or is one VOP3
    uint32_t sgnmask, one16;
    asm volatile("v_mov_b32 %0, 0x80008000" : "=v"(sgnmask));
    asm volatile("v_mov_b32 %0, 0x3c003c00" : "=v"(one16));
    const unsigned char *Abytes = reinterpret_cast<const unsigned char *>(p.A);
    const unsigned char *Bbytes = reinterpret_cast<const unsigned char *>(p.Bbits);
    const unsigned char *Cbytes = reinterpret_cast<const unsigned char *>(p.colscale) + c4 * 16;

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    f32x4_t ar[P][A_PER];
    f32x4_t cr[P];
    uint32_t br[P];

#define BLR_GLOAD(q, kt)                                                                   \
    do {                                                                                   \
        const unsigned char *a_ = Abytes + (size_t)(kt) * (BK * 4);                        \
        const unsigned char *b_ = Bbytes + (size_t)(kt) * 4;                               \
        _Pragma("unroll") for (int v = 0; v < A_PER; ++v) ar[q][v] =                       \
            *reinterpret_cast<const f32x4_t *>(a_ + aoff[v]);                              \
        cr[q] = *reinterpret_cast<const f32x4_t *>(Cbytes + (size_t)(kt) * (BK * 4));      \
        br[q] = *reinterpret_cast<const uint32_t *>(b_ + boff);                            \
    } while (0)

#define BLR_SSTORE(q, buf)                                                                 \
    do {                                                                                   \
        const f32x4_t cs_ = cr[q] * p.ascale;                                              \
        _Pragma("unroll") for (int v = 0; v < A_PER; ++v) {                                \
            half4_t hv;                                                                    \
            hv[0] = (_Float16)(ar[q][v].x * cs_.x);                                        \
            hv[1] = (_Float16)(ar[q][v].y * cs_.y);                                        \
            hv[2] = (_Float16)(ar[q][v].z * cs_.z);                                        \
            hv[3] = (_Float16)(ar[q][v].w * cs_.w);                                        \
            *reinterpret_cast<half4_t *>(BLR_AS(buf) + (arow + v * AROW_STEP) * LDK + c4 * 4) = hv; \
        }                                                                                  \
        {                                                                                  \
            u32x4_t d_[UB / 8];                                                            \
            decode_signs<UB>(br[q] >> bsh, sgnmask, one16, d_);                            \
            u32x4_t *bdst_ = reinterpret_cast<u32x4_t *>(                                  \
                __builtin_assume_aligned(BLR_BS(buf) + bofs, 16));                         \
            _Pragma("unroll") for (int e = 0; e < UB / 8; ++e) bdst_[e] = d_[e];           \
        }                                                                                  \
    } while (0)

#define BLR_COMPUTE(buf)                                                                   \
    do {                                                                                   \
        _Pragma("unroll") for (int s = 0; s < BK / 16; ++s) {                              \
            half8_t af[FM], bf[FN];                                                        \
            _Pragma("unroll") for (int i = 0; i < FM; ++i) af[i] =                         \
                *reinterpret_cast<const half8_t *>(                                        \
                    BLR_AS(buf) + (wm * TM + i * 32 + (lane & 31)) * LDK + s * 16 + (lane >> 5) * 8); \
            _Pragma("unroll") for (int j = 0; j < FN; ++j) bf[j] =                         \
                *reinterpret_cast<const half8_t *>(                                        \
                    BLR_BS(buf) + (wn * TN + j * 32 + (lane & 31)) * LDK + s * 16 + (lane >> 5) * 8); \
            _Pragma("unroll") for (int i = 0; i < FM; ++i)                                 \
                _Pragma("unroll") for (int j = 0; j < FN; ++j) acc[i][j] =                 \
                    __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0); \
        }                                                                                  \
    } while (0)

    // The two roles run separate loops with the same barriers: one per K
    // step. In iteration kt the MMA waves multiply stage kt from LDS buffer
    // kt&1 while the loaders issue stage kt+P into the register set stage kt
    // used and stage kt+1 into the other buffer. The loader loop is
    // unrolled by P so every register-set index is static; its loads are
    // unconditional (stages past the end re-read the last stage and are
    // never multiplied), so the compiler counts outstanding loads exactly and
    // waits only for the stage it converts.
    if (loader) {
#pragma unroll
        for (int q = 0; q < P; ++q) BLR_GLOAD(q, q);
        BLR_SSTORE(0, 0);
        __syncthreads();
        for (int kt0 = 0; kt0 < nk; kt0 += P) {
#pragma unroll
            for (int q = 0; q < P; ++q) {
                const int kt = kt0 + q;
                BLR_GLOAD(q, kt + P < nk ? kt + P : nk - 1);
                BLR_SSTORE((q + 1) % P, (q + 1) & 1);
                __syncthreads();
                // keep the next stages' conversions out of this iteration:
                // hoisted above the barrier they would wait for loads just issued
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else {
        __syncthreads();
        for (int kt0 = 0; kt0 < nk; kt0 += P) {
#pragma unroll
            for (int q = 0; q < P; ++q) {
                BLR_COMPUTE(q & 1);
                __syncthreads();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
#undef BLR_GLOAD
#undef BLR_SSTORE
#undef BLR_COMPUTE
#undef BLR_AS
#undef BLR_BS

    // Epilogue, one 32-row strip of the MMA wave tiles at a time: the MMA
    // waves stage their accumulators through LDS, then every wave handles
    // float4 column groups of 16 whole rows (MMA wave: rows 0-15 of its
    // strip, loader partner: rows 16-31): products, tapes, scaled outputs
    // and column partials.
    const float *stage = reinterpret_cast<const float *>(smem) + rw * 32 * EPS;
    const bool epi = !loader || partner;  // waves that read back and store
    const int lr0 = (loader ? 16 : 0) + lane / LANES_PER_ROW;
    const int lc = (lane % LANES_PER_ROW) * 4;
    const int gn = n0 + wn * TN + lc;
    const bool full = m0 + BM <= M;
    f32x4_t c2 = {0.f, 0.f, 0.f, 0.f};
    if (OUT2) c2 = *reinterpret_cast<const f32x4_t *>(p.out2col + gn);
    // The column-sum operand streams from HBM once: issue every load of this
    // lane's rows now (rows past M read row M-1 and are not used), so their
    // latencies overlap instead of following one another.
    f32x4_t pre[DOT ? FM : 1][DOT ? RPT : 1];
    if (DOT && epi) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int it = 0; it < RPT; ++it) {
                int64_t gm = m0 + wm * TM + i * 32 + it * ROWS_PER_READ + lr0;
                gm = gm < M ? gm : M - 1;
                pre[i][it] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p.dot_other + gm * N + gn));
            }
    }
    f32x4_t dsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        f32x4_t old[OUT2 ? RPT : 1];
        if (OUT2 && p.out2acc && epi) {
#pragma unroll
            for (int it = 0; it < RPT; ++it) {
                int64_t gm = m0 + wm * TM + i * 32 + it * ROWS_PER_READ + lr0;
                gm = gm < M ? gm : M - 1;
                old[it] = *reinterpret_cast<const f32x4_t *>(p.out2 + gm * N + gn);
            }
        }
        if (!loader) {
            float *st = reinterpret_cast<float *>(smem) + rw * 32 * EPS;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    st[(8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * EPS + j * 32 + (lane & 31)] = acc[i][j][v];
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < RPT; ++it) {
            if (!epi) break;
            const int lr = it * ROWS_PER_READ + lr0;
            const int64_t gm = m0 + wm * TM + i * 32 + lr;
            f32x4_t val = *reinterpret_cast<const f32x4_t *>(stage + lr * EPS + lc);
            val *= p.oscale;
            if (full || gm < M) {
                const int64_t o = gm * N + gn;
                if (OUT) *reinterpret_cast<f32x4_t *>(p.out + o) = val;
                if (OUT2) {
                    f32x4_t y = val * c2;
                    if (p.out2acc) y = old[it] + y;
                    *reinterpret_cast<f32x4_t *>(p.out2 + o) = y;
                }
                if (DOT) dsum += val * pre[i][it];
            }
        }
        __syncthreads();
    }
    if (DOT) {
        // lanes with the same columns (l mod LANES_PER_ROW) fold in a fixed
        // butterfly; then the 2*WM waves of a column strip (MMA waves first,
        // then loaders, each in row order) add in that order
#pragma unroll
        for (int off = LANES_PER_ROW; off < 64; off <<= 1) {
            dsum.x += __shfl_xor(dsum.x, off);
            dsum.y += __shfl_xor(dsum.y, off);
            dsum.z += __shfl_xor(dsum.z, off);
            dsum.w += __shfl_xor(dsum.w, off);
        }
        float *red = reinterpret_cast<float *>(smem + EPI_BYTES);  // [2*WM][BN]
        const int rrow = (loader ? WM : 0) + wm;
        if (epi && lane < LANES_PER_ROW) *reinterpret_cast<f32x4_t *>(red + rrow * BN + wn * TN + lc) = dsum;
        __syncthreads();
        for (int c = tid; c < BN; c += (1 + LW) * NW * 64) {
            float sum = 0.0f;
#pragma unroll
            for (int w = 0; w < 2 * WM; ++w) sum += red[w * BN + c];
            p.dot_partial[(int64_t)mt * N + n0 + c] = sum;
        }
    }
}

template <int BM, int BN, int BK, int WM, int WN, int LW, int P, bool OUT, bool OUT2, bool DOT, int GM>
static hipError_t launch_gemm_t(int id, const GemmArgs &a, hipStream_t s) {
    if (a.N % BN != 0 || a.K % (BK * P) != 0 || a.K / BK < P) return hipErrorInvalidValue;
    const int64_t tiles = (int64_t)(a.N / BN) * ((a.M + BM - 1) / BM);
    prof_begin(id, s);
    hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, WM, WN, LW, P, OUT, OUT2, DOT, GM>), dim3((unsigned)tiles),
                       dim3((1 + LW) * WM * WN * 64), 0, s, a);
    hipError_t e = hipGetLastError();
    prof_end(s);
    return e;
}

// Tile shapes per kind: 128x128 tiles of 2x2 MMA waves (64x64 each) plus 4
// loader waves; F2/B2/DH (N = d_out or d_in, K = r) walk groups of 8 M
// tiles per N tile.
int gemm_tile_rows(GemmKind) { return 128; }

hipError_t launch_gemm(GemmKind kind, const GemmArgs &a, hipStream_t s) {
    switch (kind) {
        case GEMM_F1: return launch_gemm_t<128, 128, 32, 2, 2, 1, 4, true, false, false, 1>(K_GEMM_F1, a, s);
        case GEMM_F2: return launch_gemm_t<128, 128, 32, 2, 2, 1, 4, true, true, false, 8>(K_GEMM_F2, a, s);
        case GEMM_F2_NOTAPE: return launch_gemm_t<128, 128, 32, 2, 2, 1, 4, false, true, false, 8>(K_GEMM_F2, a, s);
        case GEMM_DH: return launch_gemm_t<128, 128, 32, 2, 2, 1, 4, false, false, true, 8>(K_GEMM_DH, a, s);
        case GEMM_B1: return launch_gemm_t<128, 128, 32, 2, 2, 2, 4, true, false, true, 1>(K_GEMM_B1, a, s);
        case GEMM_B2: return launch_gemm_t<128, 128, 32, 2, 2, 2, 4, false, true, true, 8>(K_GEMM_B2, a, s);
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Column reduction (page: `colsum_prod`, one thread per column with a serial
// row loop, later two-pass): here each thread owns 4 adjacent columns
// (float4, so a wavefront reads 1 KB contiguous per row) over COLSUM_ROWS
// tokens, 8 rows per step (16 loads in flight); partial[chunk][col] is
// summed in chunk order by finish_kernel.
__global__ __launch_bounds__(256) void colsum_prod_kernel(const float *__restrict__ A, const float *__restrict__ B,
                                                          int64_t M, int N, float *__restrict__ partial) {
    const int col = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (col >= N) return;
    const int64_t t0 = (int64_t)blockIdx.y * COLSUM_ROWS;
    const int64_t t1 = t0 + COLSUM_ROWS < M ? t0 + COLSUM_ROWS : M;
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
    int64_t t = t0;
    for (; t + 8 <= t1; t += 8) {
        f32x4_t a[8], b[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            a[u] = *reinterpret_cast<const f32x4_t *>(A + (t + u) * N + col);
            b[u] = *reinterpret_cast<const f32x4_t *>(B + (t + u) * N + col);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) s += a[u] * b[u];
    }
    for (; t < t1; ++t)
        s += *reinterpret_cast<const f32x4_t *>(A + t * N + col) * *reinterpret_cast<const f32x4_t *>(B + t * N + col);
    *reinterpret_cast<f32x4_t *>(partial + (int64_t)blockIdx.y * N + col) = s;
}

hipError_t launch_colsum(const float *A, const float *B, int64_t M, int N, float *partial, hipStream_t s) {
    dim3 grid((unsigned)((N + 1023) / 1024), (unsigned)((M + COLSUM_ROWS - 1) / COLSUM_ROWS));
    prof_begin(K_COLSUM, s);
    hipLaunchKernelGGL(colsum_prod_kernel, grid, dim3(256), 0, s, A, B, M, N, partial);
    hipError_t e = hipGetLastError();
    prof_end(s);
    return e;
}

// out[n] += sum over parts of partial[part][n], for up to three vectors in
// one launch (each workgroup owns 64 columns of one job; its 4 waves take
// every 4th part in order, then the 4 wave sums are added in wave order: a
// fixed order, so results are deterministic).
__global__ __launch_bounds__(256) void finish_kernel(FinishJobs jobs) {
    __shared__ float red[4][64];
    int b = blockIdx.x, j = 0;
    while (j + 1 < jobs.count && b >= jobs.blocks_before[j + 1]) ++j;
    const FinishJob &jb = jobs.job[j];
    const float *__restrict__ partial = jb.partial;
    const int64_t nparts = jb.nparts;
    const int N = jb.N;
    const int c = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int col = (b - jobs.blocks_before[j]) * 64 + c;
    float s = 0.0f;
    if (col < N) {
        int64_t pi = q;
        for (; pi + 12 < nparts; pi += 16) {
            const float v0 = partial[pi * N + col], v1 = partial[(pi + 4) * N + col];
            const float v2 = partial[(pi + 8) * N + col], v3 = partial[(pi + 12) * N + col];
            s += v0;
            s += v1;
            s += v2;
            s += v3;
        }
        for (; pi < nparts; pi += 4) s += partial[pi * N + col];
    }
    red[q][c] = s;
    __syncthreads();
    if (q == 0 && col < N) jb.out[col] = jb.out[col] + (((red[0][c] + red[1][c]) + red[2][c]) + red[3][c]);
}

hipError_t launch_finish(FinishJobs jobs, hipStream_t s) {
    int total = 0;
    for (int j = 0; j < jobs.count; ++j) {
        jobs.blocks_before[j] = total;
        total += (jobs.job[j].N + 63) / 64;
    }
    prof_begin(K_FINISH, s);
    hipLaunchKernelGGL(finish_kernel, dim3((unsigned)total), dim3(256), 0, s, jobs);
    hipError_t e = hipGetLastError();
    prof_end(s);
    return e;
}

const char *kernel_name(int id) {
    switch (id) {
        case K_EXPAND: return "expand_signs";
        case K_TRANSPOSE: return "transpose_bits";
        case K_GEMM_F1: return "gemm_f1_xg_sv";
        case K_GEMM_F2: return "gemm_f2_al_sut";
        case K_GEMM_B1: return "gemm_b1_dyh_su";
        case K_GEMM_B2: return "gemm_b2_dbl_svt";
        case K_COLSUM: return "colsum_dy_c";
        case K_GEMM_DH: return "gemm_dh_recompute_c";
        case K_FINISH: return "colsum_finish";
    }
    return "?";
}

}  // namespace blr
