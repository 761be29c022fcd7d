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
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

// f16 bit pattern of -1 (+1 is the same with the sign bit clear).
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
// S is the +-1 plane [N][K], read as its bitmap (a u32 holds 32 k of a
// plane row) and decoded to f16 in registers: the page's expanded f16
// planes are never materialised. ascale is a power of two, so folding it
// into colscale is exact except where an f32 intermediate would overflow.
//
// A workgroup of WM x WN waves computes a BM x BN tile; each wave owns a
// TM x TN block of it. Per K step (BK = 64 for the plain kinds, 32 for the
// fused dh launch and the 128-row tiles):
//  - activation: every thread keeps P stages of float4 loads in flight in a
//    register ring (16 threads per row at K steps of 64, so one wave load
//    covers 4 whole 256-byte row segments). A stage is scaled and rounded to
//    f16 (a multiply and a packed conversion per pair of elements) and
//    written to a 3-deep LDS ring two steps before it is used;
//  - each wave reads the next step's A fragments from LDS while this
//    step's MFMAs (v_mfma_f32_32x32x16_f16, f32 accumulators) run; one
//    barrier per step;
//  - sign operand: each wave decodes its own B fragments from the bitmap
//    words (fetched as 16-byte groups of 128 k, one group ahead) straight
//    into registers; it never passes through LDS;
//  - epilogue straight from the accumulators: for a fixed accumulator
//    register the 64 lanes hold 2 rows x 32 consecutive columns, so every
//    store instruction writes two whole 128-byte lines.
//
// Tile order: workgroups are dealt round-robin to the 8 XCDs, each with its
// own L2. The launch index is remapped so that tiles sharing operands run
// on the same XCD (see GM below).
//
// MFMA 32x32x16 operand layout: lane l supplies row (l % 32) of A and column
// (l % 32) of B, each with the 8 consecutive k of group (l / 32) in each 16-k
// block. The accumulator register v of lane l holds row
// 8*(v/4) + 4*(l/32) + v%4, column l % 32.
constexpr int NUM_XCD = 8;

// Two f16 lanes of one dword: f16(a0 * s0), f16(a1 * s1), each product
// rounded to f32 and then to f16 (round to nearest even; f16 subnormals
// kept, overflow gives inf). On gfx950 this is two multiplies and one
// packed conversion, all of which issue while an MFMA runs (a fused
// multiply-and-convert to f16 does not).
// v from the lane that DPP control CTRL selects (quad_perm / row_shl)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t f16x2_scaled(float a0, float s0, float a1, float s1) {
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
    half2_t h;
    h[0] = (_Float16)(a0 * s0);
    h[1] = (_Float16)(a1 * s1);
    return __builtin_bit_cast(uint32_t, h);
}

// Raw buffer access (offset = per-lane VGPR byte offset + uniform byte
// offset, computed by the address unit). The range is the operand's size.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0,
                                             (int)(uint32_t)(bytes < 0xFFFFFFFFull ? bytes : 0xFFFFFFFFull),
                                             0x00020000);
}
__device__ __forceinline__ f32x4_t load_f32x4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ u32x4_t load_u32x4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ u32x2_t load_u32x2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
// streaming (non-temporal) variants: the data is not re-read soon
__device__ __forceinline__ float load_f32_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 2));
}
__device__ __forceinline__ void store_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, soff, 0);
}
__device__ __forceinline__ void store_f32_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, soff, 2);
}

// Signs 2q and 2q+1 of a byte as two f16 values of the NEGATED plane (set
// bit -> -1, clear -> +1). Both 16-bit lanes of y hold the byte; a packed
// shift moves bit 2q (low lane) and bit 2q+1 (high lane) to the lanes' sign
// positions, and the and-or keeps those sign bits over the pattern of +1.
// Decoding -S saves the inversion; the contraction's epilogue multiplies by
// -oscale, which restores the sign exactly (round to nearest even is
// symmetric, so every f32 partial sum is the exact negative).
__device__ __forceinline__ uint32_t sign_dword(uint32_t y, int q, uint32_t sgnmask, uint32_t one16) {
    const u16x2_t sh = {(uint16_t)(15 - 2 * q), (uint16_t)(14 - 2 * q)};
    const u16x2_t t = __builtin_bit_cast(u16x2_t, y) << sh;
    return (__builtin_bit_cast(uint32_t, t) & sgnmask) | one16;
}
// B fragment of -S: the 8 signs of byte `sel & 3` of w (sel replicates that
// byte into all four bytes).
__device__ __forceinline__ half8_t sign_frag(uint32_t w, uint32_t sel, uint32_t sgnmask, uint32_t one16) {
    const uint32_t y = __builtin_amdgcn_perm(w, w, sel);
    u32x4_t d;
    d[0] = sign_dword(y, 0, sgnmask, one16);
    d[1] = sign_dword(y, 1, sgnmask, one16);
    d[2] = sign_dword(y, 2, sgnmask, one16);
    d[3] = sign_dword(y, 3, sgnmask, one16);
    return __builtin_bit_cast(half8_t, d);
}

// B fragment of -S times a column scale: h2 holds the column's f16 scale in
// both halves; the sign bit XORed into it gives -S * scale exactly (one
// v_bitop3 per dword on gfx950)
__device__ __forceinline__ half8_t sign_frag_h(uint32_t w, uint32_t sel, uint32_t sgnmask, uint32_t h2) {
    const uint32_t y = __builtin_amdgcn_perm(w, w, sel);
    u32x4_t d;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const u16x2_t sh = {(uint16_t)(15 - 2 * q), (uint16_t)(14 - 2 * q)};
        const u16x2_t t = __builtin_bit_cast(u16x2_t, y) << sh;
        d[q] = (__builtin_bit_cast(uint32_t, t) & sgnmask) ^ h2;
    }
    return __builtin_bit_cast(half8_t, d);
}

// Bitmap transpose: out [r][rows/32] from bits [rows][r/32]. A wavefront
// takes 64 rows x one word column (32 ranks): lane i loads row i's word, and
// the two 32 x 32 bit blocks (rows 0-31 and 32-63) are transposed across the
// lanes in five swap stages, lanes i and i ^ j exchanging the j x j
// sub-blocks that sit off the diagonal (j = 16, 8, 4, 2, 1). Lane b then
// holds rank 32 w + (b % 32) of its 32 rows, one output word, and lanes b
// and b + 32 store the two adjacent words of that rank. Consecutive waves
// take consecutive word columns of one row block, so a workgroup reads whole
// 64-byte row segments.
__global__ __launch_bounds__(256) void transpose_bits_kernel(const uint32_t *__restrict__ bits, int64_t rows,
                                                             int64_t r, uint32_t *__restrict__ out) {
    const int64_t W = r / 32, rw = rows / 32;
    bits += (int64_t)blockIdx.y * rows * W;  // path blockIdx.y
    out += (int64_t)blockIdx.y * r * rw;
    const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // one wavefront per (row block, word)
    const int lane = threadIdx.x & 63;
    const int64_t nrb = (rows + 63) / 64;
    if (wid >= nrb * W) return;  // uniform per wavefront
    const int64_t rb = wid / W, w = wid % W;
    const int64_t row = rb * 64 + lane;
    uint32_t a = row < rows ? bits[row * W + w] : 0u;
    const uint32_t masks[5] = {0x0000FFFFu, 0x00FF00FFu, 0x0F0F0F0Fu, 0x33333333u, 0x55555555u};
#pragma unroll
    for (int st = 0; st < 5; ++st) {
        const int j = 16 >> st;
        const uint32_t pv = (uint32_t)__shfl_xor((int)a, j);  // j < 32: within the lane's half
        const bool up = (lane & j) != 0;
        const uint32_t hi = up ? a : pv, lo = up ? pv : a;
        const uint32_t t = ((lo >> j) ^ hi) & masks[st];
        a ^= up ? t : (t << j);
    }
    // lane: rank 32 w + lane % 32, bit i = row 64 rb + 32 (lane / 32) + i
    const int64_t ow = rb * 2 + (lane >> 5);
    if (ow < rw) out[(w * 32 + (lane & 31)) * rw + ow] = a;
}

hipError_t launch_transpose_bits(const uint32_t *bits, int64_t rows, int64_t r, uint32_t *out, hipStream_t s,
                                 int paths) {
    const int64_t waves = ((rows + 63) / 64) * (r / 32);
    prof_begin(K_TRANSPOSE, s);
    hipLaunchKernelGGL(transpose_bits_kernel, dim3((unsigned)((waves + 3) / 4), (unsigned)paths), dim3(256), 0, s,
                       bits, rows, r, out);
    hipError_t e = hipGetLastError();
    prof_end(s);
    return e;
}

template <int BM, int BN, int WM, int WN, int P, int MINB, bool OUT, bool OUT2, bool DOT, int GM, bool FDH = false,
          int KB = 2, bool PLANE = false, bool MP = false>
__global__ __launch_bounds__((FDH ? 2 : 1) * WM * WN * 64, MINB) void gemm_kernel(GemmArgs p) {
    constexpr int NT = WM * WN * 64;  // threads of the contraction role
    constexpr int BK = 16 * KB;     // k per step: KB MFMA k-blocks, KB/2 bitmap words per plane row
    constexpr int U = 8 / KB;       // steps per group of 4 bitmap words (the loop unroll)
    // halves per LDS row of the f16 activation tile. At BK = 64 a pad of 8
    // makes the stagers' 8-byte writes and the fragments' 16-byte reads
    // conflict-free; at BK = 32 (8 threads a row) no pitch does both, so the
    // rows are unpadded and a row's 16-byte chunks are permuted: chunk c of
    // row m sits at chunk c ^ ((m >> 2) & 3) (both conflict-free on gfx950,
    // measured)
    constexpr bool ASW = BK == 32;
    constexpr int LDK = ASW ? BK : BK + 8;
    constexpr int NS = 3;           // LDS ring depth
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int TPR = BK / 4;     // threads per activation row, one float4 each
    constexpr int RPP = NT / TPR;   // activation rows per pass
    constexpr int PER = BM / RPP;   // float4 per thread per stage
    static_assert(TM % 32 == 0 && TN % 32 == 0 && BM % RPP == 0 && PER >= 1, "tile shape");
    static_assert((KB == 2 || KB == 4) && (2 * U) % P == 0, "the register ring must divide the unroll");
    static_assert(!FDH || KB == 2, "fused dh walks 32-column steps");
    // PLANE (dense frozen linear): the B fragments are read from an f16
    // plane [N][K] (one 16-byte load per lane and k-block, one step ahead)
    // instead of decoded from a bitmap, and the activation has no column scale.
    static_assert(!PLANE || (!FDH && !DOT), "plane path shape");
    // MP (paths along K): per-path flushes of the product; the column
    // partials need every row of a column in one wave
    static_assert(!MP || (WM == 1 && !OUT && !FDH && !PLANE), "paths along K");
    // Fused dh (B1 only): 64-token tiles, one row of waves with 64 ranks
    // each, and as many more waves in a second role (DH waves) that compute
    // the dh partials from an f32 copy of the dy tile the B1 waves also
    // stage, so each SIMD holds one wave of each role and one's VALU work
    // overlaps the other's MFMAs.
    static_assert(!FDH || (WM == 1 && BM == 64 && TN == 64 && BK == 32 && DOT && OUT), "fused dh shape");
    constexpr int FMD = BM / 32;    // fused dh: row blocks of the recomputed c
    constexpr int KD = TN / 16;     // fused dh: MFMA k-blocks over the wave's ranks (FMD * KD = 8)
    constexpr int CP = 2 / FMD;     // fused dh: accumulators per row block (two MFMA chains in flight)
    // fused dh: floats per column of the transposed f32 dy tile; element
    // (column c, row m) sits at c * LDR + (m ^ 4 * ((c >> 2) & 7)). With this
    // pitch and swizzle neither the stagers' 4-byte writes (a float4 of a row
    // per lane) nor the DH waves' 16-byte reads (4 rows of a column per lane)
    // meet a bank conflict on gfx950 (measured)
    constexpr int LDR = BM + 16;

    __shared__ __attribute__((aligned(16))) _Float16 As[NS * BM * LDK];
    // column partials (DOT) have one row per 64 tokens: a 128-row tile
    // (one row of waves, each with all 128 rows of its columns) writes two
    constexpr int HR = BM / 64;
    static_assert(BM == 64 || (BM == 128 && WM == 1 && !FDH && !MP), "128-row tiles: one row of waves");
    __shared__ float red[DOT ? HR * WM * BN : 1];
    constexpr int NSD = 4;          // fused dh: depth of the dy ring (a step's dot runs one step late)
    __shared__ __attribute__((aligned(16))) float dyT[FDH ? NSD * 32 * LDR : 1];  // [buf][column][row]
    __shared__ float redh[FDH ? 2 * WN * 64 : 1];                                // [step & 1][wave][lane]
    // fused dh: the tile's f32 a block, as the DH waves load it, for the B1
    // waves' epilogue (the dl partials); the pad of 8 keeps both sides'
    // accesses free of bank conflicts
    constexpr int LDA_ = BN + 8;
    __shared__ __attribute__((aligned(16))) float aL[FDH ? BM * LDA_ : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool dhw = FDH && wave >= WM * WN;         // DH-role wave (uniform)
    const int rwave = dhw ? wave - WM * WN : wave;   // index within the role
    const int wm = rwave / WN, wn = rwave % WN;
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
    const int nk = K / BK;  // a multiple of U (K is a multiple of 128)
    const int64_t M = p.M;

    // Activation addressing: a uniform base advanced by the stage, plus a
    // fixed 32-bit byte offset per thread (every operand is below 4 GiB,
    // checked by the caller). Rows past M read row M-1 instead: a row of the
    // product depends on its own A row only, and those rows are never stored
    // or summed.
    const int st = dhw ? tid - NT : tid;  // staging thread index within the role
    const int c4 = st % TPR, arow = st / TPR;
    uint32_t aoff[PER];
#pragma unroll
    for (int v = 0; v < PER; ++v) {
        int64_t gm = m0 + arow + v * RPP;
        gm = gm < M ? gm : M - 1;
        aoff[v] = (uint32_t)((gm * p.lda + c4 * 4) * 4);
    }
    // Buffer resources: every operand below 4 GiB (checked by the caller);
    // the loads take a 32-bit per-lane offset plus a uniform offset, so no
    // VALU address arithmetic is needed.
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A, (uint64_t)M * p.lda * 4);
    // paths: along N, this tile's path pn; along K, PKr ranks per path
    const int pn = p.path_n ? n0 / p.path_n : 0;
    const int PKr = p.path_k ? p.path_k : K;
    const __amdgpu_buffer_rsrc_t rC =
        make_rsrc(p.colscale + (int64_t)pn * p.cs_pstride, PLANE ? 0 : (uint64_t)K * 4);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.Bbits, PLANE ? 0 : (uint64_t)N * K / 8);
    const __amdgpu_buffer_rsrc_t rP = make_rsrc(p.Bplane, PLANE ? (uint64_t)N * K * 2 : 0);
    const uint32_t coff = (uint32_t)c4 * 16;
    // LDS write (halves); rows arow + v RPP share the permutation (RPP is a
    // multiple of 16 wherever BK = 32)
    const int wofs = arow * LDK + (ASW ? 8 * ((c4 >> 1) ^ ((arow >> 2) & 3)) + 4 * (c4 & 1) : c4 * 4);
    // fragment reads (halves) of k-block s: 8 halves at k = 8 (lane / 32) + 16 s
    const int rrow_ = wm * TM + (lane & 31);
    const int rofs = rrow_ * LDK + (ASW ? 8 * ((lane >> 5) ^ ((rrow_ >> 2) & 3)) : (lane >> 5) * 8);
    const int rofs1 = rrow_ * LDK + (ASW ? 8 * (((lane >> 5) + 2) ^ ((rrow_ >> 2) & 3)) : (lane >> 5) * 8 + 16);
    static_assert(!ASW || (RPP % 16 == 0 && KB == 2), "permuted activation tile");
    // Bitmap words of this lane's plane rows (one per 32-column block)
    uint32_t boff[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j)
        boff[j] = PLANE ? (uint32_t)(((int64_t)(n0 + wn * TN + j * 32 + (lane & 31)) * K + (lane >> 5) * 8) * 2)
                        : (uint32_t)((int64_t)(n0 + wn * TN + j * 32 + (lane & 31)) * (PKr / 32) * 4);
    // v_perm selectors: byte (2s + lane group) of the word into every byte
    const uint32_t grp = (uint32_t)(lane >> 5);
    const uint32_t sel[2] = {grp * 0x01010101u, (2u + grp) * 0x01010101u};
    // f16 sign patterns held in VGPRs so the decode's and-or is one VOP3
    uint32_t sgnmask, one16;
    asm volatile("v_mov_b32 %0, 0x80008000" : "=v"(sgnmask));
    asm volatile("v_mov_b32 %0, 0x3c003c00" : "=v"(one16));

    // Fused dh: the wave's A fragments f16(a * l) (row block i, k-block t
    // of its ranks at al[i * KD + t]) stay in registers (rows past M are
    // zero, so they add nothing to dh), and each step reads the bitmap words
    // of S_U rows i0 + (lane % 32), ranks of the wave: two words, one
    // 8-byte load.
    half8_t al[FDH ? FMD * KD : 1];
    uint32_t hoff = 0;
    // (paths along N: path pn's S_U, DRW words per row)
    const int DRW = p.dh_row_words ? p.dh_row_words : N / 32;
    const __amdgpu_buffer_rsrc_t rH =
        make_rsrc(p.dh_bits + (int64_t)pn * p.dh_pstride, FDH ? (uint64_t)K * DRW * 4 : 0);
    if (dhw) {
#pragma unroll
        for (int i = 0; i < FMD; ++i) {
            const int64_t gm = m0 + 32 * i + (lane & 31);
            const bool inr = gm < M;
            const float *ar_ = p.dh_a + (inr ? gm : 0) * N;
#pragma unroll
            for (int t = 0; t < KD; ++t) {
                const int k = n0 + wn * TN + 16 * t + 8 * (lane >> 5);
                const f32x4_t x0 = *reinterpret_cast<const f32x4_t *>(ar_ + k);
                const f32x4_t x1 = *reinterpret_cast<const f32x4_t *>(ar_ + k + 4);
                const f32x4_t l0 = *reinterpret_cast<const f32x4_t *>(p.dh_l + k);
                const f32x4_t l1 = *reinterpret_cast<const f32x4_t *>(p.dh_l + k + 4);
                half8_t h;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[e] = inr ? (_Float16)(x0[e] * l0[e]) : (_Float16)0.0f;
                    h[4 + e] = inr ? (_Float16)(x1[e] * l1[e]) : (_Float16)0.0f;
                }
                al[i * KD + t] = h;
                if (FDH) {
                    float *d_ = aL + (32 * i + (lane & 31)) * LDA_ + (k - n0);
                    const f32x4_t z_ = {0.0f, 0.0f, 0.0f, 0.0f};
                    *reinterpret_cast<f32x4_t *>(d_) = inr ? x0 : z_;
                    *reinterpret_cast<f32x4_t *>(d_ + 4) = inr ? x1 : z_;
                }
            }
        }
        hoff = (uint32_t)(((lane & 31) * DRW + (n0 - pn * p.path_n + wn * TN) / 32) * 4);
    }

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    f32x4_t ar[P][PER];
    f32x4_t cr[P];
    u32x4_t bq[FN], bn[FN];  // bitmap words: this 4-step group, the next
    half8_t fa[FM][KB], fb[FN][KB];
    half8_t fa2[FM][KB], fb2[FN][KB];

#define BLR_GLOAD(q, kt)                                                                   \
    do {                                                                                   \
        const int k_ = (kt) < nk ? (kt) : nk - 1;                                          \
        if (!dhw) {                                                                        \
            _Pragma("unroll") for (int v = 0; v < PER; ++v) ar[q][v] =                     \
                load_f32x4(rA, aoff[v], (uint32_t)k_ * (BK * 4));                          \
            if (!PLANE) cr[q] = load_f32x4(rC, coff, (uint32_t)k_ * (BK * 4));             \
        }                                                                                  \
    } while (0)

#define BLR_BLOAD(dst, grp4)                                                               \
    do {                                                                                   \
        const int g_ = (grp4) < nk / U ? (grp4) : nk / U - 1;                              \
        /* group g_ (128 k) lies in path g_ * 128 / PKr */                                 \
        const int pq_ = g_ * 128 / PKr;                                                    \
        const uint32_t so_ = (uint32_t)((int64_t)pq_ * p.b_pstride * 4) + (uint32_t)(g_ - pq_ * (PKr / 128)) * 16; \
        if (!PLANE) _Pragma("unroll") for (int j = 0; j < FN; ++j) dst[j] =                \
            load_u32x4(rB, boff[j], so_);                                                  \
    } while (0)

#define BLR_SSTORE(q, buf, dbuf)                                                           \
    do {                                                                                   \
        if (!dhw) {                                                                        \
            if (FDH) {                                                                     \
                /* for the DH role: the f32 dy tile, transposed, in dy ring slot           \
                   dbuf (rows past M hold row M-1, a finite copy: the recomputed           \
                   c is zero there); the lane's columns 4 c4..4 c4+3 share the row         \
                   swizzle 4 c4 */                                                         \
                _Pragma("unroll") for (int v = 0; v < PER; ++v) {                          \
                    float *dt_ = dyT + (dbuf) * (32 * LDR) + ((arow + v * RPP) ^ (4 * c4)); \
                    _Pragma("unroll") for (int e = 0; e < 4; ++e) dt_[(4 * c4 + e) * LDR] = ar[q][v][e]; \
                }                                                                          \
            }                                                                              \
            const f32x4_t cs_ = PLANE ? f32x4_t{p.ascale, p.ascale, p.ascale, p.ascale}    \
                                      : cr[q] * p.ascale;                                  \
            _Float16 *dst_ = As + (buf) * (BM * LDK) + wofs;                               \
            _Pragma("unroll") for (int v = 0; v < PER; ++v) {                              \
                uint2 h_;                                                                  \
                h_.x = f16x2_scaled(ar[q][v].x, cs_.x, ar[q][v].y, cs_.y);                 \
                h_.y = f16x2_scaled(ar[q][v].z, cs_.z, ar[q][v].w, cs_.w);                 \
                *reinterpret_cast<uint2 *>(dst_ + v * RPP * LDK) = h_;                      \
            }                                                                              \
        }                                                                                  \
    } while (0)

#define BLR_AFRAG(dst, buf)                                                                \
    do {                                                                                   \
        const _Float16 *src_ = As + (buf) * (BM * LDK);                                    \
        _Pragma("unroll") for (int i = 0; i < FM; ++i)                                     \
            _Pragma("unroll") for (int s = 0; s < KB; ++s) dst[i][s] =                     \
                *reinterpret_cast<const half8_t *>(src_ + i * 32 * LDK +                   \
                                                   (s == 0 ? rofs : s == 1 ? rofs1 : rofs + s * 16)); \
    } while (0)

#define BLR_BFRAG(dst, words, u, kstep)                                                    \
    do {                                                                                   \
        const int kp_ = (kstep) < nk ? (kstep) : nk - 1;                                   \
        _Pragma("unroll") for (int j = 0; j < FN; ++j)                                     \
            _Pragma("unroll") for (int s = 0; s < KB; ++s) dst[j][s] = PLANE ?             \
                __builtin_bit_cast(half8_t, load_u32x4(rP, boff[j], (uint32_t)(kp_ * BK + s * 16) * 2)) : \
                sign_frag(words[j][(u) * (KB / 2) + s / 2], sel[s % 2], sgnmask, one16);   \
    } while (0)

#define BLR_MMA(a_, b_)                                                                    \
    do {                                                                                   \
        _Pragma("unroll") for (int s = 0; s < KB; ++s)                                     \
            _Pragma("unroll") for (int i = 0; i < FM; ++i)                                 \
                _Pragma("unroll") for (int j = 0; j < FN; ++j) acc[i][j] =                 \
                    __builtin_amdgcn_mfma_f32_32x32x16_f16(a_[i][s], b_[j][s], acc[i][j], 0, 0, 0); \
    } while (0)

    // Fused dh, step kt (columns i0 = 32 kt of d_out): the wave's partial
    // c over its ranks (8 MFMAs), times the f32 dy of the step, summed over
    // the lane's rows; every lane's sum goes to redh, and after the step's
    // barrier the first DH wave adds them in wave and lane-group order (dh
    // is linear in c, so per-wave partial c suffice). The role
    // is software-pipelined: iteration kt issues the MFMAs of step kt,
    // decodes the signs of step kt+1 and forms the dot of step kt-1, so the
    // VALU work runs beside the MFMAs and no MFMA result is waited for.
#define BLR_DH_DECODE(BF, HB)                                                              \
    do {                                                                                   \
        _Pragma("unroll") for (int t = 0; t < KD; ++t)                                     \
            BF[t] = sign_frag(HB[t / 2], sel[t % 2], sgnmask, one16);                      \
    } while (0)
#define BLR_DH_MMA(CC, BF)                                                                 \
    do {                                                                                   \
        _Pragma("unroll") for (int i = 0; i < FMD; ++i)                                    \
            _Pragma("unroll") for (int q = 0; q < CP; ++q)                                 \
                _Pragma("unroll") for (int v = 0; v < 16; ++v) CC[i][q][v] = 0.0f;         \
        _Pragma("unroll") for (int t = 0; t < KD; ++t)                                     \
            _Pragma("unroll") for (int i = 0; i < FMD; ++i) CC[i][t % CP] =                \
                __builtin_amdgcn_mfma_f32_32x32x16_f16(al[i * KD + t], BF[t], CC[i][t % CP], 0, 0, 0); \
    } while (0)
#define BLR_DH_DYLOAD(D4, BUF)                                                             \
    do {                                                                                   \
        _Pragma("unroll") for (int i = 0; i < FMD; ++i)                                    \
            _Pragma("unroll") for (int q = 0; q < 4; ++q) D4[i][q] =                       \
                *reinterpret_cast<const f32x4_t *>(dyT + (BUF) * (32 * LDR) + (lane & 31) * LDR + \
                                                   32 * i + ((4 * (lane >> 5) + 8 * q) ^ (4 * ((lane >> 2) & 7)))); \
    } while (0)
#define BLR_DH_DOT(CC, D4, KT)                                                             \
    do {                                                                                   \
        float dq_[4] = {0.0f, 0.0f, 0.0f, 0.0f}; /* four independent chains */            \
        _Pragma("unroll") for (int i = 0; i < FMD; ++i)                                    \
            _Pragma("unroll") for (int q = 0; q < 4; ++q)                                  \
                _Pragma("unroll") for (int e = 0; e < 4; ++e) {                            \
                    float c_ = CC[i][0][4 * q + e];                                        \
                    _Pragma("unroll") for (int q2 = 1; q2 < CP; ++q2) c_ += CC[i][q2][4 * q + e]; \
                    dq_[q] += c_ * D4[i][q][e];                                            \
                }                                                                          \
        redh[((KT) & 1) * (WN * 64) + wn * 64 + lane] = (dq_[0] + dq_[1]) + (dq_[2] + dq_[3]); \
    } while (0)
    // The dh sums of step KT (after that step's barrier), formed by the B1
    // waves, which would otherwise wait at the barrier: a column's 2 WN
    // partials (WN DH waves, two lane halves each) sit in 2 WN consecutive
    // lanes of one B1 wave (32 / WN columns a wave), which fold them with
    // DPP adds (pairs, then quads, then octets) and store from the first
    // lane; the fragments hold -S, hence the sign. The others' byte offset
    // lies past the partials' buffer range, and the buffer unit drops an
    // out-of-range store.
#define BLR_B1_DHSUM(KT)                                                                   \
    do {                                                                                   \
        constexpr int PW_ = 2 * WN;  /* partials per column */                            \
        const int pi_ = lane % PW_;                                                        \
        float v_ = redh[((KT) & 1) * (WN * 64) + (pi_ >> 1) * 64 + (32 / WN) * rwave + lane / PW_ + 32 * (pi_ & 1)]; \
        v_ += dpp_f32<0xB1>(v_);                    /* lane ^ 1 */                         \
        v_ += dpp_f32<0x4E>(v_);                    /* lane ^ 2 */                         \
        if (PW_ == 8) v_ += dpp_f32<0x104>(v_);     /* lane + 4 (row_shl:4) */             \
        const bool st_ = pi_ == 0 && (KT) >= 0;                                            \
        store_f32(rHP, st_ ? hpoff + (uint32_t)(KT) * 128u : 0xFFFFFF00u, 0u, -v_);        \
    } while (0)

    // Prologue: stages 0 and 1 into LDS buffers 0 and 1, the register ring
    // refilled behind them, the bitmap words of groups 0 and 1, and the
    // fragments of step 0.
    u32x2_t hb[2];               // dh bitmap words (the wave's 64 ranks) of two steps
#define BLR_HLOAD(dst, soff_) dst = load_u32x2(rH, hoff, (soff_))
    // (the DH role's words of steps 0 and 1 go first: the loop then finds
    // as many loads issued after them as in its steady state, and waits for
    // no more than those)
    if (dhw) {
        BLR_HLOAD(hb[0], 0u);
        BLR_HLOAD(hb[1], (uint32_t)(nk > 1 ? 1 : 0) * DRW * 128);
    }
#pragma unroll
    for (int q = 0; q < P; ++q) BLR_GLOAD(q, q);
    if (!dhw) {
        BLR_BLOAD(bq, 0);
        BLR_BLOAD(bn, 1);
    }
    BLR_SSTORE(0, 0, 0);
    BLR_GLOAD(0, P);
    BLR_SSTORE(1 % P, 1, 1);
    BLR_GLOAD(1 % P, P + 1);
    __syncthreads();
    // dh partial row (mt, nt): byte offset of column `lane` of step 0
    // (rows ordered N tile first, so each path's rows are contiguous)
    const int64_t mtl = (M + BM - 1) / BM;
    const uint64_t hpbytes = FDH ? (uint64_t)mtl * ntn * K * 4 : 0;
    const __amdgpu_buffer_rsrc_t rHP = make_rsrc(p.dh_partial, hpbytes);
    // (the B1 wave's column: 32 / WN columns a wave, 2 WN lanes a column)
    const uint32_t hpoff =
        (uint32_t)((((int64_t)nt * mtl + mt) * K + (32 / WN) * rwave + lane / (2 * WN)) * 4);
    if (!dhw) {
        BLR_AFRAG(fa, 0);
        BLR_BFRAG(fb, bq, 0, 0);
    }
    int b1 = 1, b2 = 2;  // LDS buffers of steps kt+1 and kt+2

#define BLR_UOFF(i, v, j) ((uint32_t)(((i) * 32 + 8 * ((v) >> 2) + ((v) & 3)) * N + (j) * 32) * 4u)
    // MP: at the end of path q's ranks the product so far is scaled by the
    // path's output column scale into yacc (its column partials, if any,
    // written for path q), and the accumulators restart from zero
    f32x16_t yacc[MP ? FM : 1][MP ? FN : 1];
    if (MP) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) yacc[i][j][v] = 0.0f;
    }
    // (the epilogue's output addressing, formed here only for MP)
    const int64_t rl_mp = MP ? m0 + wm * TM + 4 * (lane >> 5) : 0;
    const int cb_mp = MP ? n0 + wn * TN + (lane & 31) : 0;
    const uint32_t loff_mp = MP ? (uint32_t)((rl_mp * N + cb_mp) * 4) : 0u;
    const __amdgpu_buffer_rsrc_t rD_mp = make_rsrc(p.dot_other, (MP && DOT) ? (uint64_t)M * N * 4 : 0);
#define BLR_FLUSH(q)                                                                       \
    do {                                                                                   \
        const float osc_ = -p.oscale;                                                      \
        const bool full_ = m0 + BM <= M;                                                   \
        const float *c2p_ = p.out2col + (int64_t)(q) * p.o2_pstride;                       \
        float c2_[FN], ds_[FN];                                                            \
        _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                   \
            c2_[j] = c2p_[cb_mp + j * 32];                                                 \
            ds_[j] = 0.0f;                                                                 \
        }                                                                                  \
        _Pragma("unroll") for (int i = 0; i < FM; ++i)                                     \
            _Pragma("unroll") for (int v = 0; v < 16; ++v)                                 \
                _Pragma("unroll") for (int j = 0; j < FN; ++j) {                           \
                    const float val_ = acc[i][j][v] * osc_;                                \
                    if (DOT) {                                                             \
                        const bool in_ = full_ || rl_mp + i * 32 + 8 * (v >> 2) + (v & 3) < M; \
                        ds_[j] += val_ * (in_ ? load_f32_nt(rD_mp, loff_mp, BLR_UOFF(i, v, j)) : 0.0f); \
                    }                                                                      \
                    yacc[i][j][v] += val_ * c2_[j];                                        \
                    acc[i][j][v] = 0.0f;                                                   \
                }                                                                          \
        if (DOT) _Pragma("unroll") for (int j = 0; j < FN; ++j) {                          \
            const float t_ = ds_[j] + __shfl_xor(ds_[j], 32);                              \
            if (lane < 32) p.dot_partial[(int64_t)(q) * p.dot_pstride + (int64_t)mt * N + cb_mp + j * 32] = t_; \
        }                                                                                  \
    } while (0)

    // Iteration kt: fragments of step kt+1 are read and decoded while the
    // MFMAs of step kt run, stage kt+2 goes to LDS and stage kt+2+P is
    // loaded. Buffer kt+2 (mod 3) was last read in iteration kt-2. The
    // loads are unconditional (stages and groups past the end re-read the
    // last one and are never multiplied), so the compiler counts outstanding
    // loads exactly and waits only for the stage it converts.
    if (dhw) {
        // DH role, per step the partial c of the wave's ranks and its dh
        // sums. Iteration kt: MFMAs of step kt, signs of step kt+1 (words
        // loaded an iteration ago), words of step kt+2, the dot of step kt-1
        // (its dy in ring slot (kt-1) % 4, rewritten only after this
        // iteration's barrier) and the dh store of step kt-2; the B1 waves
        // stage dy.
        // The iteration is one basic block: the dot of step -1 (iteration 0)
        // multiplies a zero c by whatever slot 3 holds, and its sums and the
        // stores of steps -2 and -1 are never kept.
        half8_t hf[2][KD];       // decoded signs of steps kt and kt+1
        f32x16_t cc[2][FMD][CP]; // partial c of steps kt and kt-1
        f32x4_t d4[FMD][4];      // dy of step kt-1 in the accumulator layout
#pragma unroll
        for (int i = 0; i < FMD; ++i)
#pragma unroll
            for (int q = 0; q < CP; ++q)
#pragma unroll
                for (int v = 0; v < 16; ++v) cc[1][i][q][v] = 0.0f;
        BLR_DH_DECODE(hf[0], hb[0]);
        for (int kt0 = 0; kt0 < nk; kt0 += 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int kt = kt0 + u;
                BLR_DH_DYLOAD(d4, (kt + NSD - 1) & (NSD - 1));
                BLR_DH_MMA(cc[u & 1], hf[u & 1]);
                BLR_DH_DECODE(hf[(u + 1) & 1], hb[(u + 1) & 1]);
                const int kn_ = kt + 2 < nk ? kt + 2 : nk - 1;
                BLR_HLOAD(hb[u & 1], (uint32_t)kn_ * DRW * 128);
                BLR_DH_DOT(cc[(u + 1) & 1], d4, kt - 1);
                // the dy reads first, then each MFMA followed by VALU work
                // (decode, dot), which issues while the MFMA runs
                __builtin_amdgcn_sched_group_barrier(0x100, 4 * FMD, 0);
#pragma unroll
                for (int m_ = 0; m_ < 8; ++m_) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                }
                __syncthreads();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        BLR_DH_DYLOAD(d4, (nk - 1) & (NSD - 1));
        BLR_DH_DOT(cc[1], d4, nk - 1);  // nk is a multiple of 4: step nk-1 is odd
        __syncthreads();
    } else {
        // Two bitmap groups per iteration: group g's words in bq, group g+1's
        // in bn; each buffer is refilled (group g+2, g+3) right after its
        // last step's decode, so no register copy carries words across the
        // back edge. An odd last group leaves after the first half.
        for (int kt0 = 0; kt0 < nk; kt0 += 2 * U) {
#pragma unroll
            for (int u2 = 0; u2 < 2 * U; ++u2) {
                if (u2 == U && kt0 + U >= nk) break;
                const int u = u2 % U;        // step within its group
                const bool second = u2 >= U; // the group of this step is in bn
                const int kt = kt0 + u2;
                if (u2 % 2 == 0) {
                    BLR_AFRAG(fa2, b1);
                    if (second) {
                        BLR_BFRAG(fb2, bn, u + 1, kt + 1);
                    } else {
                        BLR_BFRAG(fb2, bq, u + 1, kt + 1);
                    }
                    BLR_MMA(fa, fb);
                } else {
                    BLR_AFRAG(fa, b1);
                    if (u < U - 1) {
                        if (second) {
                            BLR_BFRAG(fb, bn, u + 1, kt + 1);
                        } else {
                            BLR_BFRAG(fb, bq, u + 1, kt + 1);
                        }
                    } else if (second) {
                        BLR_BFRAG(fb, bq, 0, kt + 1);
                    } else {
                        BLR_BFRAG(fb, bn, 0, kt + 1);
                    }
                    BLR_MMA(fa2, fb2);
                }
                if (u == U - 1) {
                    if (second) {
                        BLR_BLOAD(bn, kt0 / U + 3);
                    } else {
                        BLR_BLOAD(bq, kt0 / U + 2);
                    }
                }
                if (FDH) BLR_B1_DHSUM(kt - 2);
                BLR_SSTORE((u2 + 2) % P, b2, (kt + 2) & (NSD - 1));
                BLR_GLOAD((u2 + 2) % P, kt + 2 + P);
                __syncthreads();
                // keep later steps' work out of this one: hoisted above the
                // barrier it would wait for loads issued just before
                __builtin_amdgcn_sched_barrier(0);
                b1 = b2;
                b2 = b2 == NS - 1 ? 0 : b2 + 1;
                if (MP && ((kt + 1) * BK) % PKr == 0) BLR_FLUSH((kt + 1) * BK / PKr - 1);
            }
        }
        if (FDH) {
            BLR_B1_DHSUM(nk - 2);
            __syncthreads();  // matches the DH role's final barrier
            BLR_B1_DHSUM(nk - 1);
        }
    }
#undef BLR_DH_DYLOAD
#undef BLR_DH_DECODE
#undef BLR_DH_MMA
#undef BLR_DH_DOT
#undef BLR_B1_DHSUM
#undef BLR_HLOAD
#undef BLR_GLOAD
#undef BLR_BLOAD
#undef BLR_SSTORE
#undef BLR_AFRAG
#undef BLR_BFRAG
#undef BLR_MMA

#undef BLR_FLUSH
    // Epilogue from the accumulators: products, tapes, scaled outputs and
    // column partials. Element (i, v, j) of a lane sits at row
    // rl + i*32 + 8*(v/4) + v%4 and column cb + j*32; the lane part of the
    // byte offset is a VGPR, the rest a uniform offset. Rows past M are
    // neither loaded, stored nor summed (only a tile that ends past M checks).
    const float osc = PLANE ? p.oscale : -p.oscale;  // decoded fragments hold -S
    const int64_t rl = m0 + wm * TM + 4 * (lane >> 5);
    const int cb = n0 + wn * TN + (lane & 31);
    const uint32_t loff = (uint32_t)((rl * N + cb) * 4);
    const bool full = m0 + BM <= M;
    const uint64_t obytes = (uint64_t)M * N * 4;
    const __amdgpu_buffer_rsrc_t rO = make_rsrc(p.out, OUT ? obytes : 0);
    const __amdgpu_buffer_rsrc_t rO2 = make_rsrc(p.out2, OUT2 ? obytes : 0);
    const __amdgpu_buffer_rsrc_t rD = make_rsrc(p.dot_other, DOT ? obytes : 0);
    float c2[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) c2[j] = (OUT2 && !MP) ? p.out2col[cb + j * 32] : 0.0f;
    float dsum[HR][FN];  // [64-row half of the wave's rows][column block]
#pragma unroll
    for (int h = 0; h < HR; ++h)
#pragma unroll
        for (int j = 0; j < FN; ++j) dsum[h][j] = 0.0f;
    // (GUARD: check rows against M; ACC: y or dx accumulate, so the old
    // values are loaded. The common case, a full tile written without
    // accumulation, has its own copy with no load: a load under a
    // per-element condition makes every store after it wait for all earlier
    // stores, which share the load counter.)
#define BLR_EPI_BLOCK(GUARD, ACC)                                                          \
    do {                                                                                   \
        _Pragma("unroll") for (int i = 0; i < FM; ++i) {                                   \
            float oth[DOT ? FN : 1][DOT ? 16 : 1], old[OUT2 ? FN : 1][OUT2 ? 16 : 1];      \
            _Pragma("unroll") for (int v = 0; v < 16; ++v) {                               \
                const bool in_ = !(GUARD) || rl + i * 32 + 8 * (v >> 2) + (v & 3) < M;     \
                _Pragma("unroll") for (int j = 0; j < FN; ++j) {                           \
                    if (DOT && !MP) oth[j][v] = !in_ ? 0.0f : FDH ?                                   \
                        aL[(4 * (lane >> 5) + i * 32 + 8 * (v >> 2) + (v & 3)) * LDA_ + wn * TN + (lane & 31) + j * 32] : \
                        load_f32_nt(rD, loff, BLR_UOFF(i, v, j));                                 \
                    if (OUT2) old[j][v] = ((ACC) && in_) ? load_f32(rO2, loff, BLR_UOFF(i, v, j)) : 0.0f; \
                }                                                                          \
            }                                                                              \
            _Pragma("unroll") for (int v = 0; v < 16; ++v) {                               \
                if (!(GUARD) || rl + i * 32 + 8 * (v >> 2) + (v & 3) < M) {                \
                    _Pragma("unroll") for (int j = 0; j < FN; ++j) {                       \
                        const float val = MP ? yacc[i][j][v] : acc[i][j][v] * osc;         \
                        if (OUT) store_f32(rO, loff, BLR_UOFF(i, v, j), val);              \
                        if (OUT2) store_f32_nt(rO2, loff, BLR_UOFF(i, v, j), old[j][v] + (MP ? val : val * c2[j])); \
                        if (DOT && !MP) dsum[HR == 1 ? 0 : i / 2][j] += val * oth[j][v];  \
                    }                                                                      \
                }                                                                          \
            }                                                                              \
        }                                                                                  \
    } while (0)
    if (!dhw) {
        if (full && !(OUT2 && p.out2acc)) {
            BLR_EPI_BLOCK(false, false);
        } else {
            BLR_EPI_BLOCK(true, p.out2acc);
        }
    }
#undef BLR_EPI_BLOCK
#undef BLR_UOFF
    if (DOT && !MP) {
        // lanes l and l+32 hold the same columns; then the WM waves of a
        // column strip add in row order
        if (!dhw) {
#pragma unroll
            for (int h = 0; h < HR; ++h)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const float t_ = dsum[h][j] + __shfl_xor(dsum[h][j], 32);
                    if (lane < 32) red[(h * WM + wm) * BN + wn * TN + j * 32 + lane] = t_;
                }
        }
        __syncthreads();
        for (int c = tid; c < HR * BN && tid < NT; c += NT) {
            const int h = c / BN, cc = c - h * BN;
            float sum = 0.0f;
#pragma unroll
            for (int w = 0; w < WM; ++w) sum += red[(h * WM + w) * BN + cc];
            if ((int64_t)(mt * HR + h) * 64 < M) p.dot_partial[((int64_t)mt * HR + h) * N + n0 + cc] = sum;
        }
    }
}

template <int BM, int BN, int WM, int WN, int P, int MINB, bool OUT, bool OUT2, bool DOT, int GM, bool FDH = false,
          int KB = 2, bool PLANE = false, bool MP = false>
static hipError_t launch_gemm_t(int id, const GemmArgs &a, hipStream_t s) {
    if (a.N % BN != 0 || a.K % 128 != 0 || a.K < 128) return hipErrorInvalidValue;
    if (a.path_k && (a.path_k % 128 || a.K % a.path_k)) return hipErrorInvalidValue;
    if (a.path_n && a.path_n % BN) return hipErrorInvalidValue;
    const int64_t tiles = (int64_t)(a.N / BN) * ((a.M + BM - 1) / BM);
    prof_begin(id, s);
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, P, MINB, OUT, OUT2, DOT, GM, FDH, KB, PLANE, MP>),
                       dim3((unsigned)tiles),
                       dim3((FDH ? 2 : 1) * WM * WN * 64), 0, s, a);
    hipError_t e = hipGetLastError();
    prof_end(s);
    return e;
}

// ---------------------------------------------------------------------------
// Short-K contraction with the activation block held in LDS (the kinds with
// K = r: F2, B2). A workgroup of 4 or 8 waves loads the bitmap words of its
// tiles into registers, stages its 64 x K activation rows once (scaled and
// rounded to f16, as in gemm_kernel), then walks a run of TPW consecutive
// 64 x 256 output tiles with no further barrier and no load before its
// epilogue: per tile each wave (64 rows x 64 or 32 columns) reads A fragments
// from LDS, decodes B fragments from its words, and stores its block from
// the accumulators, so one tile's stores drain while the next tile's MFMAs
// run (a load issued after the stores would have to wait for them: vector
// loads and stores share one counter). The column partials need no
// cross-wave sum: every wave holds all 64 rows of its columns.
constexpr int AS_BM = 64, AS_BN = 256, AS_KMAX = 512;  // LDS: 64 x (K + 8) halves, 66.5 KB at K = 512
// K = 1024 also takes the held block (129 KB of LDS: one workgroup per CU,
// eight waves of 64 x 32 for every kind, two a SIMD)
constexpr int AS_KBIG = 1024;

// PR > 0: several paths along K, PR * 128 ranks each (K = paths * PR * 128),
// the bitmap of path q at Bbits + q * b_pstride words ([N][PR * 4] words),
// and out2 (+)= sum over paths of out2col_q . product_q: path q's column scale
// (rounded to f16) is folded into its decoded signs, so one sweep over K
// forms the sum (no column partials in this mode).
template <int KG, int TPW, bool OUT, bool OUT2, bool DOT, int PR = 0, int NWV = 4>
__global__ __launch_bounds__(64 * NWV, KG > 4 ? 2 : NWV / 2) void gemm_as_kernel(GemmArgs p, int groups_n) {
    constexpr int K = 128 * KG, LDK = K + 8;
    static_assert(PR == 0 || (OUT2 && !OUT && !DOT && KG % PR == 0), "paths folded along K");
    constexpr int NP = PR ? KG / PR : 1;  // paths
    __shared__ __attribute__((aligned(16))) _Float16 As[AS_BM * LDK];
    // NWV waves, each 64 rows x 256 / NWV columns of a tile: 4 (64 x 64,
    // two workgroups of 4 waves per CU) or 8 (64 x 32: four waves a SIMD,
    // in at most 128 registers)
    constexpr int NTH = 64 * NWV, TN = AS_BN / NWV, FM = 2, FN = TN / 32;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wn = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = p.N;
    const int64_t M = p.M;
    const int L = blockIdx.x, G = gridDim.x;
    const int T = (G % NUM_XCD == 0) ? (L % NUM_XCD) * (G / NUM_XCD) + L / NUM_XCD : L;
    const int mt = T / groups_n, gn = T - mt * groups_n;
    const int t0 = gn * TPW;  // the workgroup's tiles: t0 .. t0 + TPW - 1
    const int64_t m0 = (int64_t)mt * AS_BM;

    // bitmap words of this lane's two plane rows in each tile, KG 16-byte
    // groups per row; tile 0's first (they arrive while the block is
    // staged), each later tile's at the start of the one before
    constexpr int KW = PR ? PR * 4 : K / 32;  // bitmap words per plane row (of a path)
    u32x4_t wall[TPW][FN][KG];
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.Bbits, PR ? (uint64_t)(NP - 1) * p.b_pstride * 4 + (uint64_t)N * KW * 4
                                                            : (uint64_t)N * K / 8);
#define AS_WLOAD(tt)                                                                       \
    do {                                                                                   \
        _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                   \
            const uint32_t bo_ = (uint32_t)(((t0 + (tt)) * AS_BN + wn * TN + j * 32 + (lane & 31)) * KW * 4); \
            _Pragma("unroll") for (int g = 0; g < KG; ++g) wall[tt][j][g] = load_u32x4(rB, bo_, \
                PR ? (uint32_t)((g / (PR ? PR : 1)) * p.b_pstride * 4 + (g % (PR ? PR : 1)) * 16) : (uint32_t)g * 16); \
        }                                                                                  \
    } while (0)
    AS_WLOAD(0);

    // Stage the block: chunk i (float4) of the 64 x K block is row i / (K/4),
    // columns 4 (i % (K/4)); rows past M read row M-1 (never stored or summed).
    // The column scales of the epilogue (OUT2) for every tile, first.
    float c2all[TPW][FN];
    uint32_t h2all[PR ? TPW : 1][PR ? FN : 1][NP];  // PR: each path's f16 column scale, both halves
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n_ = (t0 + tt) * AS_BN + wn * TN + j * 32 + (lane & 31);
            c2all[tt][j] = (OUT2 && !PR) ? p.out2col[n_] : 1.0f;
            if (PR) {
#pragma unroll
                for (int q = 0; q < NP; ++q) {
                    const uint32_t h_ = __builtin_bit_cast(uint16_t, (_Float16)p.out2col[q * p.o2_pstride + n_]);
                    h2all[PR ? tt : 0][PR ? j : 0][q] = h_ | (h_ << 16);
                }
            }
        }
    {
        // all of a thread's chunks in flight at once (up to 32 float4); when
        // 256 is a multiple of the chunks per row, a thread's chunks share
        // one column group and its scales are loaded once
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A, (uint64_t)M * p.lda * 4);
        const __amdgpu_buffer_rsrc_t rC = make_rsrc(p.colscale, (uint64_t)K * 4);
        constexpr int cpr = K / 4, nch = AS_BM * cpr;  // chunks per row, in the block
        constexpr int UNR = nch / NTH < 32 ? nch / NTH : 32;
        constexpr bool onecol = NTH % cpr == 0;
        const f32x4_t c1 = onecol ? load_f32x4(rC, (uint32_t)(16 * (tid % cpr)), 0u) : f32x4_t{};
        if (onecol && m0 + AS_BM <= M) {
            // full block: thread tid takes rows tid / cpr + u * (256 / cpr) of
            // column group tid % cpr; the row step is a uniform offset, so
            // every load is issued before the first is waited for
            constexpr int rstep = NTH / (onecol ? cpr : NTH);
            const int r0 = tid / cpr, c4 = tid % cpr;
            const uint32_t vb = (uint32_t)(((m0 + r0) * p.lda + 4 * c4) * 4);
            f32x4_t v[nch / NTH];
#pragma unroll
            for (int u = 0; u < nch / NTH; ++u) v[u] = load_f32x4(rA, vb, (uint32_t)(u * rstep * p.lda * 4));
            const f32x4_t cs = c1 * p.ascale;
#pragma unroll
            for (int u = 0; u < nch / NTH; ++u) {
                uint2 h;
                h.x = f16x2_scaled(v[u].x, cs.x, v[u].y, cs.y);
                h.y = f16x2_scaled(v[u].z, cs.z, v[u].w, cs.w);
                *reinterpret_cast<uint2 *>(As + (r0 + u * rstep) * LDK + 4 * c4) = h;
            }
        } else
        for (int i0 = 0; i0 < nch; i0 += NTH * UNR) {
            f32x4_t v[UNR], c[onecol ? 1 : UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int i = i0 + u * NTH + tid;
                const int ic = i < nch ? i : nch - 1;
                const int row = ic / cpr, c4 = ic - row * cpr;
                int64_t gm = m0 + row;
                gm = gm < M ? gm : M - 1;
                v[u] = load_f32x4(rA, (uint32_t)((gm * p.lda + 4 * c4) * 4), 0u);
                if (!onecol) c[u] = load_f32x4(rC, (uint32_t)(16 * c4), 0u);
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int i = i0 + u * NTH + tid;
                if (i < nch) {
                    const int row = i / cpr, c4 = i - row * cpr;
                    const f32x4_t cs = (onecol ? c1 : c[onecol ? 0 : u]) * p.ascale;
                    uint2 h;
                    h.x = f16x2_scaled(v[u].x, cs.x, v[u].y, cs.y);
                    h.y = f16x2_scaled(v[u].z, cs.z, v[u].w, cs.w);
                    *reinterpret_cast<uint2 *>(As + row * LDK + 4 * c4) = h;
                }
            }
        }
    }
    __syncthreads();

    const uint32_t grp = (uint32_t)(lane >> 5);
    const uint32_t sel[2] = {grp * 0x01010101u, (2u + grp) * 0x01010101u};
    uint32_t sgnmask, one16;
    asm volatile("v_mov_b32 %0, 0x80008000" : "=v"(sgnmask));
    asm volatile("v_mov_b32 %0, 0x3c003c00" : "=v"(one16));
    const _Float16 *arow = As + (lane & 31) * LDK + (lane >> 5) * 8;  // fragment read base

    const float osc = -p.oscale;  // decoded fragments hold -S
    const uint64_t obytes = (uint64_t)M * N * 4;
    const __amdgpu_buffer_rsrc_t rO = make_rsrc(p.out, OUT ? obytes : 0);
    const __amdgpu_buffer_rsrc_t rO2 = make_rsrc(p.out2, OUT2 ? obytes : 0);
    const __amdgpu_buffer_rsrc_t rD = make_rsrc(p.dot_other, DOT ? obytes : 0);
    const int64_t rl = m0 + 4 * (lane >> 5);
    const bool full = m0 + AS_BM <= M;

#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        const int t = t0 + tt;
        if (tt + 1 < TPW) AS_WLOAD(tt + 1);
        // epilogue addressing: element (i, v, j) at row rl + 32 i + 8 (v/4) +
        // v%4, column cb + 32 j; the row stride is re-read per tile (opaque
        // to the compiler), so its uniform offsets are formed per tile
        // rather than held across tiles
        int Nl = N;
        asm volatile("" : "+s"(Nl));
        const int cb = t * AS_BN + wn * TN + (lane & 31);
        const uint32_t loff = (uint32_t)((rl * Nl + cb) * 4);
#define AS_UOFF(i, v, j) ((uint32_t)((8 * ((v) >> 2) + ((v) & 3)) * Ni + (j) * 32) * 4u)
        // the dot operand of the epilogue (DOT), loaded before the MFMAs so
        // its latency is hidden behind them
        float oth[DOT ? FM : 1][DOT ? FN : 1][DOT ? 16 : 1];
        if (DOT) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                int Ni = Nl;
                asm volatile("" : "+s"(Ni));
                const uint32_t lo_ = loff + (uint32_t)(i * 32 * Ni * 4);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const bool in_ = full || rl + i * 32 + 8 * (v >> 2) + (v & 3) < M;
#pragma unroll
                    for (int j = 0; j < FN; ++j) oth[i][j][v] = in_ ? load_f32_nt(rD, lo_, AS_UOFF(i, v, j)) : 0.0f;
                }
            }
        }
        f32x16_t acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
        // k-blocks of 16 (word kb/2 of group kb/8): the A fragments and signs
        // of block kb+1 are read and decoded while block kb's MFMAs run
        constexpr int NKB = 8 * KG;
        half8_t fa[2][FM], fb[2][FN];
#define AS_FRAGS(buf, kb)                                                                  \
        do {                                                                               \
            _Pragma("unroll") for (int i = 0; i < FM; ++i) fa[buf][i] =                    \
                *reinterpret_cast<const half8_t *>(arow + i * 32 * LDK + 16 * (kb));       \
            _Pragma("unroll") for (int j = 0; j < FN; ++j) fb[buf][j] = PR ?               \
                sign_frag_h(wall[tt][j][(kb) / 8][((kb) / 2) % 4], sel[(kb) % 2], sgnmask,  \
                            h2all[PR ? tt : 0][PR ? j : 0][(kb) / (8 * (PR ? PR : 1))]) :  \
                sign_frag(wall[tt][j][(kb) / 8][((kb) / 2) % 4], sel[(kb) % 2], sgnmask, one16); \
        } while (0)
        AS_FRAGS(0, 0);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            if (kb + 1 < NKB) AS_FRAGS((kb + 1) & 1, kb + 1);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[kb & 1][i], fb[kb & 1][j], acc[i][j], 0, 0, 0);
            // this block: the next block's reads first, then MFMAs with the
            // decode in between
            if (kb + 1 < NKB) {
                __builtin_amdgcn_sched_group_barrier(0x100, FM, 0);
#pragma unroll
                for (int m_ = 0; m_ < FM * FN; ++m_) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#undef AS_FRAGS
        float dsum[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) dsum[j] = 0.0f;
#define AS_EPI(GUARD, ACC) /* as BLR_EPI_BLOCK */                                           \
        do {                                                                               \
            _Pragma("unroll") for (int i = 0; i < FM; ++i) {                               \
                /* one row block at a time: 16 uniform row offsets live */                  \
                int Ni = Nl;                                                               \
                asm volatile("" : "+s"(Ni));                                               \
                const uint32_t lo_ = loff + (uint32_t)(i * 32 * Ni * 4);                   \
                float old[OUT2 ? FN : 1][OUT2 ? 16 : 1];                                   \
                _Pragma("unroll") for (int v = 0; v < 16; ++v) {                           \
                    const bool in_ = !(GUARD) || rl + i * 32 + 8 * (v >> 2) + (v & 3) < M; \
                    _Pragma("unroll") for (int j = 0; j < FN; ++j)                         \
                        if (OUT2) old[j][v] = ((ACC) && in_) ? load_f32(rO2, lo_, AS_UOFF(i, v, j)) : 0.0f; \
                }                                                                          \
                _Pragma("unroll") for (int v = 0; v < 16; ++v) {                           \
                    if (!(GUARD) || rl + i * 32 + 8 * (v >> 2) + (v & 3) < M) {            \
                        _Pragma("unroll") for (int j = 0; j < FN; ++j) {                   \
                            const float val = acc[i][j][v] * osc;                          \
                            if (OUT) store_f32(rO, lo_, AS_UOFF(i, v, j), val);           \
                            if (OUT2) store_f32_nt(rO2, lo_, AS_UOFF(i, v, j), old[j][v] + val * c2all[tt][j]); \
                            if (DOT) dsum[j] += val * oth[i][j][v];                        \
                        }                                                                  \
                    }                                                                      \
                }                                                                          \
            }                                                                              \
        } while (0)
        if (full && !(OUT2 && p.out2acc)) {
            AS_EPI(false, false);
        } else {
            AS_EPI(true, p.out2acc);
        }
#undef AS_EPI
#undef AS_UOFF
        if (DOT) {
            // lanes l and l+32 hold other rows of the same column
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const float sum = dsum[j] + __shfl_xor(dsum[j], 32);
                if (lane < 32) p.dot_partial[(int64_t)mt * N + cb + j * 32] = sum;
            }
        }
    }
#undef AS_WLOAD
}

template <int KG, int TPW, bool OUT, bool OUT2, bool DOT, int PR = 0, int NWV = 4>
static hipError_t launch_gemm_as_tt(int id, const GemmArgs &a, hipStream_t s) {
    const int64_t mtiles = (a.M + AS_BM - 1) / AS_BM;
    const int64_t gn = a.N / AS_BN / TPW;
    prof_begin(id, s);
    hipLaunchKernelGGL((gemm_as_kernel<KG, TPW, OUT, OUT2, DOT, PR, NWV>), dim3((unsigned)(mtiles * gn)), dim3(64 * NWV), 0, s,
                       a, (int)gn);
    hipError_t e = hipGetLastError();
    prof_end(s);
    return e;
}

template <int KG, bool OUT, bool OUT2, bool DOT, int PR = 0>
static hipError_t launch_gemm_as_t(int id, const GemmArgs &a, hipStream_t s) {
    if (a.N % AS_BN != 0 || a.K != 128 * KG) return hipErrorInvalidValue;
    const int64_t mtiles = (a.M + AS_BM - 1) / AS_BM;
    const int ntiles = a.N / AS_BN;
    if constexpr (KG > 4) {
        // one workgroup per CU: runs of four tiles while that leaves a
        // workgroup for every CU, else two, else one
        if (ntiles % 4 == 0 && mtiles * (ntiles / 4) >= 256) return launch_gemm_as_tt<KG, 4, OUT, OUT2, DOT, PR, 8>(id, a, s);
        if (ntiles % 2 == 0 && mtiles * (ntiles / 2) >= 256) return launch_gemm_as_tt<KG, 2, OUT, OUT2, DOT, PR, 8>(id, a, s);
        return launch_gemm_as_tt<KG, 1, OUT, OUT2, DOT, PR, 8>(id, a, s);
    } else {
    // the longest run of tiles (its words fit in registers: TPW * KG <= 16)
    // that still gives about two workgroups per CU; the runs of one M tile
    // land on one XCD. Without the dot operand every run takes 8 waves of
    // 64 x 32 (four a SIMD): 5-14% faster than 4 waves of 64 x 64 for F2 at
    // M = 2048..8192, d = 4096, r = 512; with it they would spill.
    if (KG <= 4 && ntiles % 4 == 0 && mtiles * (ntiles / 4) >= 512)
        return launch_gemm_as_tt<KG, 4, OUT, OUT2, DOT, PR, DOT ? 4 : 8>(id, a, s);
    // (a run of 2 with the dot operand spills: at M = 2048..8192, d = 4096,
    // r = 512 it took 1.4-1.55x a run of 1 or 4, so that kind goes to runs of 1)
    if constexpr (!DOT) {
        if (ntiles % 2 == 0 && mtiles * (ntiles / 2) >= 512) return launch_gemm_as_tt<KG, 2, OUT, OUT2, DOT, PR, 8>(id, a, s);
    }
    return launch_gemm_as_tt<KG, 1, OUT, OUT2, DOT, PR, DOT ? 4 : 8>(id, a, s);
    }
}

// B2 of a layer of NP paths on the held activation block (K = NP paths of
// 128 KGP ranks, the paths' db side by side): per output tile each path's
// product is formed in turn from its own ranks (its accumulators restarting
// from zero), its dot with the tile's x goes to that path's column partials,
// and its g_p-scaled value is added to the tile's dx sum, which is stored
// once after the last path. Each path's words are loaded while the path
// before it runs, and the next tile's x while its last path runs. One
// workgroup of 8 waves per CU (the block of K <= 1024 ranks takes up to
// 129 KB of LDS), each walking a run of tpw consecutive tiles; the tile loop
// is not unrolled.
template <int KGP, int NP>
__global__ __launch_bounds__(512, 1) void gemm_as_paths_kernel(GemmArgs p, int groups_n, int tpw) {
    constexpr int KG = KGP * NP, K = 128 * KG, LDK = K + 8;
    static_assert(K <= 1024 && NP >= 2, "paths block");
    __shared__ __attribute__((aligned(16))) _Float16 As[AS_BM * LDK];
    // 8 waves, each 64 rows x 32 columns of the 64 x 256 tile: two waves a
    // SIMD, so one's VALU work and waits overlap the other's MFMAs
    constexpr int NW = 8, NT = 64 * NW, FM = 2, FN = 1, TN = 32, NKB = 8 * KGP;  // NKB: k-blocks per path
    const int tid = threadIdx.x, lane = tid & 63;
    const int wn = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = p.N;
    const int64_t M = p.M;
    const int L = blockIdx.x, G = gridDim.x;
    const int T = (G % NUM_XCD == 0) ? (L % NUM_XCD) * (G / NUM_XCD) + L / NUM_XCD : L;
    const int mt = T / groups_n, gn = T - mt * groups_n;
    const int t0 = gn * tpw;
    const int64_t m0 = (int64_t)mt * AS_BM;

    // bitmap words of path q for this lane's two plane rows of tile t: KGP
    // 16-byte groups per row, path q at Bbits + q * b_pstride words
    u32x4_t w[2][FN][KGP];
    const __amdgpu_buffer_rsrc_t rB =
        make_rsrc(p.Bbits, (uint64_t)(NP - 1) * p.b_pstride * 4 + (uint64_t)N * KGP * 16);
#define ASP_WLOAD(buf, t_, q_)                                                             \
    do {                                                                                   \
        _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                   \
            const uint32_t bo_ = (uint32_t)(((t_) * AS_BN + wn * TN + j * 32 + (lane & 31)) * KGP * 16); \
            _Pragma("unroll") for (int g = 0; g < KGP; ++g) w[buf][j][g] =                 \
                load_u32x4(rB, bo_, (uint32_t)((q_) * p.b_pstride * 4 + g * 16));          \
        }                                                                                  \
    } while (0)
    ASP_WLOAD(0, t0, 0);

    // Stage the block, as the single-path kernel does: chunk i (float4) is
    // row i / (K/4), columns 4 (i % (K/4)); rows past M read row M-1. When
    // 256 is a multiple of the chunks per row, a thread's chunks share one
    // column group and its scales are loaded once.
    {
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A, (uint64_t)M * p.lda * 4);
        const __amdgpu_buffer_rsrc_t rC = make_rsrc(p.colscale, (uint64_t)K * 4);
        constexpr int cpr = K / 4, nch = AS_BM * cpr;
        constexpr int UNR = 8;
        constexpr bool onecol = NT % cpr == 0;
        const f32x4_t c1 = onecol ? load_f32x4(rC, (uint32_t)(16 * (tid % cpr)), 0u) * p.ascale : f32x4_t{};
        for (int i0 = 0; i0 < nch; i0 += NT * UNR) {
            f32x4_t v[UNR], c[onecol ? 1 : UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int i = i0 + u * NT + tid;
                const int ic = i < nch ? i : nch - 1;
                const int row = ic / cpr, c4 = ic - row * cpr;
                int64_t gm = m0 + row;
                gm = gm < M ? gm : M - 1;
                v[u] = load_f32x4(rA, (uint32_t)((gm * p.lda + 4 * c4) * 4), 0u);
                if (!onecol) c[u] = load_f32x4(rC, (uint32_t)(16 * c4), 0u);
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int i = i0 + u * NT + tid;
                if (i < nch) {
                    const int row = i / cpr, c4 = i - row * cpr;
                    const f32x4_t cs = onecol ? c1 : c[onecol ? 0 : u] * p.ascale;
                    uint2 h;
                    h.x = f16x2_scaled(v[u].x, cs.x, v[u].y, cs.y);
                    h.y = f16x2_scaled(v[u].z, cs.z, v[u].w, cs.w);
                    *reinterpret_cast<uint2 *>(As + row * LDK + 4 * c4) = h;
                }
            }
        }
    }
    __syncthreads();

    const uint32_t grp = (uint32_t)(lane >> 5);
    const uint32_t sel[2] = {grp * 0x01010101u, (2u + grp) * 0x01010101u};
    uint32_t sgnmask, one16;
    asm volatile("v_mov_b32 %0, 0x80008000" : "=v"(sgnmask));
    asm volatile("v_mov_b32 %0, 0x3c003c00" : "=v"(one16));
    const _Float16 *arow = As + (lane & 31) * LDK + (lane >> 5) * 8;  // fragment read base
    const float osc = -p.oscale;  // decoded fragments hold -S
    const uint64_t obytes = (uint64_t)M * N * 4;
    const __amdgpu_buffer_rsrc_t rO2 = make_rsrc(p.out2, obytes);
    const __amdgpu_buffer_rsrc_t rD = make_rsrc(p.dot_other, obytes);
    const int64_t rl = m0 + 4 * (lane >> 5);
    const bool full = m0 + AS_BM <= M;

    // the x of tile t_ (the dot operand of every path); a tile's is loaded
    // while the previous tile's last path runs, ahead of that tile's stores
    // (loads and stores share one counter, in order)
#define ASP_UOFF(i, v, j) ((uint32_t)((8 * ((v) >> 2) + ((v) & 3)) * Ni + (j) * 32) * 4u)
#define ASP_XLOAD(dst, t_)                                                                 \
    do {                                                                                   \
        int Nx_ = N;                                                                       \
        asm volatile("" : "+s"(Nx_));                                                      \
        const uint32_t lx_ = (uint32_t)((rl * Nx_ + (t_) * AS_BN + wn * TN + (lane & 31)) * 4); \
        _Pragma("unroll") for (int i = 0; i < FM; ++i) {                                   \
            int Ni = Nx_;                                                                  \
            asm volatile("" : "+s"(Ni));                                                   \
            const uint32_t lo_ = lx_ + (uint32_t)(i * 32 * Ni * 4);                        \
            _Pragma("unroll") for (int v = 0; v < 16; ++v) {                               \
                const bool in_ = full || rl + i * 32 + 8 * (v >> 2) + (v & 3) < M;         \
                _Pragma("unroll") for (int j = 0; j < FN; ++j)                             \
                    dst[i][j][v] = in_ ? load_f32_nt(rD, lo_, ASP_UOFF(i, v, j)) : 0.0f;   \
            }                                                                              \
        }                                                                                  \
    } while (0)
    float oth[FM][FN][16], othn[FM][FN][16];
    ASP_XLOAD(oth, t0);

    for (int tt = 0; tt < tpw; ++tt) {
        const int t = t0 + tt;
        int Nl = N;
        asm volatile("" : "+s"(Nl));
        const int cb = t * AS_BN + wn * TN + (lane & 31);
        const uint32_t loff = (uint32_t)((rl * Nl + cb) * 4);
        f32x16_t ysum[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) ysum[i][j][v] = 0.0f;
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            // the next path's words (this tile's, or the next tile's first)
            if (q + 1 < NP) {
                ASP_WLOAD((q + 1) & 1, t, q + 1);
            } else if (tt + 1 < tpw) {
                ASP_WLOAD((q + 1) & 1, t + 1, 0);
                ASP_XLOAD(othn, t + 1);
            }
            float c2[FN];  // g_p, times the output scale (the fragments hold -S)
#pragma unroll
            for (int j = 0; j < FN; ++j) c2[j] = p.out2col[(int64_t)q * p.o2_pstride + cb + j * 32] * osc;
            f32x16_t acc[FM][FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
            half8_t fa[2][FM], fb[2][FN];
#define ASP_FRAGS(buf, kb)                                                                 \
            do {                                                                           \
                _Pragma("unroll") for (int i = 0; i < FM; ++i) fa[buf][i] =                \
                    *reinterpret_cast<const half8_t *>(arow + i * 32 * LDK + q * (128 * KGP) + 16 * (kb)); \
                _Pragma("unroll") for (int j = 0; j < FN; ++j) fb[buf][j] =                \
                    sign_frag(w[q & 1][j][(kb) / 8][((kb) / 2) % 4], sel[(kb) % 2], sgnmask, one16); \
            } while (0)
            ASP_FRAGS(0, 0);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                if (kb + 1 < NKB) ASP_FRAGS((kb + 1) & 1, kb + 1);
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[kb & 1][i], fb[kb & 1][j], acc[i][j], 0, 0, 0);
                if (kb + 1 < NKB) {
                    __builtin_amdgcn_sched_group_barrier(0x100, FM, 0);
#pragma unroll
                    for (int m_ = 0; m_ < FM * FN; ++m_) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#undef ASP_FRAGS
            // this path's product: its dot with x (rows past M hold zero x)
            // and its g_p-scaled share of dx
            float ds[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) ds[j] = 0.0f;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v)
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        ds[j] += acc[i][j][v] * oth[i][j][v];
                        ysum[i][j][v] += acc[i][j][v] * c2[j];
                    }
            // lanes l and l+32 hold other rows of the same column
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const float sum = (ds[j] + __shfl_xor(ds[j], 32)) * osc;
                if (lane < 32) p.dot_partial[(int64_t)q * p.dot_pstride + (int64_t)mt * N + cb + j * 32] = sum;
            }
        }
        if (tt + 1 < tpw) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) oth[i][j][v] = othn[i][j][v];
        }
        if (NP & 1) {  // the next tile's first words arrived in buffer 1
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int g = 0; g < KGP; ++g) w[0][j][g] = w[1][j][g];
        }
        // dx (+)= the sum over paths, one row block at a time
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            int Ni = Nl;
            asm volatile("" : "+s"(Ni));
            const uint32_t lo_ = loff + (uint32_t)(i * 32 * Ni * 4);
            float old[FN][16];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const bool in_ = full || rl + i * 32 + 8 * (v >> 2) + (v & 3) < M;
#pragma unroll
                for (int j = 0; j < FN; ++j) old[j][v] = (p.out2acc && in_) ? load_f32(rO2, lo_, ASP_UOFF(i, v, j)) : 0.0f;
            }
#pragma unroll
            for (int v = 0; v < 16; ++v)
                if (full || rl + i * 32 + 8 * (v >> 2) + (v & 3) < M) {
#pragma unroll
                    for (int j = 0; j < FN; ++j) store_f32_nt(rO2, lo_, ASP_UOFF(i, v, j), old[j][v] + ysum[i][j][v]);
                }
        }
    }
#undef ASP_XLOAD
#undef ASP_UOFF
#undef ASP_WLOAD
}

template <int KGP, int NP>
static hipError_t launch_gemm_as_paths_t(int id, const GemmArgs &a, hipStream_t s) {
    const int64_t mtiles = (a.M + AS_BM - 1) / AS_BM;
    const int ntiles = a.N / AS_BN;
    // the longest run of tiles that still gives every CU a workgroup
    int tpw = 1;
    while (tpw * 2 <= 8 && ntiles % (tpw * 2) == 0 && mtiles * (ntiles / (tpw * 2)) >= 256) tpw *= 2;
    const int64_t gn = ntiles / tpw;
    prof_begin(id, s);
    hipLaunchKernelGGL((gemm_as_paths_kernel<KGP, NP>), dim3((unsigned)(mtiles * gn)), dim3(512), 0, s, a, (int)gn,
                       tpw);
    hipError_t e = hipGetLastError();
    prof_end(s);
    return e;
}

template <bool OUT, bool OUT2, bool DOT>
static hipError_t launch_gemm_as(int id, const GemmArgs &a, hipStream_t s) {
    switch (a.K) {
        case 128: return launch_gemm_as_t<1, OUT, OUT2, DOT>(id, a, s);
        case 256: return launch_gemm_as_t<2, OUT, OUT2, DOT>(id, a, s);
        case 384: return launch_gemm_as_t<3, OUT, OUT2, DOT>(id, a, s);
        case 512: return launch_gemm_as_t<4, OUT, OUT2, DOT>(id, a, s);
        case 1024: return launch_gemm_as_t<8, OUT, OUT2, DOT>(id, a, s);
    }
    return hipErrorInvalidValue;
}

// Every kind writes its column partials in rows of 64 tokens (the 128-row
// tiles write two), so they have ceil(M/64) rows.
int gemm_tile_rows(GemmKind) { return 64; }
int b1dh_cols(int64_t M, int64_t r, int64_t P) {
    if (r != 128 && r != 256 && r != 512) return 0;
    // 256 ranks a workgroup, or 128 where that would leave half the CUs idle
    if (r == 128 || ((M + 63) / 64) * (P * r / 256) <= SMALL_GRID) return 128;
    return 256;
}
int b1dh_tile_rows(int64_t r) { return (r == 128 || r == 256 || r == 512) ? 64 : 0; }

hipError_t launch_gemm(GemmKind kind, const GemmArgs &a, hipStream_t s) {
    const bool wide = a.N % 256 == 0;
    const bool as = wide && (a.K <= AS_KMAX || a.K == AS_KBIG);  // activation block held in LDS
    // F1 and B1 (N = r, K a model dimension) on 128 x 256 tiles (8 waves of
    // 128 x 32, 32-wide K steps) when that still gives at least 256
    // workgroups: each decoded sign fragment feeds four MFMAs instead of two.
    // Measured at r = 1024 and 2048: 16-20% faster than 64 x 256 tiles; the
    // short-K kinds (F2, DH, B2) were 5-18% slower on them, so they keep
    // 64-row tiles
    const bool t128 = wide && !a.path_n && !a.path_k && ((a.M + 127) / 128) * (a.N / 256) >= 256;
    // F1 and B1 on 64 x 128 tiles (two workgroups a CU) where 64 x 256 tiles
    // would leave half the CUs idle: measured at 2048 tokens, 16-18% faster
    const bool few = ((a.M + 63) / 64) * (a.N / 256) <= SMALL_GRID;
    switch (kind) {
        case GEMM_F1:
            // 256 columns per tile when they stay inside one path: the x tile
            // is staged once for twice the columns, and with one workgroup per
            // CU four stages of x are loaded ahead. Eight waves of 64 x 32, two
            // a SIMD, so one wave's decode and staging issue beside the other's
            // MFMAs: measured 5-6% faster than four waves of 64 x 64 at 6144 to
            // 12288 tokens (d_in = 4096, r = 512)
            if (t128) return launch_gemm_t<128, 256, 1, 8, 2, 1, true, false, false, 1, false, 2>(K_GEMM_F1, a, s);
            if ((a.path_n ? a.path_n : a.N) % 256 == 0 && !few)
                return launch_gemm_t<64, 256, 1, 8, 4, 1, true, false, false, 1, false, 4>(K_GEMM_F1, a, s);
            return launch_gemm_t<64, 128, 1, 4, 2, 2, true, false, false, 1, false, 4>(K_GEMM_F1, a, s);
        case GEMM_F2:
            if (as) return launch_gemm_as<true, true, false>(K_GEMM_F2, a, s);
            return wide ? launch_gemm_t<64, 256, 1, 4, 2, 2, true, true, false, 8, false, 4>(K_GEMM_F2, a, s)
                        : launch_gemm_t<64, 128, 1, 4, 2, 2, true, true, false, 8, false, 4>(K_GEMM_F2, a, s);
        case GEMM_F2_NOTAPE:
            if (as) return launch_gemm_as<false, true, false>(K_GEMM_F2, a, s);
            return wide ? launch_gemm_t<64, 256, 1, 4, 2, 2, false, true, false, 8, false, 4>(K_GEMM_F2, a, s)
                        : launch_gemm_t<64, 128, 1, 4, 2, 2, false, true, false, 8, false, 4>(K_GEMM_F2, a, s);
        case GEMM_DH:
            if (as) return launch_gemm_as<false, false, true>(K_GEMM_DH, a, s);
            return wide ? launch_gemm_t<64, 256, 1, 4, 2, 2, false, false, true, 8, false, 4>(K_GEMM_DH, a, s)
                        : launch_gemm_t<64, 128, 1, 4, 2, 2, false, false, true, 8, false, 4>(K_GEMM_DH, a, s);
        case GEMM_B1:
            // (the same tiles as F1; eight waves measured 6% faster here too)
            if (t128) return launch_gemm_t<128, 256, 1, 8, 2, 1, true, false, true, 1, false, 2>(K_GEMM_B1, a, s);
            if ((a.path_n ? a.path_n : a.N) % 256 == 0 && !few)
                return launch_gemm_t<64, 256, 1, 8, 4, 1, true, false, true, 1, false, 4>(K_GEMM_B1, a, s);
            return launch_gemm_t<64, 128, 1, 4, 2, 2, true, false, true, 1, false, 4>(K_GEMM_B1, a, s);
        case GEMM_B2:
            if (as) return launch_gemm_as<false, true, true>(K_GEMM_B2, a, s);
            return wide ? launch_gemm_t<64, 256, 1, 4, 2, 2, false, true, true, 8, false, 4>(K_GEMM_B2, a, s)
                        : launch_gemm_t<64, 128, 1, 4, 2, 2, false, true, true, 8, false, 4>(K_GEMM_B2, a, s);
        case GEMM_PLANE: return launch_gemm_t<64, 128, 1, 4, 2, 2, true, false, false, 1, false, 4, true>(K_GEMM_PLANE, a, s);
        case GEMM_F2_MP:
            // the held-activation kernel with each path's h folded into its
            // signs, when the paths' ranks fit it; else one flush per path
            if (as && a.N % AS_BN == 0 && (a.path_k == 128 || a.path_k == 256)) {
                switch (a.K / 128 * 10 + a.path_k / 128) {
                    case 21: return launch_gemm_as_t<2, false, true, false, 1>(K_GEMM_F2, a, s);
                    case 31: return launch_gemm_as_t<3, false, true, false, 1>(K_GEMM_F2, a, s);
                    case 41: return launch_gemm_as_t<4, false, true, false, 1>(K_GEMM_F2, a, s);
                    case 42: return launch_gemm_as_t<4, false, true, false, 2>(K_GEMM_F2, a, s);
                }
            }
            return launch_gemm_t<64, 128, 1, 4, 2, 2, false, true, false, 8, false, 4, false, true>(K_GEMM_F2, a, s);
        case GEMM_B2_MP:
            // the held-activation kernel, each path's product in turn, when
            // the paths' ranks fit its block; else one flush per path
            if (wide && a.K <= 1024 && a.path_k % 128 == 0) {
                switch (a.K / 128 * 10 + a.path_k / 128) {
                    case 21: return launch_gemm_as_paths_t<1, 2>(K_GEMM_B2, a, s);
                    case 31: return launch_gemm_as_paths_t<1, 3>(K_GEMM_B2, a, s);
                    case 41: return launch_gemm_as_paths_t<1, 4>(K_GEMM_B2, a, s);
                    case 42: return launch_gemm_as_paths_t<2, 2>(K_GEMM_B2, a, s);
                    case 62: return launch_gemm_as_paths_t<2, 3>(K_GEMM_B2, a, s);
                    case 63: return launch_gemm_as_paths_t<3, 2>(K_GEMM_B2, a, s);
                    case 82: return launch_gemm_as_paths_t<2, 4>(K_GEMM_B2, a, s);
                    case 84: return launch_gemm_as_paths_t<4, 2>(K_GEMM_B2, a, s);
                }
            }
            return launch_gemm_t<64, 128, 1, 4, 2, 2, false, true, true, 8, false, 4, false, true>(K_GEMM_B2, a, s);
        case GEMM_B1_DH: {
            // 64 tokens x 128 or 256 ranks of one path, 64 per wave
            const int pn = a.path_n ? a.path_n : a.N;
            switch (b1dh_cols(a.M, pn, a.N / pn)) {
                case 128: return launch_gemm_t<64, 128, 1, 2, 2, 1, true, false, true, 1, true>(K_GEMM_B1_DH, a, s);
                case 256: return launch_gemm_t<64, 256, 1, 4, 2, 1, true, false, true, 1, true>(K_GEMM_B1_DH, a, s);
            }
            return hipErrorInvalidValue;
        }
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Sign gradients (page: `blr_backward` with sign state, `cvt_t` staging):
// contractions over the tokens of two [T][*] activations,
//   out[m][n] (+)= (sum_t f16(A[t][m] acol[m] ascale) f16(B[t][n] bcol[n] bscale)) oscale.
// 128x128 tiles, 8 waves. Per step of 32 tokens, waves 0-3 stage A and
// waves 4-7 stage B: each thread loads a 4-token x 4-column block (a wave's
// loads cover 8 rows x 128 bytes), scales and rounds it to f16 and writes it
// transposed ([column][token]) into LDS, so both MFMA operands read 8
// consecutive tokens per lane. A register ring keeps the loads TP - 1 steps
// ahead; two LDS buffers; tokens past T are zero (only the last step checks).
// The 8 waves multiply in a 4x2 layout of 32x64 blocks. One launch serves
// both gradients.
constexpr int TN_BM = 128, TN_BN = 128, TN_LDK = 32;
__global__ __launch_bounds__(512, 2) void gemm_tn_kernel(TnJobs jobs) {
    __shared__ __attribute__((aligned(16))) _Float16 As[2][TN_BM * TN_LDK];
    __shared__ __attribute__((aligned(16))) _Float16 Bs[2][TN_BN * TN_LDK];
    // consecutive tiles (the N tiles of an M tile first) on one XCD: its
    // workgroups share their A columns and the B operand in its L2
    const int G = gridDim.x;
    int b = (G % NUM_XCD == 0) ? (int)(blockIdx.x % NUM_XCD) * (G / NUM_XCD) + (int)(blockIdx.x / NUM_XCD)
                               : (int)blockIdx.x;
    int j = 0;
    while (j + 1 < jobs.count && b >= jobs.job[j + 1].tiles_before) ++j;
    const TnJob &jb = jobs.job[j];
    b -= jb.tiles_before;
    const int ntn = jb.No / TN_BN;
    const int mt = b / ntn, nt = b - mt * ntn;
    const int m0 = mt * TN_BM, n0 = nt * TN_BN;
    const int64_t T = jobs.T;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;   // 32-row x 64-column MMA block
    const bool bside = wave >= 4;              // stages B (else A)
    // staging block: tokens 4*tb .. +3 of the step, columns 4*cb .. +3 of the
    // tile; consecutive lanes take consecutive column groups of one token row,
    // so each group of lanes reads whole 128-byte lines
    const int tb = lane >> 3, cb = (wave & 3) * 8 + (lane & 7);
    const float *col = bside ? jb.bcol + n0 : jb.acol + m0;
    const float sc = bside ? jb.bscale : jb.ascale;
    f32x4_t cs;
#pragma unroll
    for (int e = 0; e < 4; ++e) cs[e] = col[4 * cb + e] * sc;
    const int64_t ld = bside ? jb.ldb : jb.lda;
    const float *src = (bside ? jb.B + n0 : jb.A + m0) + 4 * cb;
    // the tiles are [column][32 tokens] f16 with no pad; the 8-token chunk c of
    // column n sits at chunk c ^ ((n >> 2) & 3) (two passes for the 8-byte
    // writes, conflict-free 16-byte fragment reads)
    _Float16 *dst0 = (bside ? &Bs[0][0] : &As[0][0]) + 4 * cb * TN_LDK + 8 * ((tb >> 1) ^ (cb & 3)) + 4 * (tb & 1);
    constexpr int BUFH = TN_BM * TN_LDK;  // halves per buffer (A and B alike)
    const int64_t nk = (T + 31) / 32;
    constexpr int TP = 4;
    f32x4_t rg[TP][4];
#define TN_LOAD(q, kt)                                                                     \
    do {                                                                                   \
        const int64_t k_ = (kt) < nk ? (kt) : nk - 1;                                      \
        const int64_t t0_ = k_ * 32 + 4 * tb;                                              \
        if (k_ * 32 + 32 <= T) {                                                           \
            _Pragma("unroll") for (int e = 0; e < 4; ++e)                                  \
                rg[q][e] = *reinterpret_cast<const f32x4_t *>(src + (t0_ + e) * ld);       \
        } else {                                                                           \
            _Pragma("unroll") for (int e = 0; e < 4; ++e) {                                \
                const int64_t tc_ = t0_ + e < T ? t0_ + e : T - 1;                         \
                const f32x4_t v_ = *reinterpret_cast<const f32x4_t *>(src + tc_ * ld);     \
                const f32x4_t z_ = {0.f, 0.f, 0.f, 0.f};                                   \
                rg[q][e] = t0_ + e < T ? v_ : z_;                                          \
            }                                                                              \
        }                                                                                  \
    } while (0)
#define TN_STORE(q, buf)                                                                   \
    do {                                                                                   \
        _Pragma("unroll") for (int c_ = 0; c_ < 4; ++c_) {                                 \
            uint2 h_;                                                                      \
            h_.x = f16x2_scaled(rg[q][0][c_], cs[c_], rg[q][1][c_], cs[c_]);               \
            h_.y = f16x2_scaled(rg[q][2][c_], cs[c_], rg[q][3][c_], cs[c_]);               \
            *reinterpret_cast<uint2 *>(dst0 + (buf) * BUFH + c_ * TN_LDK) = h_;            \
        }                                                                                  \
    } while (0)
    f32x16_t acc[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[jj][v] = 0.0f;
#pragma unroll
    for (int q = 0; q < TP; ++q) TN_LOAD(q, q);
    TN_STORE(0, 0);
    TN_LOAD(0, TP);
    __syncthreads();
    const int fsw = (lane >> 2) & 3;  // the permutation of the lane's columns
    const int aro = (wm * 32 + (lane & 31)) * TN_LDK;
    const int bro = (wn * 64 + (lane & 31)) * TN_LDK;
    for (int64_t kt0 = 0; kt0 < nk; kt0 += TP) {
#pragma unroll
        for (int u = 0; u < TP; ++u) {
            const int64_t kt = kt0 + u;
            if (kt >= nk) break;  // uniform
            const int cur = (int)(kt & 1);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int ko = 8 * (((lane >> 5) + 2 * s) ^ fsw);
                const half8_t fa = *reinterpret_cast<const half8_t *>(&As[cur][aro + ko]);
                half8_t fb[2];
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    fb[jj] = *reinterpret_cast<const half8_t *>(&Bs[cur][bro + jj * 32 * TN_LDK + ko]);
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    acc[jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa, fb[jj], acc[jj], 0, 0, 0);
            }
            TN_STORE((u + 1) % TP, cur ^ 1);
            TN_LOAD((u + 1) % TP, kt + 1 + TP);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#undef TN_LOAD
#undef TN_STORE
    // out rows m0 + wm*32 + 8*(v/4) + 4*(lane/32) + v%4, columns
    // n0 + wn*64 + jj*32 + lane%32
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        float *o = jb.out + row * jb.No + n0 + wn * 64 + (lane & 31);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const float val = acc[jj][v] * jb.oscale;
            o[jj * 32] = jb.acc ? o[jj * 32] + val : val;
        }
    }
}

// The same contractions on 256x256 tiles, the tokens split into `splits`
// ranges of tps tokens (a multiple of 32) so that the few large tiles still
// fill the GPU. Range 0 writes (or adds to) `out`; every later range stores
// its partial sums in the workspace, and sign_reduce_kernel then adds them
// to `out` in range order, so the result does not depend on which range
// finishes first (no atomics: reruns give identical bits). Per output element and token
// this reads 8 bytes of activations for 256 + 256 products, half the bytes
// per product of the 128x128 tiling. Blocks: job, then range, then tile, so
// the tiles of one (job, range) run on one XCD and share their B rows and
// their A columns in its L2. 8 waves in a 4x2 layout of 64x128 blocks; per
// step of 32 tokens each thread stages a 4-token x 4-column block of both
// operands (rounded to f16, transposed into LDS), two register stages ahead.
constexpr int TN2_T = 256, TN2_LDK = 32, TN2_TP = 2;
__global__ __launch_bounds__(512, 1) void gemm_tn2_kernel(TnJobs jobs, int64_t tps, int64_t part_stride) {
    __shared__ __attribute__((aligned(16))) _Float16 As[2][TN2_T * TN2_LDK];
    __shared__ __attribute__((aligned(16))) _Float16 Bs[2][TN2_T * TN2_LDK];
    const int G = gridDim.x;
    int b = (G % NUM_XCD == 0) ? (int)(blockIdx.x % NUM_XCD) * (G / NUM_XCD) + (int)(blockIdx.x / NUM_XCD)
                               : (int)blockIdx.x;
    int j = 0;
    while (j + 1 < jobs.count && b >= jobs.job[j + 1].tiles_before) ++j;
    const TnJob &jb = jobs.job[j];
    b -= jb.tiles_before;
    const int ntn = jb.No / TN2_T, tiles = (jb.Mo / TN2_T) * ntn;
    const int sp = b / tiles, tl = b - sp * tiles;
    const int mt = tl / ntn, nt = tl - mt * ntn;
    const int m0 = mt * TN2_T, n0 = nt * TN2_T;
    const int64_t T = jobs.T;
    const int64_t tb0 = (int64_t)sp * tps;                       // first token of the range
    const int64_t tend = tb0 + tps < T ? tb0 + tps : T;          // one past its last
    if (tb0 >= tend) return;  // an empty range (uniform per workgroup)
    const int64_t nk = (tend - tb0 + 31) / 32;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;  // 64 A columns x 128 B columns
    // staging block: tokens 4*tq .. +3 of the step, columns 4*cq .. +3 of both
    // tiles; consecutive lanes take consecutive column groups of one token row,
    // so each group of lanes reads whole 128-byte lines
    const int tq = lane >> 3, cq = wave * 8 + (lane & 7);
    f32x4_t csa, csb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        csa[e] = jb.acol[m0 + 4 * cq + e] * jb.ascale;
        csb[e] = jb.bcol[n0 + 4 * cq + e] * jb.bscale;
    }
    // (the job's fields in registers: read from the argument block once)
    const int64_t lda = jb.lda, ldb = jb.ldb;
    const int No = jb.No, accf = jb.acc;
    const float osc = jb.oscale;
    float *const outp = jb.out;
    // the tiles are [column][32 tokens] f16 with no pad; the 8-token chunk c of
    // column n sits at chunk c ^ ((n >> 2) & 3), which keeps the stagers'
    // 8-byte writes at two passes and the fragments' 16-byte reads
    // conflict-free on gfx950 (measured)
    const int wofs = 4 * cq * TN2_LDK + 8 * ((tq >> 1) ^ (cq & 3)) + 4 * (tq & 1);
    f32x4_t ra[TN2_TP][4], rb[TN2_TP][4];
    // Buffer loads: a token row at or past T lies past the buffer's range
    // and reads as zero (only the last range has a partial step; the others
    // end on a multiple of 32 tokens); byte offsets of tokens 4 tq + e of the
    // range's first step, advanced by whole steps
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(jb.A, (uint64_t)T * lda * 4);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(jb.B, (uint64_t)T * ldb * 4);
    uint32_t oa[4], ob[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        oa[e] = (uint32_t)(((tb0 + 4 * tq + e) * lda + m0 + 4 * cq) * 4);
        ob[e] = (uint32_t)(((tb0 + 4 * tq + e) * ldb + n0 + 4 * cq) * 4);
    }
#define TN2_LOAD(q, kt)                                                                    \
    do {                                                                                   \
        const uint32_t k_ = (uint32_t)((kt) < nk ? (kt) : nk - 1);                         \
        const uint32_t sa_ = k_ * (uint32_t)(32 * lda * 4), sb_ = k_ * (uint32_t)(32 * ldb * 4); \
        _Pragma("unroll") for (int e = 0; e < 4; ++e) {                                    \
            ra[q][e] = load_f32x4(rA, oa[e] + sa_, 0u);                                    \
            rb[q][e] = load_f32x4(rB, ob[e] + sb_, 0u);                                    \
        }                                                                                  \
    } while (0)
#define TN2_STORE(q, buf)                                                                  \
    do {                                                                                   \
        _Pragma("unroll") for (int c_ = 0; c_ < 4; ++c_) {                                 \
            uint2 ha_, hb_;                                                                \
            ha_.x = f16x2_scaled(ra[q][0][c_], csa[c_], ra[q][1][c_], csa[c_]);            \
            ha_.y = f16x2_scaled(ra[q][2][c_], csa[c_], ra[q][3][c_], csa[c_]);            \
            hb_.x = f16x2_scaled(rb[q][0][c_], csb[c_], rb[q][1][c_], csb[c_]);            \
            hb_.y = f16x2_scaled(rb[q][2][c_], csb[c_], rb[q][3][c_], csb[c_]);            \
            *reinterpret_cast<uint2 *>(&As[buf][wofs + c_ * TN2_LDK]) = ha_;               \
            *reinterpret_cast<uint2 *>(&Bs[buf][wofs + c_ * TN2_LDK]) = hb_;               \
        }                                                                                  \
    } while (0)
    f32x16_t acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.0f;
#pragma unroll
    for (int q = 0; q < TN2_TP; ++q) TN2_LOAD(q, q);
    TN2_STORE(0, 0);
    TN2_LOAD(0, TN2_TP);
    __syncthreads();
    const int fsw = (lane >> 2) & 3;  // the permutation of the lane's columns
    const int aro = (wm * 64 + (lane & 31)) * TN2_LDK;
    const int bro = (wn * 128 + (lane & 31)) * TN2_LDK;
    for (int64_t kt0 = 0; kt0 < nk; kt0 += TN2_TP) {
#pragma unroll
        for (int u = 0; u < TN2_TP; ++u) {
            const int64_t kt = kt0 + u;
            if (kt >= nk) break;  // uniform
            const int cur = (int)(kt & 1);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                half8_t fa[2], fb[4];
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    fa[i] = *reinterpret_cast<const half8_t *>(
                        &As[cur][aro + i * 32 * TN2_LDK + 8 * (((lane >> 5) + 2 * ks) ^ fsw)]);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    fb[jj] = *reinterpret_cast<const half8_t *>(
                        &Bs[cur][bro + jj * 32 * TN2_LDK + 8 * (((lane >> 5) + 2 * ks) ^ fsw)]);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[jj], acc[i][jj], 0, 0, 0);
            }
            TN2_STORE((u + 1) % TN2_TP, cur ^ 1);
            TN2_LOAD((u + 1) % TN2_TP, kt + 1 + TN2_TP);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#undef TN2_LOAD
#undef TN2_STORE
    // out row m0 + wm*64 + i*32 + 8*(v/4) + 4*(lane/32) + v%4, column
    // n0 + wn*128 + jj*32 + lane%32: range 0 stores (or accumulates) into
    // out, range sp > 0 stores into its slice of the partials
    float *const o0 = (sp == 0 ? outp : jobs.part + (int64_t)(sp - 1) * part_stride + jb.elems_before) +
                      (int64_t)(m0 + wm * 64 + 4 * (lane >> 5)) * No + n0 + wn * 128 + (lane & 31);
#define TN2_EPI(OP)                                                                        \
    _Pragma("unroll") for (int i = 0; i < 2; ++i)                                          \
        _Pragma("unroll") for (int v = 0; v < 16; ++v)                                     \
            _Pragma("unroll") for (int jj = 0; jj < 4; ++jj) {                             \
                float *o = o0 + (int64_t)(i * 32 + 8 * (v >> 2) + (v & 3)) * No + jj * 32; \
                const float val = acc[i][jj][v] * osc;                                     \
                OP;                                                                        \
            }
    if (sp == 0 && accf) {
        TN2_EPI(*o += val)
    } else {
        TN2_EPI(*o = val)
    }
#undef TN2_EPI
}

// out += partials of token ranges 1 .. splits-1, in range order, for every
// job's output (float4 groups over the jobs' outputs back to back; every
// Mo * No is a multiple of 4).
__global__ __launch_bounds__(256) void sign_reduce_kernel(TnJobs jobs, int splits, int64_t part_stride) {
    const int64_t n4 = part_stride / 4;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
        const int64_t e = 4 * i;
        int j = 0;
        while (j + 1 < jobs.count && e >= jobs.job[j + 1].elems_before) ++j;
        f32x4_t *o = reinterpret_cast<f32x4_t *>(jobs.job[j].out + (e - jobs.job[j].elems_before));
        f32x4_t v = *o;
        for (int s = 1; s < splits; ++s) v += *reinterpret_cast<const f32x4_t *>(jobs.part + (int64_t)(s - 1) * part_stride + e);
        *o = v;
    }
}

int sign_splits(int64_t tiles256, int64_t T) {
    if (tiles256 < 1 || T < 1) return 1;
    const int64_t steps = (T + 31) / 32;
    int64_t splits = (256 + tiles256 - 1) / tiles256;
    if (splits > steps / 16) splits = steps / 16;
    return splits < 1 ? 1 : (int)splits;
}

hipError_t launch_gemm_tn(TnJobs jobs, hipStream_t s) {
    if (jobs.T < 1) return hipErrorInvalidValue;
    bool big = true;
    for (int j = 0; j < jobs.count; ++j) {
        if (jobs.job[j].Mo % TN_BM || jobs.job[j].No % TN_BN) return hipErrorInvalidValue;
        if (jobs.job[j].Mo % TN2_T || jobs.job[j].No % TN2_T) big = false;
    }
    int64_t elems = 0;
    for (int j = 0; j < jobs.count; ++j) {
        jobs.job[j].elems_before = elems;
        elems += (int64_t)jobs.job[j].Mo * jobs.job[j].No;
    }
    if (big) {
        // tiles of all jobs, then as many token ranges (of at least 512
        // tokens) as bring the workgroups to about 256
        int tiles = 0;
        for (int j = 0; j < jobs.count; ++j) tiles += (jobs.job[j].Mo / TN2_T) * (jobs.job[j].No / TN2_T);
        const int64_t steps = (jobs.T + 31) / 32;
        const int splits = sign_splits(tiles, jobs.T);
        if (splits > 1 && jobs.part == nullptr) return hipErrorInvalidValue;
        const int64_t tps = ((steps + splits - 1) / splits) * 32;
        int total = 0;
        for (int j = 0; j < jobs.count; ++j) {
            jobs.job[j].tiles_before = total;
            total += (jobs.job[j].Mo / TN2_T) * (jobs.job[j].No / TN2_T) * splits;
        }
        prof_begin(K_GEMM_SIGNS, s);
        hipLaunchKernelGGL(gemm_tn2_kernel, dim3((unsigned)total), dim3(512), 0, s, jobs, tps, elems);
        hipError_t e = hipGetLastError();
        prof_end(s);
        if (e != hipSuccess || splits == 1) return e;
        int64_t blocks = (elems / 4 + 255) / 256;
        if (blocks > 2048) blocks = 2048;
        prof_begin(K_SIGNS_REDUCE, s);
        hipLaunchKernelGGL(sign_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, jobs, splits, elems);
        e = hipGetLastError();
        prof_end(s);
        return e;
    }
    int total = 0;
    for (int j = 0; j < jobs.count; ++j) {
        jobs.job[j].tiles_before = total;
        total += (jobs.job[j].Mo / TN_BM) * (jobs.job[j].No / TN_BN);
    }
    prof_begin(K_GEMM_SIGNS, s);
    hipLaunchKernelGGL(gemm_tn_kernel, dim3((unsigned)total), dim3(512), 0, s, jobs);
    hipError_t e = hipGetLastError();
    prof_end(s);
    return e;
}

// ---------------------------------------------------------------------------
// Sum of squares (page: `sumsq` shader, the host's finite check): nparts
// workgroups of 256 threads; thread t of workgroup p adds the squares of the
// float4 groups p*256 + t + k*nparts*256 in order (workgroup 0 also takes the
// n % 4 tail), then the 256 sums fold in a fixed tree. Non-finite values
// propagate into the partial.
__global__ __launch_bounds__(256) void sumsq_kernel(const float *__restrict__ a, int64_t n,
                                                    float *__restrict__ partials) {
    __shared__ float red[256];
    const int t = threadIdx.x;
    const int64_t n4 = n / 4;
    const int64_t stride = (int64_t)gridDim.x * 256;
    float acc = 0.0f;
    for (int64_t c = (int64_t)blockIdx.x * 256 + t; c < n4; c += stride) {
        const f32x4_t v = reinterpret_cast<const f32x4_t *>(a)[c];
        acc += v.x * v.x;
        acc += v.y * v.y;
        acc += v.z * v.z;
        acc += v.w * v.w;
    }
    if (blockIdx.x == 0 && t < n - n4 * 4) {
        const float v = a[n4 * 4 + t];
        acc += v * v;
    }
    red[t] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (t < w) red[t] = red[t] + red[t + w];
        __syncthreads();
    }
    if (t == 0) partials[blockIdx.x] = red[0];
}

hipError_t launch_sumsq(const float *a, int64_t n, float *partials, int nparts, hipStream_t s) {
    prof_begin(K_SUMSQ, s);
    hipLaunchKernelGGL(sumsq_kernel, dim3((unsigned)nparts), dim3(256), 0, s, a, n, partials);
    hipError_t e = hipGetLastError();
    prof_end(s);
    return e;
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
// one launch. Each workgroup owns 32 columns of one job; its 8 groups of 32
// lanes take every 8th part, 16 loads in flight at a time, each adding its
// parts in order; then the 8 group sums are added in group order. The order
// is fixed, so results are deterministic.
constexpr int FIN_COLS = 32;
__global__ __launch_bounds__(256) void finish_kernel(FinishJobs jobs) {
    __shared__ float red[8][FIN_COLS];
    int b = blockIdx.x, j = 0;
    while (j + 1 < jobs.count && b >= jobs.blocks_before[j + 1]) ++j;
    const FinishJob &jb = jobs.job[j];
    const float *__restrict__ partial = jb.partial;
    const int64_t nparts = jb.nparts;
    const int N = jb.N;
    const int c = threadIdx.x & (FIN_COLS - 1), q = threadIdx.x / FIN_COLS;
    const int col = (b - jobs.blocks_before[j]) * FIN_COLS + c;
    float s = 0.0f;
    if (col < N) {
        int64_t pi = q;
        for (; pi + 15 * 8 < nparts; pi += 16 * 8) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = partial[(pi + 8 * u) * N + col];
#pragma unroll
            for (int u = 0; u < 16; ++u) s += v[u];
        }
        for (; pi < nparts; pi += 8) s += partial[pi * N + col];
    }
    red[q][c] = s;
    __syncthreads();
    if (q == 0 && col < N) {
        float t = red[0][c];
#pragma unroll
        for (int g = 1; g < 8; ++g) t += red[g][c];
        jb.out[col] = jb.out[col] + t;
    }
}

hipError_t launch_finish(FinishJobs jobs, hipStream_t s) {
    int total = 0;
    for (int j = 0; j < jobs.count; ++j) {
        jobs.blocks_before[j] = total;
        total += (jobs.job[j].N + FIN_COLS - 1) / FIN_COLS;
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
        case K_GEMM_B1_DH: return "gemm_b1_dh_fused";
        case K_GEMM_SIGNS: return "gemm_sign_grads";
        case K_SUMSQ: return "sumsq";
        case K_GEMM_PLANE: return "gemm_plane_linear";
        case K_SIGNS_REDUCE: return "sign_grads_reduce";
    }
    return "?";
}

}  // namespace blr
