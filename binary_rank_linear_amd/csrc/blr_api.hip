// C ABI of the `blr` layer (include/blr.h): argument validation, workspace
// layout and launch order on the caller's stream. The order of the steps is
// the one of `blr_forward` / `blr_backward` on the cortiq-engine page
// "src/gpu_wgpu/train_mm.rs"; their staging and scaling passes live inside
// the contraction kernels.
#include <math.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/blr.h"
#include "blr_internal.h"

namespace blr {

// ------------------------------------------------------------ profiling --
namespace {
struct ProfState {
    bool on = false;
    std::vector<hipEvent_t> ev;  // pairs
    std::vector<int> ids;        // kernel id per recorded pair
    size_t used = 0;
    int pending_id = -1;
    int64_t counts[K_COUNT] = {};
    double total_ms[K_COUNT] = {};
};
ProfState g_prof;
std::mutex g_prof_mu;

void prof_release() {
    for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
    g_prof.ev.clear();
    g_prof.ids.clear();
    g_prof.used = 0;
    g_prof.on = false;
}
}  // namespace

void prof_begin(int id, hipStream_t s) {
    if (!g_prof.on) return;
    g_prof.pending_id = -1;
    if (2 * (g_prof.used + 1) > g_prof.ev.size()) return;  // pool full: launch goes untimed
    (void)hipEventRecord(g_prof.ev[2 * g_prof.used], s);
    g_prof.pending_id = id;
}

void prof_end(hipStream_t s) {
    if (!g_prof.on || g_prof.pending_id < 0) return;
    (void)hipEventRecord(g_prof.ev[2 * g_prof.used + 1], s);
    g_prof.ids.push_back(g_prof.pending_id);
    g_prof.used += 1;
    g_prof.pending_id = -1;
}

// ------------------------------------------------------------ workspace --
namespace {
constexpr size_t ALIGN = 256;
size_t up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

struct Layout {
    size_t bits_t;  // transposed bitmaps [P][r][max(d_in, d_out)/32] (u32)
    size_t db;      // f32 [M][P r]
    size_t part_h, part_l, part_g;
    size_t part_s;  // sign gradients: partials of token ranges 1.. (f32)
    size_t total;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// P paths (1 for a plain layer); the paths' ranks lie side by side.
Layout layout(int64_t M, int64_t d_in, int64_t d_out, int64_t r, int64_t P = 1) {
    Layout L;
    size_t off = 0;
    L.bits_t = off;
    off += up((size_t)(P * r * ((d_in > d_out ? d_in : d_out) / 32)) * 4);
    L.db = off;
    off += up((size_t)(M * P * r) * 4);
    // dh partials per path: ceil(M/64) rows from the c-tape column sum or the
    // recomputed-c contraction, ceil(M/64) per rank tile from B1 with dh
    // fused (up to four tiles of 128 ranks); dl partials: one row per 32
    // tokens; dg partials: one row per 64 tokens and path
    const int64_t bc = b1dh_cols(M, r, P);
    const int64_t hrows = ceil_div(M, GEMM_BM_MIN) * (bc ? r / bc : 1);
    L.part_h = off;
    off += up((size_t)(P * hrows * d_out) * 4);
    L.part_l = off;
    off += up((size_t)(ceil_div(M, PART_ROWS_MIN) * P * r) * 4);
    L.part_g = off;
    off += up((size_t)(P * ceil_div(M, GEMM_BM_MIN) * d_in) * 4);
    // the sign gradients' token ranges past the first (256 x 256 tiles only):
    // (splits - 1) copies of G_U and G_V, under 64 MB whatever the shape
    // (splits * tiles stays near 256)
    L.part_s = off;
    if (d_in % 256 == 0 && d_out % 256 == 0 && r % 256 == 0) {
        const int64_t tiles = P * ((d_out / 256) * (r / 256) + (d_in / 256) * (r / 256));
        const int64_t splits = sign_splits(tiles, M);
        off += up((size_t)((splits - 1) * P * (d_out + d_in) * r) * 4);
    }
    L.total = off;
    return L;
}

// Sizes the kernels accept: d_in, d_out, r multiples of 128 (the page's GEMM
// contract), M >= 1, and everything small enough for 32-bit grid and column
// indices.
bool shape_ok(int64_t M, int64_t d_in, int64_t d_out, int64_t r, int64_t P = 1) {
    if (P < 1 || P > MAX_PATHS) return false;
    if (P > 1) {
        // the paths' ranks side by side are one operand dimension
        if (!shape_ok(M, d_in, d_out, P * r)) return false;
    }
    if (M < 1 || d_in < 128 || d_out < 128 || r < 128) return false;
    if (d_in % 128 || d_out % 128 || r % 128) return false;
    const int64_t LIM = (int64_t)1 << 24;  // ranks
    if (r > LIM) return false;
    if ((d_in + 63) / 64 > 65535 || (d_out + 63) / 64 > 65535) return false;  // expansion grid rows
    if (ceil_div(M, COLSUM_ROWS) > 65535) return false;
    // the contraction kernels address every operand with 32-bit byte offsets
    const int64_t widest = d_in > d_out ? (d_in > r ? d_in : r) : (d_out > r ? d_out : r);
    if (M * widest * 4 > (int64_t)0xFFFFFFFF) return false;
    if ((d_out / 128) * ceil_div(M, GEMM_BM_MIN) > ((int64_t)1 << 31) - 1) return false;
    if ((d_in / 128) * ceil_div(M, GEMM_BM_MIN) > ((int64_t)1 << 31) - 1) return false;
    return true;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

bool pow2_scale_ok(float s) {
    if (!(s > 0.0f) || !isfinite(s)) return false;
    int e;
    return frexpf(s, &e) == 0.5f;
}

int g_supported[64];  // 0 unknown, 1 yes, -1 no
std::mutex g_dev_mu;

int current_device_ok() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return BLR_ERR_HIP;
    if (dev < 0 || dev >= 64) return blr_device_supported(dev) ? BLR_OK : BLR_ERR_DEVICE;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_supported[dev] == 0) g_supported[dev] = blr_device_supported(dev) ? 1 : -1;
    return g_supported[dev] == 1 ? BLR_OK : BLR_ERR_DEVICE;
}

#define BLR_TRY(expr)                                   \
    do {                                                \
        if ((expr) != hipSuccess) return BLR_ERR_HIP;   \
    } while (0)
}  // namespace

}  // namespace blr

using namespace blr;

extern "C" {

const char *blr_status_string(int status) {
    switch (status) {
        case BLR_OK: return "ok";
        case BLR_ERR_NULL: return "a required pointer is NULL";
        case BLR_ERR_SHAPE: return "invalid shape (d_in, d_out, r must be multiples of 128; M >= 1)";
        case BLR_ERR_SCALE: return "gscale must be a positive finite power of two";
        case BLR_ERR_WORKSPACE: return "workspace missing or smaller than blr_workspace_bytes()";
        case BLR_ERR_DEVICE: return "the current device is not gfx950";
        case BLR_ERR_HIP: return "HIP runtime error";
        case BLR_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case BLR_ERR_SCRATCH: return "sizes need more than the allocation-free forward's scratch (r * d_in / 8 bytes)";
    }
    return "unknown status";
}

int blr_device_supported(int hip_device) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, hip_device) != hipSuccess) return 0;
    return strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
}

size_t blr_workspace_bytes(int64_t M, int64_t d_in, int64_t d_out, int64_t r) {
    if (!shape_ok(M, d_in, d_out, r)) return 0;
    return layout(M, d_in, d_out, r).total;
}

int blr_expand_signs(const uint32_t *bits, int64_t rows, int64_t r, uint16_t *plane, uint16_t *plane_t,
                     void *stream) {
    if (bits == nullptr || (plane == nullptr && plane_t == nullptr)) return BLR_ERR_NULL;
    if (rows < 1 || r < 1 || (rows + 63) / 64 > 65535 || r > ((int64_t)1 << 30) || rows * r > ((int64_t)1 << 40))
        return BLR_ERR_SHAPE;
    if (!aligned4(bits) || (plane && !aligned16(plane)) || (plane_t && !aligned16(plane_t))) return BLR_ERR_ALIGN;
    int st = current_device_ok();
    if (st != BLR_OK) return st;
    ExpandJobs jobs = {};
    jobs.job[0] = {bits, rows, r, plane, plane_t};
    jobs.count = 1;
    return launch_expand(jobs, (hipStream_t)stream) == hipSuccess ? BLR_OK : BLR_ERR_HIP;
}

// A layer of P paths (P = 1: the plain layer). Path p's operands are the
// p-th blocks of bits_u [P][d_out][r/32], bits_v [P][d_in][r/32],
// h [P][d_out], l [P][r], g [P][d_in]; the a tape is [M][P r] (the paths'
// ranks side by side). F1 runs once over the concatenated ranks; F2 runs
// once with the paths along K (one flush per path) when P > 1.
// Arguments of the forward, workspace aside.
static int forward_check(int64_t M, int64_t d_in, int64_t d_out, int64_t r, int64_t P, const float *x,
                         const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                         const float *g, const float *y, const float *tape_a, const float *tape_c) {
    if (!x || !bits_u || !bits_v || !h || !l || !g || !y || !tape_a) return BLR_ERR_NULL;
    if (!shape_ok(M, d_in, d_out, r, P)) return BLR_ERR_SHAPE;
    if (P > 1 && tape_c) return BLR_ERR_SHAPE;  // no c tape for several paths
    const void *f16a[] = {x, h, l, g, y, tape_a, tape_c ? tape_c : tape_a};
    for (const void *p : f16a)
        if (!aligned16(p)) return BLR_ERR_ALIGN;
    if (!aligned16(bits_u) || !aligned16(bits_v)) return BLR_ERR_ALIGN;
    return BLR_OK;
}

// The forward's launches, after validation. bits_vt: room for the
// transposed S_V bitmaps, [P][r][d_in/32] u32 (16-byte aligned), the only
// scratch the forward uses.
static int forward_launch(int64_t M, int64_t d_in, int64_t d_out, int64_t r, int64_t P, const float *x,
                          const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                          const float *g, float *y, int accumulate_y, float *tape_a, float *tape_c,
                          uint32_t *bits_vt, hipStream_t s) {
    BLR_TRY(launch_transpose_bits(bits_v, d_in, r, bits_vt, s, (int)P));

    GemmArgs f1 = {};
    f1.A = x;
    f1.lda = d_in;
    f1.colscale = g;
    f1.ascale = 1.0f;
    f1.Bbits = bits_vt;
    f1.M = M;
    f1.N = (int)(P * r);
    f1.K = (int)d_in;
    f1.oscale = 1.0f;
    f1.out = tape_a;
    if (P > 1) {
        f1.path_n = (int)r;      // path n0 / r: x staged with g_p
        f1.cs_pstride = d_in;
    }
    BLR_TRY(launch_gemm(GEMM_F1, f1, s));

    GemmArgs f2 = {};
    f2.A = tape_a;
    f2.lda = P * r;
    f2.colscale = l;
    f2.ascale = 1.0f;
    f2.Bbits = bits_u;
    f2.M = M;
    f2.N = (int)d_out;
    f2.K = (int)(P * r);
    f2.oscale = 1.0f;
    f2.out = tape_c;
    f2.out2 = y;
    f2.out2col = h;
    f2.out2acc = accumulate_y ? 1 : 0;
    if (P > 1) {
        f2.path_k = (int)r;                 // S_U of path q: bits_u + q d_out r/32 words
        f2.b_pstride = d_out * (r / 32);
        f2.o2_pstride = d_out;              // h_q
        BLR_TRY(launch_gemm(GEMM_F2_MP, f2, s));
    } else {
        BLR_TRY(launch_gemm(tape_c ? GEMM_F2 : GEMM_F2_NOTAPE, f2, s));
    }
    return BLR_OK;
}

static int forward_impl(int64_t M, int64_t d_in, int64_t d_out, int64_t r, int64_t P, const float *x,
                        const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                        const float *g, float *y, int accumulate_y, float *tape_a, float *tape_c, void *workspace,
                        size_t workspace_bytes, void *stream) {
    int st = forward_check(M, d_in, d_out, r, P, x, bits_u, bits_v, h, l, g, y, tape_a, tape_c);
    if (st != BLR_OK) return st;
    const Layout L = layout(M, d_in, d_out, r, P);
    if (workspace == nullptr || workspace_bytes < L.total) return BLR_ERR_WORKSPACE;
    if (!aligned16(workspace)) return BLR_ERR_ALIGN;
    st = current_device_ok();
    if (st != BLR_OK) return st;
    uint32_t *bits_vt = (uint32_t *)((char *)workspace + L.bits_t);  // S_V^T per path, [P][r][d_in/32]
    return forward_launch(M, d_in, d_out, r, P, x, bits_u, bits_v, h, l, g, y, accumulate_y, tape_a, tape_c, bits_vt,
                          (hipStream_t)stream);
}

int blr_forward(int64_t M, int64_t d_in, int64_t d_out, int64_t r, const float *x, const uint32_t *bits_u,
                const uint32_t *bits_v, const float *h, const float *l, const float *g, float *y, int accumulate_y,
                float *tape_a, float *tape_c, void *workspace, size_t workspace_bytes, void *stream) {
    return forward_impl(M, d_in, d_out, r, 1, x, bits_u, bits_v, h, l, g, y, accumulate_y, tape_a, tape_c, workspace,
                        workspace_bytes, stream);
}

// ------------------------------------------------------ no allocation --
// The allocation-free forward's scratch: room for the transposed S_V bitmap.
// Each GPU the library runs on holds its own copy until the process ends.
// In host code this name is not a device address: the address each device
// uses comes from hipGetSymbolAddress (scratch_on_device below).
static __device__ __align__(256) uint8_t scratch[BLR_NOALLOC_SCRATCH_BYTES];

namespace {
void *g_scratch_ptr[64];  // per device, looked up on its first call
std::mutex g_scratch_mu;

int scratch_on_device(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return BLR_ERR_HIP;
    if (dev < 0 || dev >= 64) return BLR_ERR_DEVICE;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return BLR_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return BLR_OK;
}
}  // namespace

int blr_forward_noalloc(int64_t M, int64_t d_in, int64_t d_out, int64_t r, const float *x, const uint32_t *bits_u,
                        const uint32_t *bits_v, const float *h, const float *l, const float *g, float *y,
                        int accumulate_y, float *tape_a, float *tape_c, void *stream) {
    int st = forward_check(M, d_in, d_out, r, 1, x, bits_u, bits_v, h, l, g, y, tape_a, tape_c);
    if (st != BLR_OK) return st;
    if ((uint64_t)r * (uint64_t)d_in / 8 > (uint64_t)BLR_NOALLOC_SCRATCH_BYTES) return BLR_ERR_SCRATCH;
    st = current_device_ok();
    if (st != BLR_OK) return st;
    void *bits_vt = nullptr;
    st = scratch_on_device(&bits_vt);
    if (st != BLR_OK) return st;
    return forward_launch(M, d_in, d_out, r, 1, x, bits_u, bits_v, h, l, g, y, accumulate_y, tape_a, tape_c,
                          (uint32_t *)bits_vt, (hipStream_t)stream);
}

int blr_forward_paths(int64_t M, int64_t d_in, int64_t d_out, int64_t r, int64_t paths, const float *x,
                      const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l, const float *g,
                      float *y, int accumulate_y, float *tape_a, void *workspace, size_t workspace_bytes,
                      void *stream) {
    return forward_impl(M, d_in, d_out, r, paths, x, bits_u, bits_v, h, l, g, y, accumulate_y, tape_a, nullptr,
                        workspace, workspace_bytes, stream);
}

size_t blr_workspace_bytes_paths(int64_t M, int64_t d_in, int64_t d_out, int64_t r, int64_t paths) {
    if (!shape_ok(M, d_in, d_out, r, paths)) return 0;
    return layout(M, d_in, d_out, r, paths).total;
}

// The backward of P paths, and with grad_u / grad_v the sign gradients
// after it (both or neither). dh [P][d_out], dl [P][r], dg [P][d_in],
// grad_u [P][d_out][r], grad_v [P][d_in][r].
static int backward_impl(int64_t M, int64_t d_in, int64_t d_out, int64_t r, int64_t P, const float *x,
                         const float *dy, const uint32_t *bits_u, const uint32_t *bits_v, const float *h,
                         const float *l, const float *g, const float *tape_a, const float *tape_c, float gscale,
                         float *dh, float *dl, float *dg, float *dx, int accumulate_dx, float *grad_u, float *grad_v,
                         int accumulate_signs, void *workspace, size_t workspace_bytes, void *stream) {
    if (!x || !dy || !bits_u || !bits_v || !h || !l || !g || !tape_a || !dh || !dl || !dg || !dx)
        return BLR_ERR_NULL;
    if ((grad_u == nullptr) != (grad_v == nullptr)) return BLR_ERR_NULL;
    if (grad_u && (!aligned16(grad_u) || !aligned16(grad_v))) return BLR_ERR_ALIGN;
    if (!shape_ok(M, d_in, d_out, r, P)) return BLR_ERR_SHAPE;
    if (P > 1 && tape_c) return BLR_ERR_SHAPE;
    if (!pow2_scale_ok(gscale)) return BLR_ERR_SCALE;
    const Layout L = layout(M, d_in, d_out, r, P);
    if (workspace == nullptr || workspace_bytes < L.total) return BLR_ERR_WORKSPACE;
    const void *f16a[] = {x, dy, h, l, g, tape_a, tape_c ? tape_c : tape_a, dh, dl, dg, dx, workspace};
    for (const void *p : f16a)
        if (!aligned16(p)) return BLR_ERR_ALIGN;
    if (!aligned16(bits_u) || !aligned16(bits_v)) return BLR_ERR_ALIGN;
    int st = current_device_ok();
    if (st != BLR_OK) return st;

    hipStream_t s = (hipStream_t)stream;
    char *ws = (char *)workspace;
    uint32_t *bits_ut = (uint32_t *)(ws + L.bits_t);  // S_U^T per path, [P][r][d_out/32]
    float *db = (float *)(ws + L.db);                 // [M][P r]
    float *part_h = (float *)(ws + L.part_h);
    float *part_l = (float *)(ws + L.part_l);
    float *part_g = (float *)(ws + L.part_g);
    const float inv = 1.0f / gscale;  // exact: gscale is a power of two
    const int64_t Pr = P * r;
    const int64_t b1dh_c = b1dh_cols(M, r, P);
    const bool fused = tape_c == nullptr && b1dh_c > 0;  // B1 with dh fused
    const int64_t mt_b1 = ceil_div(M, fused ? b1dh_tile_rows(r) : gemm_tile_rows(GEMM_B1));
    const int64_t mt_b2 = ceil_div(M, gemm_tile_rows(P > 1 ? GEMM_B2_MP : GEMM_B2));

    BLR_TRY(launch_transpose_bits(bits_u, d_out, r, bits_ut, s, (int)P));

    // partials of dh_p = sum_t dy.c_p, nparts_h rows per path: inside B1
    // below, from the stored tape, or with c recomputed by F2's contraction
    // (same tiles, so the same c)
    int64_t nparts_h = 0;
    if (fused) {
        nparts_h = mt_b1 * (r / b1dh_c);  // one row per (rank tile, row tile) of the path
    } else if (tape_c) {
        BLR_TRY(launch_colsum(dy, tape_c, M, (int)d_out, part_h, s));
        nparts_h = ceil_div(M, COLSUM_ROWS);
    } else {
        nparts_h = ceil_div(M, gemm_tile_rows(GEMM_DH));
        for (int64_t q = 0; q < P; ++q) {
            GemmArgs rc = {};
            rc.A = tape_a + q * r;
            rc.lda = Pr;
            rc.colscale = l + q * r;
            rc.ascale = 1.0f;
            rc.Bbits = bits_u + q * d_out * (r / 32);
            rc.M = M;
            rc.N = (int)d_out;
            rc.K = (int)r;
            rc.oscale = 1.0f;
            rc.dot_other = dy;
            rc.dot_partial = part_h + q * nparts_h * d_out;
            BLR_TRY(launch_gemm(GEMM_DH, rc, s));
        }
    }

    // db_p = f16(dy.h_p.gs) S_U,p / gs for all paths side by side; dl += sum_t a.db
    GemmArgs b1 = {};
    b1.A = dy;
    b1.lda = d_out;
    b1.colscale = h;
    b1.ascale = gscale;
    b1.Bbits = bits_ut;
    b1.M = M;
    b1.N = (int)Pr;
    b1.K = (int)d_out;
    b1.oscale = inv;
    b1.out = db;
    b1.dot_other = tape_a;
    b1.dot_partial = part_l;
    if (P > 1) {
        b1.path_n = (int)r;  // path n0 / r: dy staged with h_p
        b1.cs_pstride = d_out;
    }
    if (fused) {
        // and, per 32-column block of dy, c_p = f16(a_p.l_p) S_U,p^T recomputed
        // and dh partials sum_t dy.c_p (c is not stored)
        b1.dh_bits = bits_u;
        b1.dh_a = tape_a;
        b1.dh_l = l;
        b1.dh_partial = part_h;
        if (P > 1) {
            b1.dh_pstride = d_out * (r / 32);
            b1.dh_row_words = (int)(r / 32);
        }
        BLR_TRY(launch_gemm(GEMM_B1_DH, b1, s));
    } else {
        BLR_TRY(launch_gemm(GEMM_B1, b1, s));
    }

    // dx'_p = f16(db_p.l_p.gs) S_V,p^T / gs; dx (+)= sum_p g_p.dx'_p;
    // dg_p += sum_t x.dx'_p
    GemmArgs b2 = {};
    b2.A = db;
    b2.lda = Pr;
    b2.colscale = l;
    b2.ascale = gscale;
    b2.Bbits = bits_v;
    b2.M = M;
    b2.N = (int)d_in;
    b2.K = (int)Pr;
    b2.oscale = inv;
    b2.out2 = dx;
    b2.out2col = g;
    b2.out2acc = accumulate_dx ? 1 : 0;
    b2.dot_other = x;
    b2.dot_partial = part_g;
    if (P > 1) {
        b2.path_k = (int)r;
        b2.b_pstride = d_in * (r / 32);
        b2.o2_pstride = d_in;
        b2.dot_pstride = mt_b2 * d_in;
        BLR_TRY(launch_gemm(GEMM_B2_MP, b2, s));
    } else {
        BLR_TRY(launch_gemm(GEMM_B2, b2, s));
    }

    // dh_p, dl, dg_p += their partial sums, one launch
    FinishJobs fin = {};
    int nj = 0;
    for (int64_t q = 0; q < P; ++q) fin.job[nj++] = {part_h + q * nparts_h * d_out, nparts_h, (int)d_out, dh + q * d_out};
    fin.job[nj++] = {part_l, mt_b1, (int)Pr, dl};
    for (int64_t q = 0; q < P; ++q) fin.job[nj++] = {part_g + q * mt_b2 * d_in, mt_b2, (int)d_in, dg + q * d_in};
    fin.count = nj;
    BLR_TRY(launch_finish(fin, s));

    if (grad_u) {
        // G_U,p = diag(h_p) dy^T a_p diag(l_p) from f16(dy.h_p.gs) and
        // f16(a_p.l_p); G_V,p = diag(g_p) x^T db_p diag(l_p) from f16(x.g_p)
        // and f16(db_p.l_p.gs); both / gs. The a tape and db hold the paths
        // side by side, so path p's columns start at p r with row stride P r.
        TnJobs tj = {};
        tj.T = M;
        tj.count = 0;
        tj.part = (float *)(ws + L.part_s);
        for (int64_t q = 0; q < P; ++q) {
            tj.job[tj.count++] = {dy, h + q * d_out, gscale, tape_a + q * r, l + q * r, 1.0f, (int)d_out, (int)r, inv,
                                  grad_u + q * d_out * r, accumulate_signs ? 1 : 0, 0, d_out, Pr, 0};
            tj.job[tj.count++] = {x, g + q * d_in, 1.0f, db + q * r, l + q * r, gscale, (int)d_in, (int)r, inv,
                                  grad_v + q * d_in * r, accumulate_signs ? 1 : 0, 0, d_in, Pr, 0};
        }
        BLR_TRY(launch_gemm_tn(tj, s));
    }
    return BLR_OK;
}

int blr_backward(int64_t M, int64_t d_in, int64_t d_out, int64_t r, const float *x, const float *dy,
                 const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l, const float *g,
                 const float *tape_a, const float *tape_c, float gscale, float *dh, float *dl, float *dg, float *dx,
                 int accumulate_dx, void *workspace, size_t workspace_bytes, void *stream) {
    return backward_impl(M, d_in, d_out, r, 1, x, dy, bits_u, bits_v, h, l, g, tape_a, tape_c, gscale, dh, dl, dg,
                         dx, accumulate_dx, nullptr, nullptr, 0, workspace, workspace_bytes, stream);
}

int blr_backward_signs(int64_t M, int64_t d_in, int64_t d_out, int64_t r, const float *x, const float *dy,
                       const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l, const float *g,
                       const float *tape_a, const float *tape_c, float gscale, float *dh, float *dl, float *dg,
                       float *dx, int accumulate_dx, float *grad_u, float *grad_v, int accumulate_signs,
                       void *workspace, size_t workspace_bytes, void *stream) {
    if (!grad_u || !grad_v) return BLR_ERR_NULL;
    return backward_impl(M, d_in, d_out, r, 1, x, dy, bits_u, bits_v, h, l, g, tape_a, tape_c, gscale, dh, dl, dg,
                         dx, accumulate_dx, grad_u, grad_v, accumulate_signs, workspace, workspace_bytes, stream);
}

int blr_backward_paths(int64_t M, int64_t d_in, int64_t d_out, int64_t r, int64_t paths, const float *x,
                       const float *dy, const uint32_t *bits_u, const uint32_t *bits_v, const float *h,
                       const float *l, const float *g, const float *tape_a, float gscale, float *dh, float *dl,
                       float *dg, float *dx, int accumulate_dx, float *grad_u, float *grad_v, int accumulate_signs,
                       void *workspace, size_t workspace_bytes, void *stream) {
    return backward_impl(M, d_in, d_out, r, paths, x, dy, bits_u, bits_v, h, l, g, tape_a, nullptr, gscale, dh, dl,
                         dg, dx, accumulate_dx, grad_u, grad_v, accumulate_signs, workspace, workspace_bytes, stream);
}

int blr_plane_linear(int64_t M, int64_t n, int64_t k, const float *x, const uint16_t *plane, float *y, float scale,
                     void *stream) {
    if (!x || !plane || !y) return BLR_ERR_NULL;
    if (M < 1 || n < 128 || k < 128 || n % 128 || k % 128) return BLR_ERR_SHAPE;
    const int64_t widest = n > k ? n : k;
    if (M * widest * 4 > (int64_t)0xFFFFFFFF || n * k * 2 > (int64_t)0xFFFFFFFF) return BLR_ERR_SHAPE;
    if ((n / 128) * ceil_div(M, 64) > ((int64_t)1 << 31) - 1) return BLR_ERR_SHAPE;
    if (!pow2_scale_ok(scale)) return BLR_ERR_SCALE;
    if (!aligned16(x) || !aligned16(plane) || !aligned16(y)) return BLR_ERR_ALIGN;
    int st = current_device_ok();
    if (st != BLR_OK) return st;
    GemmArgs a = {};
    a.A = x;
    a.lda = k;
    a.ascale = scale;
    a.Bplane = plane;
    a.M = M;
    a.N = (int)n;
    a.K = (int)k;
    a.oscale = 1.0f / scale;  // exact: scale is a power of two
    a.out = y;
    BLR_TRY(launch_gemm(GEMM_PLANE, a, (hipStream_t)stream));
    return BLR_OK;
}

int blr_sumsq(const float *a, int64_t n, float *partials, int nparts, void *stream) {
    if (!a || !partials) return BLR_ERR_NULL;
    if (n < 1 || nparts < 1 || nparts > 1024) return BLR_ERR_SHAPE;
    if (!aligned16(a) || !aligned4(partials)) return BLR_ERR_ALIGN;
    int st = current_device_ok();
    if (st != BLR_OK) return st;
    BLR_TRY(launch_sumsq(a, n, partials, nparts, (hipStream_t)stream));
    return BLR_OK;
}

int blr_profile_enable(int max_launches) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    prof_release();
    if (max_launches <= 0) return BLR_OK;
    g_prof.ev.resize(2 * (size_t)max_launches);
    for (size_t i = 0; i < g_prof.ev.size(); ++i) {
        if (hipEventCreate(&g_prof.ev[i]) != hipSuccess) {
            g_prof.ev.resize(i);
            prof_release();
            return BLR_ERR_HIP;
        }
    }
    g_prof.on = true;
    return BLR_OK;
}

int blr_profile_read(const char **names, int64_t *counts, double *total_ms, int max) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (size_t q = 0; q < g_prof.used; ++q) {
        if (hipEventSynchronize(g_prof.ev[2 * q + 1]) != hipSuccess) return BLR_ERR_HIP;
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, g_prof.ev[2 * q], g_prof.ev[2 * q + 1]) != hipSuccess) return BLR_ERR_HIP;
        g_prof.counts[g_prof.ids[q]] += 1;
        g_prof.total_ms[g_prof.ids[q]] += ms;
    }
    g_prof.used = 0;
    g_prof.ids.clear();
    int n = 0;
    for (int id = 0; id < K_COUNT; ++id) {
        if (g_prof.counts[id] == 0) continue;
        if (n < max) {
            if (names) names[n] = kernel_name(id);
            if (counts) counts[n] = g_prof.counts[id];
            if (total_ms) total_ms[n] = g_prof.total_ms[id];
        }
        ++n;
    }
    return n;
}

int blr_profile_reset(void) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (int id = 0; id < K_COUNT; ++id) {
        g_prof.counts[id] = 0;
        g_prof.total_ms[id] = 0.0;
    }
    return BLR_OK;
}

}  // extern "C"
