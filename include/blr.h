/*
 * blr.h: C ABI of the binary low-rank (`blr`) linear layer on AMD Instinct
 * MI355X (CDNA4, gfx950).
 *
 * The layer (cortiq-engine "src/gpu_wgpu/train_mm.rs", module doc block):
 *
 *     W^ = diag(h) . S_U . diag(l) . S_V^T . diag(g)
 *
 * with sign matrices S_U [d_out][r] and S_V [d_in][r] of +-1 stored as
 * bitmaps, h [d_out], l [r] (the diagonal ell), g [d_in] in f32.
 *
 *   forward   a = (x.g) S_V        c = (a.l) S_U^T       y  = h.c  (or +=)
 *   backward  dh += sum_t dy.c     db = (dy.h) S_U       dl += sum_t a.db
 *             dx' = (db.l) S_V^T   dg += sum_t x.dx'     dx = g.dx' (or +=)
 *
 * Bitmaps (page: `expand` shader): row-major [rows][W] u32 words with
 * W = ceil(r/32); bit j of word w is rank 32w+j; a set bit is +1, a clear
 * bit -1. Bits at ranks >= r in the last word are ignored.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are HIP device pointers to row-major, contiguous
 *     arrays. The caller owns every buffer. Inputs must not alias outputs.
 *   - Shapes are int64. GPU-path rule (the page's GEMM contract: N a multiple
 *     of 128, K of 32, activation rows padded to 128): d_in, d_out and r are
 *     multiples of 128; the token count M is any value >= 1 (padding is
 *     internal; exactly M rows are read and written).
 *   - `stream` is a hipStream_t (passed as void*); NULL is the default
 *     stream. Every call only enqueues work on it and returns without a host
 *     synchronisation.
 *   - Arguments are validated before anything is enqueued: on an error no
 *     kernel is launched and no output is touched. Return value: BLR_OK or a
 *     negative blr_status. A launch failure reported by the runtime after
 *     validation returns BLR_ERR_HIP (earlier kernels of the call may have
 *     run).
 *   - The library never allocates device memory and never frees any; the
 *     caller passes a device workspace of at least blr_workspace_bytes().
 *     Two calls that share a workspace must be ordered (same stream).
 *   - Arithmetic: operands of the four contractions are staged as f16 (round
 *     to nearest even, subnormals kept, overflow gives +-inf) and multiplied
 *     on the MFMA units with f32 accumulation; every reduction and every
 *     output is f32. Results are deterministic: reruns give identical bits.
 */
#ifndef BLR_H
#define BLR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BLR_OK = 0,
    BLR_ERR_NULL = -1,      /* a required pointer is NULL */
    BLR_ERR_SHAPE = -2,     /* a size is out of range or breaks the multiple-of-128 rule */
    BLR_ERR_SCALE = -3,     /* gscale is not a positive finite power of two */
    BLR_ERR_WORKSPACE = -4, /* workspace NULL or smaller than blr_workspace_bytes() */
    BLR_ERR_DEVICE = -5,    /* current device is not gfx950 */
    BLR_ERR_HIP = -6,       /* the HIP runtime reported an error */
    BLR_ERR_ALIGN = -7,     /* a pointer is not 16-byte aligned */
    BLR_ERR_SCRATCH = -8    /* sizes exceed the allocation-free forward's scratch */
} blr_status;

/* Human-readable text of a status code (static storage). */
const char *blr_status_string(int status);

/* 1 when `hip_device` is a gfx950 device this library's kernels run on, 0
 * otherwise (the page's `matrix_units` capability check). */
int blr_device_supported(int hip_device);

/* Bytes of device workspace blr_forward, blr_backward and
 * blr_backward_signs need for these sizes (the same figure serves all
 * three; it includes the token-range partials of the sign gradients, under
 * 64 MB for any shape). 0 for invalid sizes. */
size_t blr_workspace_bytes(int64_t M, int64_t d_in, int64_t d_out, int64_t r);

/*
 * Sign expansion (page: `expand` shader and its wrapper): bitmap
 * bits [rows][ceil(r/32)] -> f16 planes
 *     plane   [rows][r]   plane[i][k]   = S[i][k]   (0x3C00 = +1, 0xBC00 = -1)
 *     plane_t [r][rows]   plane_t[k][i] = S[i][k]
 * Either output may be NULL (not both). Any rows >= 1 and r >= 1 (no
 * multiple-of-128 rule here). Bit-exact; writes exactly rows*r halves per
 * plane. Output pointers must be 16-byte aligned; bits 4-byte aligned.
 */
int blr_expand_signs(const uint32_t *bits, int64_t rows, int64_t r, uint16_t *plane, uint16_t *plane_t,
                     void *stream);

/*
 * Forward (page: `blr_forward`, doc block forward line).
 *   x [M][d_in]; bits_u [d_out][W]; bits_v [d_in][W]; h [d_out]; l [r]; g [d_in]
 *   y [M][d_out]: accumulate_y = 0 writes y = h.c, 1 adds h.c to y (the page
 *     overwrites for its first path and adds for later ones).
 *   tape_a [M][r]: receives a (f32), which blr_backward reads.
 *   tape_c [M][d_out] or NULL: receives c (f32) when given (the page keeps
 *     c for its backward). When NULL, c is not stored and blr_backward
 *     recomputes it with the same contraction (bit-identical c): 2*M*r*d_out
 *     more MFMA flops instead of 8*M*d_out bytes of HBM traffic.
 *   The tapes must come from a forward on the same x and parameters.
 * The sign planes are decoded from the bitmaps on every call (the page
 * re-expands its planes per layer call). Float and bitmap pointers must be
 * 16-byte aligned.
 */
int blr_forward(int64_t M, int64_t d_in, int64_t d_out, int64_t r, const float *x, const uint32_t *bits_u,
                const uint32_t *bits_v, const float *h, const float *l, const float *g, float *y, int accumulate_y,
                float *tape_a, float *tape_c, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory or
 * pass a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Arguments, rules and results are those
 * of blr_forward (bit for bit, the same kernels), without the workspace.
 * The forward's only scratch, the transposed S_V bitmap (r * d_in / 8
 * bytes), goes to a device array of BLR_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends; its address
 * is looked up (not allocated) on the first call on each device. Nothing in
 * it needs clearing: every call writes the part it reads. Sizes with
 * r * d_in / 8 > BLR_NOALLOC_SCRATCH_BYTES return BLR_ERR_SCRATCH before
 * anything is enqueued. Every call on one GPU shares that GPU's array, so
 * calls that overlap on a GPU (other streams, other host threads) race:
 * order them on one stream.
 */
#define BLR_NOALLOC_SCRATCH_BYTES (4u << 20)
int blr_forward_noalloc(int64_t M, int64_t d_in, int64_t d_out, int64_t r, const float *x, const uint32_t *bits_u,
                        const uint32_t *bits_v, const float *h, const float *l, const float *g, float *y,
                        int accumulate_y, float *tape_a, float *tape_c, void *stream);

/*
 * Backward (page: `blr_backward`, doc block backward lines).
 *   x [M][d_in] the forward's input; dy [M][d_out]; tape_a and tape_c from
 *     blr_forward on the same x and parameters; tape_c NULL exactly when
 *     the forward stored none (then c is recomputed from tape_a).
 *   gscale: the power of two the gradients are staged under in f16 (dy.h
 *     and db.l are multiplied by it before rounding to f16; the products are
 *     divided by it in f32, exactly). Must be a positive finite power of two.
 *   dh [d_out], dl [r], dg [d_in]: always accumulate (+=); zero them first
 *     for a plain gradient.
 *   dx [M][d_in]: accumulate_dx = 0 writes dx = g.dx', 1 adds.
 * Float and bitmap pointers must be 16-byte aligned.
 */
int blr_backward(int64_t M, int64_t d_in, int64_t d_out, int64_t r, const float *x, const float *dy,
                 const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l, const float *g,
                 const float *tape_a, const float *tape_c, float gscale, float *dh, float *dl, float *dg, float *dx,
                 int accumulate_dx, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward with the sign gradients (page: `blr_backward` with sign state;
 * the f64 host reference of its tests): blr_backward, then
 *   grad_u [d_out][r]: G_U = diag(h) . dy^T . a . diag(l)
 *   grad_v [d_in][r]:  G_V = diag(g) . x^T . db . diag(l),  db = (dy.h) S_U
 * the gradients of sum(dy.y) with respect to the entries of S_U and S_V
 * taken as real numbers (what a sign update consumes). As on the page both
 * are contractions over the tokens of f16-staged operands with f32
 * accumulation: f16(dy.h.gscale) with f16(a.l), and f16(x.g) with
 * f16(db.l.gscale), each product divided by gscale. accumulate_signs = 0
 * overwrites grad_u / grad_v, 1 adds. Where the tokens are split into ranges
 * to fill the GPU, each range's partial sums are kept in the workspace and
 * added in range order, so reruns give identical bits here too. Every other
 * argument, rule and error is blr_backward's; grad_u and grad_v must be
 * non-NULL and 16-byte aligned.
 */
int blr_backward_signs(int64_t M, int64_t d_in, int64_t d_out, int64_t r, const float *x, const float *dy,
                       const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l, const float *g,
                       const float *tape_a, const float *tape_c, float gscale, float *dh, float *dl, float *dg,
                       float *dx, int accumulate_dx, float *grad_u, float *grad_v, int accumulate_signs,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * A layer of several paths (page: `blr_forward` / `blr_backward` over the
 * paths of a layer; y is the sum of the paths' outputs), fused: one launch
 * per contraction for all paths. paths = P, 1 <= P <= 4; path p's operands
 * are the p-th blocks of
 *   bits_u [P][d_out][r/32], bits_v [P][d_in][r/32] (16-byte aligned),
 *   h [P][d_out], l [P][r], g [P][d_in],
 * and the a tape is [M][P r] (the paths' ranks side by side). There is no c
 * tape: the backward recomputes each path's c. y (accumulate_y as in
 * blr_forward) receives sum_p h_p . c_p; dx (accumulate_dx) receives
 * sum_p g_p . dx'_p; dh [P][d_out], dl [P][r], dg [P][d_in] always
 * accumulate; with grad_u [P][d_out][r] and grad_v [P][d_in][r] (both or
 * neither) the sign gradients of every path are formed as in
 * blr_backward_signs. Sizes: P r obeys the rules for r. The workspace is
 * blr_workspace_bytes_paths(M, d_in, d_out, r, P) bytes (0 for an invalid
 * shape). Errors as blr_forward / blr_backward_signs; P out of range is
 * BLR_ERR_SHAPE. P = 1 gives exactly blr_forward / blr_backward.
 */
size_t blr_workspace_bytes_paths(int64_t M, int64_t d_in, int64_t d_out, int64_t r, int64_t paths);
int blr_forward_paths(int64_t M, int64_t d_in, int64_t d_out, int64_t r, int64_t paths, const float *x,
                      const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l, const float *g,
                      float *y, int accumulate_y, float *tape_a, void *workspace, size_t workspace_bytes,
                      void *stream);
int blr_backward_paths(int64_t M, int64_t d_in, int64_t d_out, int64_t r, int64_t paths, const float *x,
                       const float *dy, const uint32_t *bits_u, const uint32_t *bits_v, const float *h,
                       const float *l, const float *g, const float *tape_a, float gscale, float *dh, float *dl,
                       float *dg, float *dx, int accumulate_dx, float *grad_u, float *grad_v, int accumulate_signs,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Dense frozen linear (page: `plane_linear`): y [M][n] = (f16(x * scale)
 * . plane^T) / scale, x [M][k] f32, plane [n][k] f16 (IEEE binary16 bit
 * patterns), through the same staging and MFMA contraction as the layer
 * (f32 accumulation; y overwritten). scale is a positive finite power of two
 * (the page stages gradients under a gradient scale when it runs this for
 * the input gradient with the transposed plane). n and k multiples of 128,
 * M >= 1; x, plane and y 16-byte aligned.
 */
int blr_plane_linear(int64_t M, int64_t n, int64_t k, const float *x, const uint16_t *plane, float *y, float scale,
                     void *stream);

/*
 * Sum of squares (page: `sumsq` shader and wrapper, the host's check of a
 * buffer for non-finite values): writes nparts f32 partial sums of a[i]^2,
 * i < n, to the device array partials[nparts]; the caller adds them (the
 * page adds them on the host in f64). A non-finite element makes its partial
 * (and so the total) non-finite. Each partial covers a fixed set of elements
 * summed in a fixed order: deterministic. 1 <= nparts <= 1024, n >= 1; a must
 * be 16-byte aligned, partials 4-byte aligned.
 */
int blr_sumsq(const float *a, int64_t n, float *partials, int nparts, void *stream);

/*
 * Per-kernel timing with HIP events (the role of the page's trainer
 * profiling marks). blr_profile_enable(n) creates a pool of event pairs for
 * up to n launches and brackets every later launch of this library with a
 * pair on the launch's stream; blr_profile_enable(0) stops and releases the
 * pool. blr_profile_read synchronises the recorded events, adds their
 * durations into per-kernel totals, and copies up to `max` entries out:
 * names[i] (static strings), counts[i] (launches), total_ms[i]. Returns the
 * number of kernel kinds seen, or a negative status. blr_profile_reset
 * clears the totals. These calls are not thread safe.
 */
int blr_profile_enable(int max_launches);
int blr_profile_read(const char **names, int64_t *counts, double *total_ms, int max);
int blr_profile_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* BLR_H */
