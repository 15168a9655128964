/*
 * wtconv.h - C-ABI of the MI355X (gfx950) WTConv library, libwtconv.so.
 *
 * The operation
 * -------------
 * A wavelet-convolution (WTConv) layer, as named in the abstract of
 * "I/O-aware reformulation of wavelet convolution" (arXiv:2608.10805;
 * tech.sinsc.com page, Abstract, and the layerthelatestinalattice.com
 * summary): a depthwise base convolution plus an L-level Haar wavelet branch.
 * Per (b, c) plane:
 *
 *   X_0 = x;  for l = 1..L: (LL, B1, B2, B3)_l = DWT(X_{l-1}), X_l = LL_l
 *   Z_l^s = scale[l][c][s] * corr(band_l^s, w_lvl[l][c][s])        s = 0..3
 *   R_L = 0;  R_{l-1} = IWT(Z_l^0 + R_l, Z_l^1, Z_l^2, Z_l^3)
 *   y = corr(x, w_base[c]) + R_0
 *
 *   DWT on the 2x2 block (a b / c d): LL = (a+b+c+d)/2, B1 = (a+b-c-d)/2,
 *   B2 = (a-b+c-d)/2, B3 = (a-b-c+d)/2 (orthonormal); IWT is its inverse.
 *   corr(u, w)[i][j] = sum_{m,n<k} w[m][n] u[i+m-k/2][j+n-k/2], zero outside
 *   the level's own band grid (cross-correlation, 'same', stride 1).
 *   An h x w image with odd h (w) is analysed as if it had one more, zero,
 *   row (column): its bands are ceil(h/2) x ceil(w/2); IWT returns the
 *   h x w image and drops the extra row (column). Where 2^L divides H and W
 *   this is the plain halving of the pages' workloads.
 *
 * The kernels evaluate this through the three reformulations the abstract
 * lists: the Haar analysis is recomputed on chip from x (or dy) and never
 * stored, the synthesis cascade is one closed-form pass indexed by the bits of
 * the output coordinates, and the scales are folded into the convolution
 * results. The result equals the cascade up to fp32 rounding order.
 *
 * Data layout (all device pointers, caller-owned):
 *   x, y, dy, dx   [B][C][H][W] contiguous (desc->layout WTCONV_NCHW) or
 *                  [B][H][W][C] (WTCONV_NHWC), element type = desc->dtype
 *   w_base         [C][k_base][k_base]        fp32
 *   w_lvl          [L][C][4][k_level][k_level] fp32 (level index 0 = level 1)
 *   scale          [L][C][4]                  fp32
 *   gradients      fp32, same layouts as the parameters
 * Band order s: 0 LL, 1 B1 (difference across rows), 2 B2 (difference across
 * columns), 3 B3.
 *
 * Arithmetic: activations are loaded as fp32 (bf16 widened exactly), all
 * products and sums are fp32, and bf16 outputs are rounded to nearest even.
 *
 * Ownership and synchronisation: the library allocates nothing, keeps no
 * pointer after a call returns, never synchronises the stream, and is
 * reentrant. Work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream). Outputs are overwritten, never accumulated. x and y (dy and dx)
 * must not overlap.
 *
 * Errors: every argument is validated on the host before anything is
 * launched; on error nothing is enqueued and the status says why. A failed
 * launch (hipGetLastError) returns WTCONV_ERR_LAUNCH.
 */
#ifndef WTCONV_H
#define WTCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    WTCONV_F32 = 0,    /* fp32 activations */
    WTCONV_BF16 = 1    /* bf16 activations, fp32 arithmetic */
} wtconv_dtype_t;

typedef enum {
    WTCONV_NCHW = 0,   /* [B][C][H][W] contiguous */
    WTCONV_NHWC = 1    /* channels last: [B][H][W][C] contiguous */
} wtconv_layout_t;

typedef enum {
    WTCONV_OK = 0,
    WTCONV_ERR_INVALID_ARG = 1,        /* null pointer, overlap, bad dtype or
                                          layout, B < 0, C, H or W < 1 */
    WTCONV_ERR_UNSUPPORTED_SHAPE = 2,  /* even or unsupported k, L out of
                                          range, or H*W above 2^30 */
    WTCONV_ERR_WORKSPACE = 3,          /* ws too small or misaligned */
    WTCONV_ERR_LAUNCH = 4,             /* the HIP runtime rejected a launch */
    WTCONV_ERR_SCRATCH_LIMIT = 5       /* wtconv_bwd_weight_noalloc: the call needs
                                          more than WTCONV_NOALLOC_SCRATCH_BYTES */
} wtconv_status_t;

/* Size of the static device scratch array of wtconv_bwd_weight_noalloc (one
   per GPU the library runs on, held until the process ends). */
#define WTCONV_NOALLOC_SCRATCH_BYTES (64u << 20)

typedef enum {
    WTCONV_OP_FWD = 0,
    WTCONV_OP_BWD_DATA = 1,
    WTCONV_OP_BWD_WEIGHT = 2,
    WTCONV_OP_BWD = 3          /* wtconv_bwd: both backward results */
} wtconv_op_t;

typedef struct {
    int32_t B, C, H, W;   /* activation shape, NCHW; B = 0 is an empty batch:
                             the data passes write nothing (activation
                             pointers may be NULL), the weight gradients
                             are zero */
    int32_t levels;       /* L, 0..5 */
    int32_t k_base;       /* base kernel size: odd, 1..15 */
    int32_t k_level;      /* per-level kernel size: odd, 1..15 */
    int32_t dtype;        /* wtconv_dtype_t */
    int32_t layout;       /* wtconv_layout_t of x, y, dy, dx (all four alike) */
} wtconv_desc_t;

/* Bytes of device workspace `op` needs for `desc` (0 if none). Returns
   (size_t)-1 if the descriptor is invalid or unsupported. Workspace pointers
   must be 256-byte aligned. */
size_t wtconv_workspace_size(const wtconv_desc_t *desc, int32_t op);

/* How a call of `op` (wtconv_op_t) runs for `desc`, so that a caller can
   tell a shape the fused kernels cover from one that takes the generic
   chain (same results, many times slower):
   - WTCONV_ROUTE_GENERIC: the one-kernel-per-step chain (no fused kernel
     for this shape, or an empty batch, for which nothing is launched but
     the zeroing of the weight gradients);
   - WTCONV_ROUTE_FUSED: fused kernels on the activations as they are;
   - WTCONV_ROUTE_FUSED_COPIES: fused kernels on planar copies of
     channels-last activations in the workspace;
   - WTCONV_ROUTE_SINGLE_PASS (WTCONV_OP_BWD only): one kernel reads x and
     dy once for dx and every weight gradient.
   For WTCONV_OP_BWD a shape reports FUSED (or FUSED_COPIES) when both of
   its backward passes are fused, else GENERIC. Returns -1 if the
   descriptor or op is invalid. No device call is made. */
typedef enum {
    WTCONV_ROUTE_GENERIC = 0,
    WTCONV_ROUTE_FUSED = 1,
    WTCONV_ROUTE_FUSED_COPIES = 2,
    WTCONV_ROUTE_SINGLE_PASS = 3
} wtconv_route_t;
int32_t wtconv_route(const wtconv_desc_t *desc, int32_t op);

/* Forward: y = WTConv(x). One fused pass: reads x once, writes y once.
   Workspace: wtconv_workspace_size(desc, WTCONV_OP_FWD) bytes (0 for planes
   that fit one workgroup's LDS; ws may then be NULL).
   L = 0 is the plain depthwise correlation; it has its own fused kernels
   on 56x56, 28x28 and 14x14 planes with k_base 5 or 7.
   Shapes without a fused kernel (any other H, W >= 1, L in 0..5, odd k up
   to 15) run the generic
   one-kernel-per-step chain of the naive entry points below: the same
   results and semantics, with the intermediates in the workspace, which
   wtconv_workspace_size then reports. A channels-last call of a planned
   shape converts its activations to planar copies in the workspace (after
   the kernels' own part), runs the fused kernels on them and converts the
   result back: bit for bit the planar results, two extra passes over the
   activations. The same holds for wtconv_bwd_data and wtconv_bwd_weight. */
wtconv_status_t wtconv_fwd(const wtconv_desc_t *desc, const void *x,
                           const float *w_base, const float *w_lvl,
                           const float *scale, void *y, void *ws,
                           size_t ws_bytes, void *stream);

/* Backward data: dx = J^T dy. The transpose of the layer is the same layer
   with every kernel turned by 180 degrees (the orthonormal Haar analysis and
   synthesis are each other's transpose, and corr^T is corr with the flipped
   kernel), so this runs the forward kernels with rotated weight indexing. */
wtconv_status_t wtconv_bwd_data(const wtconv_desc_t *desc, const void *dy,
                                const float *w_base, const float *w_lvl,
                                const float *scale, void *dx, void *ws,
                                size_t ws_bytes, void *stream);

/* Backward weight: with G_l^s = sum_{b,i,j} (A_l^s dy)[i][j] (A_l^s x)[i+m-p][j+n-p]
   the correlation of the two Haar pyramids (A_l^s = level-l band s analysis),
     dw_base[c]      = sum_b corr-grad(x, dy)               [C][kb][kb]
     dw_lvl[l][c][s] = scale[l][c][s] * G_l^s                [L][C][4][k][k]
     dscale[l][c][s] = sum_{m,n} w_lvl[l][c][s][m][n] * G_l^s[m][n]
   (the scale-folding reformulation applied to the gradient). The batch sum
   is a fixed-order two-stage reduction, so results are bitwise
   reproducible. Workspace: wtconv_workspace_size(desc, WTCONV_OP_BWD_WEIGHT). */
wtconv_status_t wtconv_bwd_weight(const wtconv_desc_t *desc, const void *x,
                                  const void *dy, const float *w_lvl,
                                  const float *scale, float *dw_base,
                                  float *dw_lvl, float *dscale, void *ws,
                                  size_t ws_bytes, void *stream);

/* Backward weight without allocation, for callers that cannot allocate
   device memory (code under HIP graph capture, tight serving loops, harnesses
   that forbid allocation): the same kernels, results and semantics as
   wtconv_bwd_weight (bit for bit), with the scratch that call takes as a
   workspace (per-chunk partial sums, the level-split planes, channels-last
   copies) held in a static device array of WTCONV_NOALLOC_SCRATCH_BYTES
   (64 MiB) instead. A call whose wtconv_workspace_size(desc,
   WTCONV_OP_BWD_WEIGHT) exceeds that returns WTCONV_ERR_SCRATCH_LIMIT and
   enqueues nothing (the stage-shape and 128x128 workloads fit; 16 x 256 x
   256^2 at L = 4 does not). It calls no allocating routine; its first call on
   a device looks up that device's copy of the array (hipGetSymbolAddress)
   and keeps its address. Every call on one device shares that device's
   array: calls that overlap on one GPU (on different streams, or from
   different threads, without ordering) race on it and must not be made.
   Nothing in the array needs to start at zero (every word read was written
   earlier in the same call). */
wtconv_status_t wtconv_bwd_weight_noalloc(const wtconv_desc_t *desc, const void *x,
                                          const void *dy, const float *w_lvl,
                                          const float *scale, float *dw_base,
                                          float *dw_lvl, float *dscale, void *stream);

/* Whole backward pass: dx (as wtconv_bwd_data) and the weight gradients (as
   wtconv_bwd_weight) in one call. Results equal those of the two calls bit
   for bit (the same multiply-adds in the same order), except where noted
   for the one-level single pass; what the call saves depends on the shape
   (planar layout in each case):
   - L = 0 on the planes its kernel covers (56x56, 28x28, 14x14; k_base 5 or
     7): a single pass that reads x and dy once, the fused backward the I/O
     model counts at 5*N*e instead of 6*N*e bytes per step;
   - L = 1 on 14x14 planes with 5x5 kernels: a single pass that reads x and
     dy once and computes dx and every weight gradient's partial sums in one
     kernel (then the weight gradient's fixed-order second stage); dx equals
     the two calls' bit for bit, the weight gradients group their products
     differently and agree with the two calls' to fp32 rounding (both are
     deterministic);
   - planes split into fine tiles and a coarse level-L0 image (256x256 at
     L = 4 with kernels 7 and 5, and the 64x64 test plans): the weight pass
     runs first and leaves the 2^L0-block sums of dy in the workspace; the
     backward-data pass then takes its coarse levels from those sums instead
     of reading dy a second time for them, and the weight pass's fixed-order
     second stage runs as extra workgroups of that coarse step's launch;
   - whole-plane data kernels (the stage planes, 128x128, the family of
     planes of 56, 28, 14 and 7 pixels): the weight pass runs first and the
     fixed-order second stage of its reduction runs as extra workgroups of
     the backward-data launch (one launch fewer);
   - other shapes: the two backward calls in stream order on one workspace.
   x and dy must not overlap dx. Workspace:
   wtconv_workspace_size(desc, WTCONV_OP_BWD). */
wtconv_status_t wtconv_bwd(const wtconv_desc_t *desc, const void *x,
                           const void *dy, const float *w_base,
                           const float *w_lvl, const float *scale, void *dx,
                           float *dw_base, float *dw_lvl, float *dscale,
                           void *ws, size_t ws_bytes, void *stream);

/* Naive unfused baseline (comparator only): the same three operations as a
   chain of one-kernel-per-step launches (analysis, per-level convolution,
   scale, LL add, synthesis, base convolution, final add) that keeps every
   intermediate in device memory, as the abstract describes the reference
   implementation. Same semantics and layouts as the fused entry points;
   workspace from wtconv_naive_workspace_size. Any H, W >= 1. */
size_t wtconv_naive_workspace_size(const wtconv_desc_t *desc, int32_t op);
wtconv_status_t wtconv_naive_fwd(const wtconv_desc_t *desc, const void *x,
                                 const float *w_base, const float *w_lvl,
                                 const float *scale, void *y, void *ws,
                                 size_t ws_bytes, void *stream);
wtconv_status_t wtconv_naive_bwd_data(const wtconv_desc_t *desc, const void *dy,
                                      const float *w_base, const float *w_lvl,
                                      const float *scale, void *dx, void *ws,
                                      size_t ws_bytes, void *stream);
wtconv_status_t wtconv_naive_bwd_weight(const wtconv_desc_t *desc, const void *x,
                                        const void *dy, const float *w_lvl,
                                        const float *scale, float *dw_base,
                                        float *dw_lvl, float *dscale, void *ws,
                                        size_t ws_bytes, void *stream);

/* Static description of a status code. */
const char *wtconv_status_string(wtconv_status_t status);

/* Library version, e.g. "0.3.0". */
const char *wtconv_version(void);

/* Measurement probes (not operations of the layer). They measure on the
   device the two ceilings the kernels above are compared with.
   wtconv_peak_fma: `blocks` workgroups of 256 lanes; every lane runs 16
   independent chains of `iters` unpacked fp32 FMAs and writes one float to
   out[blocks * 256] (16-byte aligned): 2 * 16 * iters * 256 * blocks flops.
   blocks and iters in 1..2^20, else WTCONV_ERR_INVALID_ARG.
   wtconv_peak_copy: copies `bytes` (a multiple of 16) from src to dst, both
   16-byte aligned and not overlapping: 2 * bytes of HBM traffic.
   Both only enqueue on `stream`; time them with events. */
wtconv_status_t wtconv_peak_fma(float *out, int32_t blocks, int32_t iters, void *stream);
wtconv_status_t wtconv_peak_copy(const void *src, void *dst, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* WTCONV_H */
