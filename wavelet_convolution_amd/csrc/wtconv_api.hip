// C-ABI of libwtconv.so: argument validation on the host, then dispatch to
// the fused kernels (forward, backward data, backward weight) or to the naive
// unfused chain. Nothing is launched unless every check passes.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "../../include/wtconv.h"
#include "wtconv_plans.h"
#include "wtconv_bwdw.h"
#include "wtconv_naive.h"
#include "wtconv_tiled.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned256(const void* p) { return ((uintptr_t)p & 255u) == 0; }

size_t act_bytes(const wtconv_desc_t* d) {
    return (size_t)d->B * d->C * d->H * d->W * (d->dtype == WTCONV_BF16 ? 2 : 4);
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Shape checks shared by every entry point.
wtconv_status_t check_desc(const wtconv_desc_t* d) {
    if (!d) return WTCONV_ERR_INVALID_ARG;
    // B = 0 (an empty batch) is valid: nothing to write for the data passes,
    // zero weight gradients
    if (d->B < 0 || d->C < 1 || d->H < 1 || d->W < 1) return WTCONV_ERR_INVALID_ARG;
    if (d->dtype != WTCONV_F32 && d->dtype != WTCONV_BF16) return WTCONV_ERR_INVALID_ARG;
    if (d->layout != WTCONV_NCHW && d->layout != WTCONV_NHWC) return WTCONV_ERR_INVALID_ARG;
    if (d->levels < 0 || d->levels > 5) return WTCONV_ERR_UNSUPPORTED_SHAPE;
    const int kb = d->k_base, k = d->k_level;
    // odd kernels up to 15; the fused plans cover 3, 5 and 7, the generic chain any of them
    if (kb < 1 || kb > 15 || kb % 2 == 0) return WTCONV_ERR_UNSUPPORTED_SHAPE;
    if (k < 1 || k > 15 || k % 2 == 0) return WTCONV_ERR_UNSUPPORTED_SHAPE;
    // every index below is computed in 32 bits per plane and 64 bits across planes
    if ((int64_t)d->H * d->W > (1ll << 30) || (int64_t)d->B * d->C > (1ll << 31) - 1)
        return WTCONV_ERR_UNSUPPORTED_SHAPE;
    return WTCONV_OK;
}

wtconv_status_t check_params(const wtconv_desc_t* d, const float* w_base, const float* w_lvl,
                             const float* scale, bool need_base) {
    if (need_base && !w_base) return WTCONV_ERR_INVALID_ARG;
    if (d->levels > 0 && (!w_lvl || !scale)) return WTCONV_ERR_INVALID_ARG;
    if ((w_base && !aligned16(w_base)) || (w_lvl && !aligned16(w_lvl)) || (scale && !aligned16(scale)))
        return WTCONV_ERR_INVALID_ARG;
    return WTCONV_OK;
}

wtconv_status_t fused_data_pass(const wtconv_desc_t* d, const void* in, const float* w_base,
                                const float* w_lvl, const float* scale, void* out, void* ws,
                                size_t ws_bytes, void* stream, bool flip) {
    wtconv_status_t st = check_desc(d);
    if (st != WTCONV_OK) return st;
    if (d->B == 0) return check_params(d, w_base, w_lvl, scale, true);   // empty batch: nothing to write
    if (!in || !out) return WTCONV_ERR_INVALID_ARG;
    if (!aligned16(in) || !aligned16(out)) return WTCONV_ERR_INVALID_ARG;
    if (overlap(in, act_bytes(d), out, act_bytes(d))) return WTCONV_ERR_INVALID_ARG;
    st = check_params(d, w_base, w_lvl, scale, true);
    if (st != WTCONV_OK) return st;
    const int dt = d->dtype == WTCONV_BF16 ? 1 : 0;
    const bool nchw = d->layout == WTCONV_NCHW;
    hipError_t err;
    const wtc::PlaneEntry* pe = nchw ? wtc::find_plane_entry(d->H, d->W, d->levels, d->k_base, d->k_level) : nullptr;
    const wtc::SplitEntry* se = nchw ? wtc::find_split_entry(d->H, d->W, d->levels, d->k_base, d->k_level) : nullptr;
    if (const wtc::PlaneEntry* e = pe) {
        // the whole plane fits one workgroup: one kernel, no workspace
        err = e->fn[dt][flip ? 1 : 0](in, w_base, w_lvl, scale, out, d->B, d->C, (hipStream_t)stream);
    } else if (const wtc::SplitEntry* e = se) {
        // coarse pass on the LL band at level L0, then the fine tiles
        const size_t need = e->ws_bytes(d->B, d->C);
        if (need > 0 && (!ws || ws_bytes < need || !aligned256(ws))) return WTCONV_ERR_WORKSPACE;
        err = e->fn[dt][flip ? 1 : 0](in, w_base, w_lvl, scale, out, (float*)ws, d->B, d->C, (hipStream_t)stream);
    } else {
        // no fused kernel for this shape or layout: the generic
        // one-kernel-per-step chain (same results, intermediates in device memory)
        const int op = flip ? WTCONV_OP_BWD_DATA : WTCONV_OP_FWD;
        const size_t need = wtc::naive_workspace_bytes(d->B, d->C, d->H, d->W, d->levels, d->k_base,
                                                       d->k_level, op);
        if (need > 0 && (!ws || ws_bytes < need || !aligned256(ws))) return WTCONV_ERR_WORKSPACE;
        err = wtc::naive_data_launch(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level,
                                     d->dtype == WTCONV_BF16, flip, !nchw, in, w_base, w_lvl, scale, out, ws,
                                     (hipStream_t)stream);
    }
    return err == hipSuccess ? WTCONV_OK : WTCONV_ERR_LAUNCH;
}

// Whether the fused weight-gradient kernels have a plan for this shape (an
// empty batch takes the generic chain, which writes zero gradients).
bool fused_bwdw_planned(const wtconv_desc_t* d) {
    return d->layout == WTCONV_NCHW && d->B > 0 &&
           wtc::bwdw_workspace_bytes(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level) !=
           (size_t)-1;
}

}  // namespace

extern "C" {

size_t wtconv_workspace_size(const wtconv_desc_t* d, int32_t op) {
    if (check_desc(d) != WTCONV_OK) return (size_t)-1;
    switch (op) {
    case WTCONV_OP_FWD:
    case WTCONV_OP_BWD_DATA:
        if (d->B == 0) return 0;
        if (d->layout == WTCONV_NCHW) {
            if (wtc::find_plane_entry(d->H, d->W, d->levels, d->k_base, d->k_level)) return 0;
            if (const wtc::SplitEntry* e = wtc::find_split_entry(d->H, d->W, d->levels, d->k_base, d->k_level))
                return e->ws_bytes(d->B, d->C);
        }
        return wtc::naive_workspace_bytes(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level, op);
    case WTCONV_OP_BWD_WEIGHT:
        if (fused_bwdw_planned(d))
            return wtc::bwdw_workspace_bytes(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level);
        return wtc::naive_workspace_bytes(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level, op);
    default:
        return (size_t)-1;
    }
}

wtconv_status_t wtconv_fwd(const wtconv_desc_t* d, const void* x, const float* w_base,
                           const float* w_lvl, const float* scale, void* y, void* ws,
                           size_t ws_bytes, void* stream) {
    return fused_data_pass(d, x, w_base, w_lvl, scale, y, ws, ws_bytes, stream, false);
}

wtconv_status_t wtconv_bwd_data(const wtconv_desc_t* d, const void* dy, const float* w_base,
                                const float* w_lvl, const float* scale, void* dx, void* ws,
                                size_t ws_bytes, void* stream) {
    return fused_data_pass(d, dy, w_base, w_lvl, scale, dx, ws, ws_bytes, stream, true);
}

wtconv_status_t wtconv_bwd_weight(const wtconv_desc_t* d, const void* x, const void* dy,
                                  const float* w_lvl, const float* scale, float* dw_base,
                                  float* dw_lvl, float* dscale, void* ws, size_t ws_bytes,
                                  void* stream) {
    wtconv_status_t st = check_desc(d);
    if (st != WTCONV_OK) return st;
    if (d->B > 0 && (!x || !dy)) return WTCONV_ERR_INVALID_ARG;   // never read for an empty batch
    if (!dw_base) return WTCONV_ERR_INVALID_ARG;
    if (d->levels > 0 && (!dw_lvl || !dscale)) return WTCONV_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(dy) || !aligned16(dw_base)) return WTCONV_ERR_INVALID_ARG;
    if ((dw_lvl && !aligned16(dw_lvl)) || (dscale && !aligned16(dscale))) return WTCONV_ERR_INVALID_ARG;
    st = check_params(d, nullptr, w_lvl, scale, false);
    if (st != WTCONV_OK) return st;
    const bool fused = fused_bwdw_planned(d);
    const size_t need =
        fused ? wtc::bwdw_workspace_bytes(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level)
              : wtc::naive_workspace_bytes(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level,
                                           WTCONV_OP_BWD_WEIGHT);
    if (need > 0 && (!ws || ws_bytes < need || !aligned256(ws))) return WTCONV_ERR_WORKSPACE;
    hipError_t err;
    if (fused)
        err = wtc::bwdw_launch(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level, d->dtype == WTCONV_BF16, x,
                               dy, w_lvl, scale, dw_base, dw_lvl, dscale, ws, (hipStream_t)stream);
    else   // no fused plan for this shape: the generic chain
        err = wtc::naive_bwdw_launch(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level,
                                     d->dtype == WTCONV_BF16, d->layout == WTCONV_NHWC, x, dy, w_lvl, scale,
                                     dw_base, dw_lvl, dscale, ws, (hipStream_t)stream);
    return err == hipSuccess ? WTCONV_OK : WTCONV_ERR_LAUNCH;
}

size_t wtconv_naive_workspace_size(const wtconv_desc_t* d, int32_t op) {
    if (check_desc(d) != WTCONV_OK) return (size_t)-1;
    return wtc::naive_workspace_bytes(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level,
                                      op);
}

static wtconv_status_t naive_data(const wtconv_desc_t* d, const void* in, const float* w_base,
                                  const float* w_lvl, const float* scale, void* out, void* ws,
                                  size_t ws_bytes, void* stream, int op) {
    wtconv_status_t st = check_desc(d);
    if (st != WTCONV_OK) return st;
    if (d->B == 0) return check_params(d, w_base, w_lvl, scale, true);   // empty batch: nothing to write
    if (!in || !out || !aligned16(in) || !aligned16(out)) return WTCONV_ERR_INVALID_ARG;
    if (overlap(in, act_bytes(d), out, act_bytes(d))) return WTCONV_ERR_INVALID_ARG;
    st = check_params(d, w_base, w_lvl, scale, true);
    if (st != WTCONV_OK) return st;
    const size_t need = wtc::naive_workspace_bytes(d->B, d->C, d->H, d->W, d->levels, d->k_base,
                                                   d->k_level, op);
    if (need > 0 && (!ws || ws_bytes < need || !aligned256(ws))) return WTCONV_ERR_WORKSPACE;
    hipError_t err = wtc::naive_data_launch(d->B, d->C, d->H, d->W, d->levels, d->k_base,
                                            d->k_level, d->dtype == WTCONV_BF16,
                                            op == WTCONV_OP_BWD_DATA, d->layout == WTCONV_NHWC, in,
                                            w_base, w_lvl, scale, out, ws, (hipStream_t)stream);
    return err == hipSuccess ? WTCONV_OK : WTCONV_ERR_LAUNCH;
}

wtconv_status_t wtconv_naive_fwd(const wtconv_desc_t* d, const void* x, const float* w_base,
                                 const float* w_lvl, const float* scale, void* y, void* ws,
                                 size_t ws_bytes, void* stream) {
    return naive_data(d, x, w_base, w_lvl, scale, y, ws, ws_bytes, stream, WTCONV_OP_FWD);
}

wtconv_status_t wtconv_naive_bwd_data(const wtconv_desc_t* d, const void* dy, const float* w_base,
                                      const float* w_lvl, const float* scale, void* dx, void* ws,
                                      size_t ws_bytes, void* stream) {
    return naive_data(d, dy, w_base, w_lvl, scale, dx, ws, ws_bytes, stream, WTCONV_OP_BWD_DATA);
}

wtconv_status_t wtconv_naive_bwd_weight(const wtconv_desc_t* d, const void* x, const void* dy,
                                        const float* w_lvl, const float* scale, float* dw_base,
                                        float* dw_lvl, float* dscale, void* ws, size_t ws_bytes,
                                        void* stream) {
    wtconv_status_t st = check_desc(d);
    if (st != WTCONV_OK) return st;
    if ((d->B > 0 && (!x || !dy)) || !dw_base || !aligned16(x) || !aligned16(dy)) return WTCONV_ERR_INVALID_ARG;
    if (d->levels > 0 && (!dw_lvl || !dscale)) return WTCONV_ERR_INVALID_ARG;
    st = check_params(d, nullptr, w_lvl, scale, false);
    if (st != WTCONV_OK) return st;
    const size_t need = wtc::naive_workspace_bytes(d->B, d->C, d->H, d->W, d->levels, d->k_base,
                                                   d->k_level, WTCONV_OP_BWD_WEIGHT);
    if (need > 0 && (!ws || ws_bytes < need || !aligned256(ws))) return WTCONV_ERR_WORKSPACE;
    hipError_t err = wtc::naive_bwdw_launch(d->B, d->C, d->H, d->W, d->levels, d->k_base,
                                            d->k_level, d->dtype == WTCONV_BF16,
                                            d->layout == WTCONV_NHWC, x, dy, w_lvl, scale, dw_base,
                                            dw_lvl, dscale, ws, (hipStream_t)stream);
    return err == hipSuccess ? WTCONV_OK : WTCONV_ERR_LAUNCH;
}

const char* wtconv_status_string(wtconv_status_t s) {
    switch (s) {
    case WTCONV_OK: return "WTCONV_OK";
    case WTCONV_ERR_INVALID_ARG: return "WTCONV_ERR_INVALID_ARG: null, misaligned or overlapping pointer, or bad size, dtype or layout";
    case WTCONV_ERR_UNSUPPORTED_SHAPE: return "WTCONV_ERR_UNSUPPORTED_SHAPE: unsupported kernel size or levels, or a plane above 2^30 elements";
    case WTCONV_ERR_WORKSPACE: return "WTCONV_ERR_WORKSPACE: workspace missing, too small or not 256-byte aligned";
    case WTCONV_ERR_LAUNCH: return "WTCONV_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
    default: return "WTCONV: unknown status";
    }
}

const char* wtconv_version(void) { return "0.2.0"; }

}  // extern "C"
