// C-ABI of libwtconv.so: argument validation on the host, then dispatch to
// the fused kernels (forward, backward data, backward weight) or to the naive
// unfused chain. Nothing is launched unless every check passes.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/wtconv.h"
#include "wtconv_plans.h"
#include "wtconv_bwd1.h"
#include "wtconv_bwdw.h"
#include "wtconv_dw.h"
#include "wtconv_layout.h"
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

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// How a call is served. Planned shapes run the fused kernels; a channels-last
// call of a planned shape runs them on planar copies of its activations kept
// in the workspace (after the kernels' own part); everything else runs the
// generic chain, which reads either layout directly.
struct Route {
    const wtc::DwEntry* de = nullptr;      // L = 0 data kernels (plain depthwise correlation)
    const wtc::PlaneEntry* pe = nullptr;   // whole-plane data kernels
    const wtc::SplitEntry* se = nullptr;   // coarse + fine data kernels
    bool bw = false;                       // fused weight-gradient kernels
    bool copies = false;                   // channels last through planar copies
    size_t own = 0;                        // the kernels' own workspace bytes
    size_t need = 0;                       // total workspace bytes
};

Route route(const wtconv_desc_t* d, int op) {
    Route r;
    const bool nhwc = d->layout == WTCONV_NHWC;
    const bool convertible = !nhwc || wtc::transpose_fits(d->B, d->C, d->H, d->W);
    if (d->B > 0 && convertible) {
        if (op == WTCONV_OP_BWD_WEIGHT) {
            const size_t b = wtc::bwdw_workspace_bytes(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level);
            if (b != (size_t)-1) {
                r.bw = true;
                r.own = b;
            }
        } else if (d->levels == 0) {
            r.de = wtc::find_dw_entry(d->H, d->W, d->k_base);
            // the kernel addresses a workgroup's planes with 32-bit offsets
            if (r.de && (uint64_t)r.de->npw * d->C * d->H * d->W >= (1ull << 32)) r.de = nullptr;
        } else {
            r.pe = wtc::find_plane_entry(d->H, d->W, d->levels, d->k_base, d->k_level);
            // the whole-plane kernels address a workgroup's planes with 32-bit offsets
            if (r.pe && (uint64_t)r.pe->npw * d->C * d->H * d->W >= (1ull << 32)) r.pe = nullptr;
            if (!r.pe && (r.se = wtc::find_split_entry(d->H, d->W, d->levels, d->k_base, d->k_level)))
                r.own = r.se->ws_bytes(d->B, d->C);
        }
    }
    if (r.de || r.pe || r.se || r.bw) {
        r.copies = nhwc;
        r.need = r.copies ? align256(r.own) + 2 * align256(act_bytes(d)) : r.own;
    } else if (d->B == 0 && op != WTCONV_OP_BWD_WEIGHT) {
        r.need = 0;   // nothing to compute
    } else {
        r.need = wtc::naive_workspace_bytes(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level, op);
    }
    return r;
}

bool ws_ok(const Route& r, const void* ws, size_t ws_bytes) {
    return r.need == 0 || (ws && ws_bytes >= r.need && aligned256(ws));
}

// The two planar copies of a channels-last call, after the kernels' workspace.
void* copy_slot(const Route& r, const wtconv_desc_t* d, void* ws, int i) {
    return (char*)ws + align256(r.own) + (size_t)i * align256(act_bytes(d));
}

// fin: a deferred weight-gradient second stage for a whole-plane kernel to
// run as extra workgroups (null: none; the caller checked it fits)
wtconv_status_t fused_data_pass(const wtconv_desc_t* d, const void* in, const float* w_base,
                                const float* w_lvl, const float* scale, void* out, void* ws,
                                size_t ws_bytes, void* stream, bool flip, const wtc::FinalizeArgs* fin = nullptr) {
    wtconv_status_t st = check_desc(d);
    if (st != WTCONV_OK) return st;
    if (d->B == 0) return check_params(d, w_base, w_lvl, scale, true);   // empty batch: nothing to write
    if (!in || !out) return WTCONV_ERR_INVALID_ARG;
    if (!aligned16(in) || !aligned16(out)) return WTCONV_ERR_INVALID_ARG;
    if (overlap(in, act_bytes(d), out, act_bytes(d))) return WTCONV_ERR_INVALID_ARG;
    st = check_params(d, w_base, w_lvl, scale, true);
    if (st != WTCONV_OK) return st;
    const int op = flip ? WTCONV_OP_BWD_DATA : WTCONV_OP_FWD;
    const Route r = route(d, op);
    if (!ws_ok(r, ws, ws_bytes)) return WTCONV_ERR_WORKSPACE;
    const int dt = d->dtype == WTCONV_BF16 ? 1 : 0;
    const hipStream_t s = (hipStream_t)stream;
    if (!r.de && !r.pe && !r.se) {
        // no fused kernel for this shape: the generic one-kernel-per-step
        // chain (same results, intermediates in device memory)
        const hipError_t err = wtc::naive_data_launch(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level,
                                                      dt == 1, flip, d->layout == WTCONV_NHWC, in, w_base, w_lvl,
                                                      scale, out, ws, s);
        return err == hipSuccess ? WTCONV_OK : WTCONV_ERR_LAUNCH;
    }
    const void* kin = in;
    void* kout = out;
    if (r.copies) {
        kin = copy_slot(r, d, ws, 0);
        kout = copy_slot(r, d, ws, 1);
        if (wtc::nhwc_to_nchw(in, (void*)kin, d->B, d->C, d->H, d->W, dt == 1, s) != hipSuccess)
            return WTCONV_ERR_LAUNCH;
    }
    hipError_t err;
    if (r.de)   // L = 0: the plain depthwise correlation
        err = r.de->fn[dt][flip ? 1 : 0](kin, w_base, kout, d->B, d->C, s);
    else if (r.pe)   // the whole plane fits one workgroup: one kernel, no workspace of its own
        err = r.pe->fn[dt][flip ? 1 : 0](kin, w_base, w_lvl, scale, kout, d->B, d->C, s, fin);
    else        // coarse pass on the LL band at level L0, then the fine tiles
        err = r.se->fn[dt][flip ? 1 : 0](kin, w_base, w_lvl, scale, kout, (float*)ws, d->B, d->C, s);
    if (err == hipSuccess && r.copies) err = wtc::nchw_to_nhwc(kout, out, d->B, d->C, d->H, d->W, dt == 1, s);
    return err == hipSuccess ? WTCONV_OK : WTCONV_ERR_LAUNCH;
}

// Workspace of the single-pass backward kernel for this shape (L = 0: the
// depthwise one; L = 1: the one-level whole-plane one), or (size_t)-1.
size_t single_pass_ws(const wtconv_desc_t* d) {
    if (d->levels == 0) return wtc::bwd_single_pass_workspace_bytes(d->B, d->C, d->H, d->W, 0, d->k_base);
    return wtc::bwd1_level_workspace_bytes(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level);
}

// A single-pass backward kernel covers this shape (planar, non-empty).
bool single_pass_bwd(const wtconv_desc_t* d) {
    return d->B > 0 && d->layout == WTCONV_NCHW && single_pass_ws(d) != (size_t)-1;
}

// Shared-sums backward of a split plane: the weight-gradient plan leaves the
// level-L0 LL sums of dy in its workspace and the data pass's coarse step
// (which sums dy over the same 2^L0 blocks) reads those instead of dy.
// Workspace: the weight pass's, then the data pass's coarse image.
struct SharedSums {
    const wtc::SplitEntry* se = nullptr;
    size_t sums_offset = 0, data_offset = 0, need = 0;
};
SharedSums shared_sums_bwd(const wtconv_desc_t* d) {
    SharedSums r;
    if (d->B == 0 || d->layout != WTCONV_NCHW) return r;
    const Route rd = route(d, WTCONV_OP_BWD_DATA), rw = route(d, WTCONV_OP_BWD_WEIGHT);
    int l0 = -1;
    size_t off = 0;
    if (!rd.se || !rd.se->bwd_data_from_sums[0] || !rw.bw ||
        !wtc::bwdw_dy_sums(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level, &l0, &off) || l0 != rd.se->L0)
        return r;
    r.se = rd.se;
    r.sums_offset = off;
    r.data_offset = align256(rw.own);
    r.need = r.data_offset + rd.own;
    return r;
}

// Workspace of wtconv_bwd: the single-pass kernel's, the shared-sums pair's,
// else enough for the two backward calls run one after the other on it.
size_t bwd_workspace(const wtconv_desc_t* d) {
    if (single_pass_bwd(d)) return single_pass_ws(d);
    const SharedSums ss = shared_sums_bwd(d);
    if (ss.se) return ss.need;
    const size_t a = route(d, WTCONV_OP_BWD_DATA).need, b = route(d, WTCONV_OP_BWD_WEIGHT).need;
    return a > b ? a : b;
}


// Backward weight on a validated route. With `static_ws` set, the workspace
// is the library's static scratch array (the no-allocation entry point): the
// call's need is checked against its size first, then its device address is
// looked up; `ws` and `ws_bytes` are ignored.
wtconv_status_t bwd_weight_pass(const wtconv_desc_t* d, const void* x, const void* dy, const float* w_lvl,
                                const float* scale, float* dw_base, float* dw_lvl, float* dscale, void* ws,
                                size_t ws_bytes, void* stream, void* (*static_ws)(wtconv_status_t*)) {
    wtconv_status_t st = check_desc(d);
    if (st != WTCONV_OK) return st;
    if (d->B > 0 && (!x || !dy)) return WTCONV_ERR_INVALID_ARG;   // never read for an empty batch
    if (!dw_base) return WTCONV_ERR_INVALID_ARG;
    if (d->levels > 0 && (!dw_lvl || !dscale)) return WTCONV_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(dy) || !aligned16(dw_base)) return WTCONV_ERR_INVALID_ARG;
    if ((dw_lvl && !aligned16(dw_lvl)) || (dscale && !aligned16(dscale))) return WTCONV_ERR_INVALID_ARG;
    st = check_params(d, nullptr, w_lvl, scale, false);
    if (st != WTCONV_OK) return st;
    const Route r = route(d, WTCONV_OP_BWD_WEIGHT);
    if (static_ws) {
        if (r.need > ws_bytes) return WTCONV_ERR_SCRATCH_LIMIT;
        ws = static_ws(&st);
        if (st != WTCONV_OK) return st;
    }
    if (!ws_ok(r, ws, ws_bytes)) return WTCONV_ERR_WORKSPACE;
    const bool bf16 = d->dtype == WTCONV_BF16;
    const hipStream_t s = (hipStream_t)stream;
    hipError_t err;
    if (r.bw) {
        const void *kx = x, *kdy = dy;
        if (r.copies) {   // planar copies of x and dy, after the kernels' partial sums
            kx = copy_slot(r, d, ws, 0);
            kdy = copy_slot(r, d, ws, 1);
            err = wtc::nhwc_to_nchw(x, (void*)kx, d->B, d->C, d->H, d->W, bf16, s);
            if (err == hipSuccess) err = wtc::nhwc_to_nchw(dy, (void*)kdy, d->B, d->C, d->H, d->W, bf16, s);
            if (err != hipSuccess) return WTCONV_ERR_LAUNCH;
        }
        err = wtc::bwdw_launch(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level, bf16, kx, kdy, w_lvl,
                               scale, dw_base, dw_lvl, dscale, ws, s);
    } else   // no fused plan for this shape (or an empty batch): the generic chain
        err = wtc::naive_bwdw_launch(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level,
                                     d->dtype == WTCONV_BF16, d->layout == WTCONV_NHWC, x, dy, w_lvl, scale,
                                     dw_base, dw_lvl, dscale, ws, s);
    return err == hipSuccess ? WTCONV_OK : WTCONV_ERR_LAUNCH;
}

// Scratch of the no-allocation entry point: one array per device, held
// until the process ends. In host code `scratch` names a host-side stand-in,
// not device memory, so it is never passed to a kernel: its device address
// is looked up once per device (hipGetSymbolAddress, with that device
// current) and that address is what the kernels get. Every call on a device
// shares its array and leaves its contents behind; the weight-gradient
// kernels overwrite every word they read (partial sums, level-split LL
// planes, layout copies), so nothing in it has to start at zero. Calls that
// overlap on one device race on the array.
__device__ __align__(256) static unsigned char scratch[WTCONV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

void* scratch_device_ptr(wtconv_status_t* st) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *st = WTCONV_ERR_LAUNCH;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            *st = WTCONV_ERR_LAUNCH;
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    *st = WTCONV_OK;
    return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

size_t wtconv_workspace_size(const wtconv_desc_t* d, int32_t op) {
    if (check_desc(d) != WTCONV_OK) return (size_t)-1;
    if (op == WTCONV_OP_BWD) return bwd_workspace(d);
    if (op != WTCONV_OP_FWD && op != WTCONV_OP_BWD_DATA && op != WTCONV_OP_BWD_WEIGHT) return (size_t)-1;
    return route(d, op).need;
}

int32_t wtconv_route(const wtconv_desc_t* d, int32_t op) {
    if (check_desc(d) != WTCONV_OK) return -1;
    if (op != WTCONV_OP_FWD && op != WTCONV_OP_BWD_DATA && op != WTCONV_OP_BWD_WEIGHT && op != WTCONV_OP_BWD)
        return -1;
    if (op == WTCONV_OP_BWD && single_pass_bwd(d)) return WTCONV_ROUTE_SINGLE_PASS;
    auto one = [&](int o) -> int32_t {
        const Route r = route(d, o);
        const bool fused = o == WTCONV_OP_BWD_WEIGHT ? r.bw : (r.de || r.pe || r.se);
        if (!fused) return WTCONV_ROUTE_GENERIC;
        return r.copies ? WTCONV_ROUTE_FUSED_COPIES : WTCONV_ROUTE_FUSED;
    };
    if (op != WTCONV_OP_BWD) return one(op);
    const int32_t a = one(WTCONV_OP_BWD_DATA), b = one(WTCONV_OP_BWD_WEIGHT);
    return (a == WTCONV_ROUTE_GENERIC || b == WTCONV_ROUTE_GENERIC) ? (int32_t)WTCONV_ROUTE_GENERIC : a;
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
    return bwd_weight_pass(d, x, dy, w_lvl, scale, dw_base, dw_lvl, dscale, ws, ws_bytes, stream, nullptr);
}

wtconv_status_t wtconv_bwd_weight_noalloc(const wtconv_desc_t* d, const void* x, const void* dy,
                                          const float* w_lvl, const float* scale, float* dw_base,
                                          float* dw_lvl, float* dscale, void* stream) {
    // the static scratch stands in for the workspace; bwd_weight_pass checks
    // the call's need against its size before asking for its address
    return bwd_weight_pass(d, x, dy, w_lvl, scale, dw_base, dw_lvl, dscale, nullptr, WTCONV_NOALLOC_SCRATCH_BYTES,
                           stream, scratch_device_ptr);
}

wtconv_status_t wtconv_bwd(const wtconv_desc_t* d, const void* x, const void* dy, const float* w_base,
                           const float* w_lvl, const float* scale, void* dx, float* dw_base, float* dw_lvl,
                           float* dscale, void* ws, size_t ws_bytes, void* stream) {
    wtconv_status_t st = check_desc(d);
    if (st != WTCONV_OK) return st;
    if (d->B > 0 && (!x || !dy || !dx)) return WTCONV_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(dy) || !aligned16(dx)) return WTCONV_ERR_INVALID_ARG;
    if (overlap(dy, act_bytes(d), dx, act_bytes(d)) || overlap(x, act_bytes(d), dx, act_bytes(d)))
        return WTCONV_ERR_INVALID_ARG;
    if (!dw_base || !aligned16(dw_base)) return WTCONV_ERR_INVALID_ARG;
    if (d->levels > 0 && (!dw_lvl || !dscale)) return WTCONV_ERR_INVALID_ARG;
    if ((dw_lvl && !aligned16(dw_lvl)) || (dscale && !aligned16(dscale))) return WTCONV_ERR_INVALID_ARG;
    st = check_params(d, w_base, w_lvl, scale, true);
    if (st != WTCONV_OK) return st;
    const size_t need = bwd_workspace(d);
    if (need > 0 && (!ws || ws_bytes < need || !aligned256(ws))) return WTCONV_ERR_WORKSPACE;
    if (single_pass_bwd(d)) {
        const bool bf16 = d->dtype == WTCONV_BF16;
        const hipError_t err =
            d->levels == 0
                ? wtc::bwd_single_pass_launch(d->B, d->C, d->H, d->W, d->k_base, bf16, x, dy, w_base, dx, dw_base, ws,
                                              (hipStream_t)stream)
                : wtc::bwd1_level_launch(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level, bf16, x, dy,
                                         w_base, w_lvl, scale, dx, dw_base, dw_lvl, dscale, ws, (hipStream_t)stream);
        return err == hipSuccess ? WTCONV_OK : WTCONV_ERR_LAUNCH;
    }
    const SharedSums ss = shared_sums_bwd(d);
    if (ss.se) {
        // the weight gradient first (it leaves the dy sums), then the data
        // pass with its coarse step on those sums; the weight gradient's
        // second stage rides in that coarse step's launch as extra
        // workgroups (one launch fewer; the same sums in the same order)
        wtc::FinalizeArgs fin{};
        hipError_t err = wtc::bwdw_launch_deferred(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level,
                                                   d->dtype == WTCONV_BF16, x, dy, w_lvl, scale, dw_base, dw_lvl,
                                                   dscale, ws, (hipStream_t)stream, &fin);
        if (err != hipSuccess) return WTCONV_ERR_LAUNCH;
        const size_t scratch = (size_t)4 * fin.L * fin.K * fin.K * sizeof(float);
        if (fin.C > 0 && scratch > ss.se->coarse_lds_bytes) {
            // its scratch would not fit the coarse kernel's LDS: launch it on its own
            err = wtc::launch_finalize(fin, (hipStream_t)stream);
            if (err != hipSuccess) return WTCONV_ERR_LAUNCH;
            fin.C = 0;
        }
        err = ss.se->bwd_data_from_sums[d->dtype == WTCONV_BF16 ? 1 : 0](
            dy, (const float*)((const char*)ws + ss.sums_offset), w_base, w_lvl, scale, dx,
            (float*)((char*)ws + ss.data_offset), d->B, d->C, (hipStream_t)stream, fin.C > 0 ? &fin : nullptr);
        return err == hipSuccess ? WTCONV_OK : WTCONV_ERR_LAUNCH;
    }
    // A whole-plane data kernel: the weight gradient first, its second stage
    // then rides in the data kernel's launch as extra workgroups (one launch
    // fewer; the same sums in the same order).
    const Route rd = route(d, WTCONV_OP_BWD_DATA), rw = route(d, WTCONV_OP_BWD_WEIGHT);
    if (rd.pe && !rd.copies && rw.bw && !rw.copies && d->B > 0) {
        wtc::FinalizeArgs fin{};
        hipError_t err = wtc::bwdw_launch_deferred(d->B, d->C, d->H, d->W, d->levels, d->k_base, d->k_level,
                                                   d->dtype == WTCONV_BF16, x, dy, w_lvl, scale, dw_base, dw_lvl,
                                                   dscale, ws, (hipStream_t)stream, &fin);
        if (err != hipSuccess) return WTCONV_ERR_LAUNCH;
        const size_t scratch = (size_t)4 * fin.L * fin.K * fin.K * sizeof(float);
        if (fin.C > 0 && scratch > (size_t)rd.pe->lds_bytes) {
            // its scratch would not fit the data kernel's LDS: launch it on its own
            err = wtc::launch_finalize(fin, (hipStream_t)stream);
            if (err != hipSuccess) return WTCONV_ERR_LAUNCH;
            fin.C = 0;
        }
        return fused_data_pass(d, dy, w_base, w_lvl, scale, dx, ws, ws_bytes, stream, true,
                               fin.C > 0 ? &fin : nullptr);
    }
    // the two calls in stream order, one workspace
    st = fused_data_pass(d, dy, w_base, w_lvl, scale, dx, ws, ws_bytes, stream, true);
    if (st != WTCONV_OK) return st;
    return wtconv_bwd_weight(d, x, dy, w_lvl, scale, dw_base, dw_lvl, dscale, ws, ws_bytes, stream);
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
    case WTCONV_ERR_SCRATCH_LIMIT:
        return "WTCONV_ERR_SCRATCH_LIMIT: the call needs more scratch than the no-allocation entry point's "
               "static buffer holds (WTCONV_NOALLOC_SCRATCH_BYTES, 64 MiB)";
    default: return "WTCONV: unknown status";
    }
}

const char* wtconv_version(void) { return "0.3.0"; }

}  // extern "C"
