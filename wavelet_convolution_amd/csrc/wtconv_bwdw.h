// Backward-weight launchers (fused kernel + fixed-order second stage).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "wtconv_device.h"

namespace wtc {

// Workspace bytes for the per-chunk partial sums, or (size_t)-1 if no fused
// plan covers this shape.
size_t bwdw_workspace_bytes(int B, int C, int H, int W, int L, int KB, int K);

// Whether the fused weight-gradient plan of this shape leaves, in its
// workspace at byte `offset`, the fp32 planes [B][C][H >> l0][W >> l0] of
// unnormalised level-l0 LL sums of dy (its coarse pass's input).
bool bwdw_dy_sums(int B, int C, int H, int W, int L, int KB, int K, int* l0, size_t* offset);

hipError_t bwdw_launch(int B, int C, int H, int W, int L, int KB, int K, bool bf16,
                       const void* x, const void* dy, const float* w_lvl, const float* scale,
                       float* dw_base, float* dw_lvl, float* dscale, void* ws,
                       hipStream_t stream);

// As bwdw_launch, but the second stage (the fixed-order chunk sum) is not
// launched: its arguments go to *fin (fin->C = 0 when the plan has none), for
// a later kernel of the same stream to run (finalize_channel per channel).
hipError_t bwdw_launch_deferred(int B, int C, int H, int W, int L, int KB, int K, bool bf16,
                                const void* x, const void* dy, const float* w_lvl, const float* scale,
                                float* dw_base, float* dw_lvl, float* dscale, void* ws,
                                hipStream_t stream, FinalizeArgs* fin);

// Launch a (deferred) second stage on its own.
hipError_t launch_finalize(const FinalizeArgs& f, hipStream_t stream);

// Single-pass backward (dx and the weight gradient from one read of x and dy),
// planned for L = 0 only: its workspace bytes, or (size_t)-1 without a plan.
size_t bwd_single_pass_workspace_bytes(int B, int C, int H, int W, int L, int KB);

hipError_t bwd_single_pass_launch(int B, int C, int H, int W, int KB, bool bf16, const void* x, const void* dy,
                                  const float* w_base, void* dx, float* dw_base, void* ws, hipStream_t stream);

}  // namespace wtc
