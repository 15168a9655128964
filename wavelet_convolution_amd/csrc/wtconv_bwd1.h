// Single-pass backward of one-level whole planes: dx and every weight
// gradient from one read of x and dy (wtconv_bwd1.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

namespace wtc {

// Workspace bytes of the single-pass one-level backward for this shape, or
// (size_t)-1 where it has no plan.
size_t bwd1_level_workspace_bytes(int B, int C, int H, int W, int L, int KB, int K);

// dx, dw_base, dw_lvl and dscale of one call (the shape must have a plan;
// hipErrorInvalidValue otherwise), enqueued on `stream`: the fused kernel,
// then the fixed-order second stage of the weight gradients.
hipError_t bwd1_level_launch(int B, int C, int H, int W, int L, int KB, int K, bool bf16, const void* x,
                             const void* dy, const float* w_base, const float* w_lvl, const float* scale, void* dx,
                             float* dw_base, float* dw_lvl, float* dscale, void* ws, hipStream_t stream);

}  // namespace wtc
