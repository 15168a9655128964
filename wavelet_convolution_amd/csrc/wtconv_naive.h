// Naive unfused WTConv chain (comparator).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace wtc {

size_t naive_workspace_bytes(int B, int C, int H, int W, int L, int KB, int K, int op);

// nhwc: activations channels-last [B][H][W][C] instead of [B][C][H][W]
hipError_t naive_data_launch(int B, int C, int H, int W, int L, int KB, int K, bool bf16, bool flip,
                             bool nhwc, const void* in, const float* w_base, const float* w_lvl,
                             const float* scale, void* out, void* ws, hipStream_t stream);

hipError_t naive_bwdw_launch(int B, int C, int H, int W, int L, int KB, int K, bool bf16, bool nhwc,
                             const void* x, const void* dy, const float* w_lvl, const float* scale,
                             float* dw_base, float* dw_lvl, float* dscale, void* ws,
                             hipStream_t stream);

}  // namespace wtc
