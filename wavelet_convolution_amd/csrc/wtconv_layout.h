// Channels-last <-> planar conversion of activations (device, stream-ordered).
#pragma once

#include <hip/hip_runtime.h>

namespace wtc {

// Whether the conversion kernels' grid covers this shape (grid y and z limits).
bool transpose_fits(int B, int C, int H, int W);

// [B][H][W][C] -> [B][C][H][W] and back; src and dst must not overlap.
hipError_t nhwc_to_nchw(const void* src, void* dst, int B, int C, int H, int W, bool bf16, hipStream_t st);
hipError_t nchw_to_nhwc(const void* src, void* dst, int B, int C, int H, int W, bool bf16, hipStream_t st);

}  // namespace wtc
