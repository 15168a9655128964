// Split (coarse + fine) forward / backward-data path for large planes.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace wtc {

typedef hipError_t (*split_launch_fn)(const void* in, const float* w_base, const float* w_lvl,
                                      const float* scale, void* out, float* ws, int B, int C,
                                      hipStream_t stream);

struct SplitEntry {
    int H, W, L, KB, K, L0;
    split_launch_fn fn[2][2];          // [dtype][flip]
    size_t (*ws_bytes)(int B, int C);  // the coarse image C per plane, fp32
};

const SplitEntry* find_split_entry(int H, int W, int L, int KB, int K);

}  // namespace wtc
