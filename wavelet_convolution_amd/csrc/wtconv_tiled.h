// Split (coarse + fine) forward / backward-data path for large planes.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace wtc {

typedef hipError_t (*split_launch_fn)(const void* in, const float* w_base, const float* w_lvl,
                                      const float* scale, void* out, float* ws, int B, int C,
                                      hipStream_t stream);

struct FinalizeArgs;

// Backward data of a split plane whose coarse pass reads `sums`, the fp32
// planes [B][C][H >> L0][W >> L0] of unnormalised level-L0 LL sums of dy
// (2^L0 x 2^L0 block sums), instead of summing dy itself. fin (or null): a
// weight-gradient second stage for the coarse pass's launch to run as extra
// workgroups (the caller has checked that its scratch fits that kernel's LDS,
// `coarse_lds_bytes`).
typedef hipError_t (*split_sums_fn)(const void* in, const float* sums, const float* w_base, const float* w_lvl,
                                    const float* scale, void* out, float* ws, int B, int C, hipStream_t stream,
                                    const FinalizeArgs* fin);

struct SplitEntry {
    int H, W, L, KB, K, L0;
    split_launch_fn fn[2][2];          // [dtype][flip]
    size_t (*ws_bytes)(int B, int C);  // the coarse image C per plane, fp32
    split_sums_fn bwd_data_from_sums[2];   // [dtype]; null where L = L0 (no coarse pass)
    size_t coarse_lds_bytes;               // LDS of the coarse pass's workgroups
};

const SplitEntry* find_split_entry(int H, int W, int L, int KB, int K);

}  // namespace wtc
