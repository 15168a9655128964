// L = 0: the layer without its wavelet branch is the plain depthwise k_b x k_b
// cross-correlation (the convolution WTConv stands in for). Plans for the
// whole-plane kernels of that case: the forward / backward-data kernel in
// wtconv_dw.hip, the weight gradient in wtconv_bwdw.hip.
#pragma once

#include "wtconv_device.h"

namespace wtc {

// H x W planes, k_b x k_b taps; NT lanes per workgroup, base strips of RB
// rows x 1 column, NPW images of one channel per workgroup (data kernel) or
// per step (weight kernel).
template <int H_, int W_, int KB_, int NT_, int RB_, int NPW_>
struct DwPlan {
    static constexpr int H = H_, W = W_, KB = KB_, NT = NT_, RB = RB_, NPW = NPW_;
    static constexpr int PB = KB / 2;
    static_assert(KB % 2 == 1 && H % RB == 0 && NT % 64 == 0 && NT <= 1024, "plan shape");
    // x rows: interior from column XO (a multiple of 4), stride a multiple of 4
    static constexpr int XO = round_up(PB, 4);
    static constexpr int SX = round_up(XO + W + PB, 4);
    static constexpr int XSIZE = (H + 2 * PB) * SX;
    static constexpr int VA = lds_vec(W);   // activations per stream-in item
    static constexpr int NQ = H * (W / VA);  // stream-in items of one plane
    static constexpr int LPB = strip_lanes(W);
    static constexpr int NIB = (H / RB) * LPB;   // strip slots of one plane
    static constexpr int MB = cdiv(NPW * NIB, NT);
    static constexpr int KB2P = kpad4(KB);
    // weight kernel: dy rows next to the bordered x plane
    static constexpr int SD = round_up(W, 4);
    static constexpr int DSIZE = H * SD;
};

typedef hipError_t (*dw_launch_fn)(const void* in, const float* w_base, void* out, int B, int C,
                                   hipStream_t stream);

struct DwEntry {
    int H, W, KB;
    dw_launch_fn fn[2][2];   // [dtype: 0 fp32, 1 bf16][flip: 0 fwd, 1 bwd_data]
    int npw;                 // images per workgroup: the kernel needs npw*C*H*W < 2^32
};

// The data kernel's plan for this plane and base kernel, or nullptr.
const DwEntry* find_dw_entry(int H, int W, int KB);

}  // namespace wtc
