// Forward / backward-data kernel for L = 0, where the layer is the plain
// depthwise k_b x k_b cross-correlation with zero 'same' padding (the
// convolution WTConv stands in for; the abstract of arXiv:2608.10805 compares
// the two). Backward data is the same correlation with the taps turned by
// 180 degrees.
//
// One workgroup per channel and group of NPW images: the planes are zeroed
// in LDS with vector stores, their interiors streamed in once (widened to
// fp32), then every lane computes an RB-row column strip (conv_col: window
// rows are runs of consecutive LDS words across the wavefront) and stores it.
#include "wtconv_dw.h"

namespace wtc {
namespace {

template <class P, typename T, bool FLIP>
__global__ __launch_bounds__(P::NT) void dw_kernel(const T* __restrict__ in, const float* __restrict__ w_base,
                                                   T* __restrict__ out, int B, int C) {
    constexpr int H = P::H, W = P::W, KB = P::KB, NT = P::NT, RB = P::RB, NPW = P::NPW;
    constexpr int PB = P::PB, XO = P::XO, SX = P::SX, VA = P::VA, NQ = P::NQ, LPB = P::LPB, NIB = P::NIB;
    constexpr int PL = round_up(P::XSIZE, 4), KB2P = P::KB2P;
    __shared__ __attribute__((aligned(16))) float lds[NPW * PL + KB2P];
    float* const WB = lds + NPW * PL;

    const int tid = threadIdx.x;
    const int c = blockIdx.x % C, g = blockIdx.x / C;
    auto live = [&](int p) { return NPW == 1 || g * NPW + p < B; };
    // the workgroup's first plane is a uniform base; plane p lies p*C*H*W
    // elements further on (the host keeps NPW*C*H*W below 2^32)
    const size_t g0 = ((size_t)g * NPW * C + c) * H * W;
    auto plane_rel = [&](int p) -> uint32_t { return NPW == 1 ? 0u : (uint32_t)p * ((uint32_t)C * (H * W)); };

    for (int t = tid; t < KB2P; t += NT)
        WB[t] = t < KB * KB ? w_base[(size_t)c * KB * KB + (FLIP ? KB * KB - 1 - t : t)] : 0.f;
    {
        float4* const z = reinterpret_cast<float4*>(lds);
        for (int t = tid; t < NPW * PL / 4; t += NT) z[t] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
    // interiors: VA consecutive activations of one row per item
    for (int q = tid; q < NPW * NQ; q += NT) {
        const int p = udiv(q, NQ), r = q - p * NQ, row = udiv(r, W / VA), col = (r - row * (W / VA)) * VA;
        if (!live(p)) continue;
        RawVec<T, VA> v;
        load_raw<T, VA>(in + g0 + (plane_rel(p) + (uint32_t)(row * W + col)), v);
        store_lds<T, VA>(lds + p * PL + (PB + row) * SX + XO + col, v);
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < P::MB; ++it) {
        const int item = tid + it * NT;
        if (!((NPW * NIB) % NT == 0 || item < NPW * NIB)) continue;
        const int p = NPW == 1 ? 0 : udiv(item, NIB), r = item - p * NIB;
        const int rb = udiv(r, LPB), w = r - rb * LPB, h0 = rb * RB;
        if (!(LPB == W || w < W) || !live(p)) continue;
        float y[RB];
        conv_col<KB, RB, SX>(lds + p * PL + XO - PB + h0 * SX + w, WB, y);
        T* __restrict__ dst = out + g0 + (plane_rel(p) + (uint32_t)(h0 * W + w));
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int o = 0; o + 1 < RB; o += 2) {
                const uint32_t pr = narrow_bf16x2(y[o], y[o + 1]);
                dst[o * W] = (bf16_t)(pr & 0xffffu);
                dst[(o + 1) * W] = (bf16_t)(pr >> 16);
            }
            if constexpr (RB % 2 == 1) dst[(RB - 1) * W] = narrow_bf16(y[RB - 1]);
        } else {
#pragma unroll
            for (int o = 0; o < RB; ++o) dst[o * W] = y[o];
        }
    }
}

template <class P, typename T, bool FLIP>
hipError_t launch_dw(const void* in, const float* wb, void* out, int B, int C, hipStream_t stream) {
    const unsigned groups = (unsigned)cdiv(B, P::NPW) * (unsigned)C;
    hipLaunchKernelGGL((dw_kernel<P, T, FLIP>), dim3(groups), dim3(P::NT), 0, stream, (const T*)in, wb, (T*)out, B,
                       C);
    return hipGetLastError();
}

#define WTC_DW_ENTRY(PLAN)                                                                    \
    {PLAN::H, PLAN::W, PLAN::KB,                                                             \
     {{launch_dw<PLAN, float, false>, launch_dw<PLAN, float, true>},                         \
      {launch_dw<PLAN, bf16_t, false>, launch_dw<PLAN, bf16_t, true>}},                      \
     PLAN::NPW}

// the ConvNeXt-stage planes with the base kernels of the pages' workloads
typedef DwPlan<56, 56, 5, 256, 14, 1> DP_56_k5;
typedef DwPlan<56, 56, 7, 256, 14, 1> DP_56_k7;
typedef DwPlan<28, 28, 5, 256, 7, 2> DP_28_k5;
typedef DwPlan<28, 28, 7, 256, 7, 2> DP_28_k7;
typedef DwPlan<14, 14, 5, 256, 14, 16> DP_14_k5;
typedef DwPlan<14, 14, 7, 256, 14, 16> DP_14_k7;

const DwEntry kDwEntries[] = {
    WTC_DW_ENTRY(DP_56_k5), WTC_DW_ENTRY(DP_56_k7), WTC_DW_ENTRY(DP_28_k5),
    WTC_DW_ENTRY(DP_28_k7), WTC_DW_ENTRY(DP_14_k5), WTC_DW_ENTRY(DP_14_k7),
};

}  // namespace

const DwEntry* find_dw_entry(int H, int W, int KB) {
    for (const DwEntry& e : kDwEntries)
        if (e.H == H && e.W == W && e.KB == KB) return &e;
    return nullptr;
}

}  // namespace wtc
