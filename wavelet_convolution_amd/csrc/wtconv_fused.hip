// Registry of the whole-plane forward / backward-data kernels (the kernel
// itself is in wtconv_plane.h).
#include "wtconv_plane.h"

namespace wtc {

template <class P, typename T, bool FLIP>
static hipError_t launch_plane(const void* in, const float* wb, const float* wl, const float* sc,
                               void* out, int B, int C, hipStream_t stream) {
    const unsigned planes = (unsigned)B * (unsigned)C;
    hipLaunchKernelGGL((plane_kernel<P, T, FLIP, 0, T>), dim3(planes), dim3(P::NT), 0, stream,
                       (const T*)in, wb, wl, sc, (T*)out, C);
    return hipGetLastError();
}

template <class P, typename T, bool FLIP>
static hipError_t launch_col(const void* in, const float* wb, const float* wl, const float* sc, void* out,
                             int B, int C, hipStream_t stream) {
    // one workgroup per channel and group of NPW images
    const unsigned groups = (unsigned)cdiv(B, P::NPW) * (unsigned)C;
    hipLaunchKernelGGL((col_kernel<P, T, FLIP>), dim3(groups), dim3(P::NT), 0, stream, (const T*)in, wb, wl, sc,
                       (T*)out, B, C);
    return hipGetLastError();
}

#define WTC_COL_ENTRY(PLAN)                                                                   \
    {PLAN::H, PLAN::W, PLAN::L, PLAN::KB, PLAN::K,                                           \
     {{launch_col<PLAN, float, false>, launch_col<PLAN, float, true>},                       \
      {launch_col<PLAN, bf16_t, false>, launch_col<PLAN, bf16_t, true>}},                    \
     PLAN::TOTAL_FLOATS * 4, PLAN::NT, PLAN::NPW}

#define WTC_PLANE_ENTRY(PLAN)                                                                 \
    {PLAN::H, PLAN::W, PLAN::L, PLAN::KB, PLAN::K,                                           \
     {{launch_plane<PLAN, float, false>, launch_plane<PLAN, float, true>},                   \
      {launch_plane<PLAN, bf16_t, false>, launch_plane<PLAN, bf16_t, true>}},                \
     (PLAN::LDS_FLOATS + PLAN::WFLOATS) * 4, PLAN::NT, 1}

static const PlaneEntry kPlaneEntries[] = {
    WTC_COL_ENTRIES(WTC_COL_ENTRY),
    WTC_PLANE_ENTRIES(WTC_PLANE_ENTRY)
};

const PlaneEntry* find_plane_entry(int H, int W, int L, int KB, int K) {
    for (const PlaneEntry& e : kPlaneEntries)
        if (e.H == H && e.W == W && e.L == L && e.KB == KB && e.K == K) return &e;
    return nullptr;
}

}  // namespace wtc
