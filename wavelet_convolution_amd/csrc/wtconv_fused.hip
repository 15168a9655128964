// Registry of the whole-plane forward / backward-data kernels (the kernel
// itself is in wtconv_plane.h).
#include "wtconv_family.h"
#include "wtconv_plane.h"

namespace wtc {

#define WTC_COL_ENTRY(PLAN)                                                                   \
    {PLAN::H, PLAN::W, PLAN::L, PLAN::KB, PLAN::K,                                           \
     {{launch_col<PLAN, float, false>, launch_col<PLAN, float, true>},                       \
      {launch_col<PLAN, bf16_t, false>, launch_col<PLAN, bf16_t, true>}},                    \
     PLAN::TOTAL_FLOATS * 4, PLAN::NT, PLAN::NPW}

#define WTC_PLANE_ENTRY(PLAN)                                                                 \
    {PLAN::IH, PLAN::IW, PLAN::L, PLAN::KB, PLAN::K,                                         \
     {{launch_plane<PLAN, float, false>, launch_plane<PLAN, float, true>},                   \
      {launch_plane<PLAN, bf16_t, false>, launch_plane<PLAN, bf16_t, true>}},                \
     (PLAN::LDS_FLOATS + PLAN::WFLOATS) * 4, PLAN::NT, 1}

static const PlaneEntry kPlaneEntries[] = {
    WTC_COL_ENTRIES(WTC_COL_ENTRY),
    WTC_PLANE_ENTRIES(WTC_PLANE_ENTRY)
};

// the tuned plans first, then the stage-plane family
const PlaneEntry* find_plane_entry(int H, int W, int L, int KB, int K) {
    for (const PlaneEntry& e : kPlaneEntries)
        if (e.H == H && e.W == W && e.L == L && e.KB == KB && e.K == K) return &e;
    return find_family_plane_entry(H, W, L, KB, K);
}

}  // namespace wtc
