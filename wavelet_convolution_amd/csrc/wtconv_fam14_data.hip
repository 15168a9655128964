// Forward / backward-data kernels of the 14x14 members of the stage-plane
// family (plans and entries: wtconv_family.h).
#include "wtconv_family.h"

namespace wtc {

static const PlaneEntry kFam14Data[] = {WTC_FAM_14(WTC_FAM_DATA)};

const PlaneEntry* find_fam14_data(int H, int W, int L, int KB, int K) {
    return fam_find(kFam14Data, (int)(sizeof(kFam14Data) / sizeof(kFam14Data[0])), H, W, L, KB, K);
}

}  // namespace wtc
