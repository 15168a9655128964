// Forward / backward-data kernels of the 28x28 members of the stage-plane
// family (plans and entries: wtconv_family.h).
#include "wtconv_family.h"

namespace wtc {

static const PlaneEntry kFam28Data[] = {WTC_FAM_28(WTC_FAM_DATA)};

const PlaneEntry* find_fam28_data(int H, int W, int L, int KB, int K) {
    return fam_find(kFam28Data, (int)(sizeof(kFam28Data) / sizeof(kFam28Data[0])), H, W, L, KB, K);
}

}  // namespace wtc
