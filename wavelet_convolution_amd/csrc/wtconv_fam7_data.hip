// Forward / backward-data kernels of the 7x7 members of the stage-plane
// family (plans and entries: wtconv_family.h).
#include "wtconv_family.h"

namespace wtc {

static const PlaneEntry kFam7Data[] = {WTC_FAM_7(WTC_FAM_DATA)};

const PlaneEntry* find_fam7_data(int H, int W, int L, int KB, int K) {
    return fam_find(kFam7Data, (int)(sizeof(kFam7Data) / sizeof(kFam7Data[0])), H, W, L, KB, K);
}

}  // namespace wtc
