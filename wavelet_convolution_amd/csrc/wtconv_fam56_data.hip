// Forward / backward-data kernels of the 56x56 members of the stage-plane
// family (plans and entries: wtconv_family.h).
#include "wtconv_family.h"

namespace wtc {

static const PlaneEntry kFam56Data[] = {WTC_FAM_56(WTC_FAM_DATA)};

const PlaneEntry* find_fam56_data(int H, int W, int L, int KB, int K) {
    return fam_find(kFam56Data, (int)(sizeof(kFam56Data) / sizeof(kFam56Data[0])), H, W, L, KB, K);
}

}  // namespace wtc
