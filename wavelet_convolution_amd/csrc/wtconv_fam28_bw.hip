// Weight-gradient kernels of the 28x28 members of the stage-plane family
// (plans and entries: wtconv_family.h).
#include "wtconv_family.h"

namespace wtc {

static const BwEntry kFam28Bw[] = {WTC_FAM_28(WTC_FAM_BW)};

const BwEntry* find_fam28_bw(int H, int W, int L, int KB, int K) {
    return fam_find(kFam28Bw, (int)(sizeof(kFam28Bw) / sizeof(kFam28Bw[0])), H, W, L, KB, K);
}

}  // namespace wtc
