// Weight-gradient kernels of the 14x14 members of the stage-plane family
// (plans and entries: wtconv_family.h).
#include "wtconv_family.h"

namespace wtc {

static const BwEntry kFam14Bw[] = {WTC_FAM_14(WTC_FAM_BW)};

const BwEntry* find_fam14_bw(int H, int W, int L, int KB, int K) {
    return fam_find(kFam14Bw, (int)(sizeof(kFam14Bw) / sizeof(kFam14Bw[0])), H, W, L, KB, K);
}

}  // namespace wtc
