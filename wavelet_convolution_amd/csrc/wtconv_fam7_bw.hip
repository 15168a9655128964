// Weight-gradient kernels of the 7x7 members of the stage-plane family
// (plans and entries: wtconv_family.h).
#include "wtconv_family.h"

namespace wtc {

static const BwEntry kFam7Bw[] = {WTC_FAM_7(WTC_FAM_BW)};

const BwEntry* find_fam7_bw(int H, int W, int L, int KB, int K) {
    return fam_find(kFam7Bw, (int)(sizeof(kFam7Bw) / sizeof(kFam7Bw[0])), H, W, L, KB, K);
}

}  // namespace wtc
