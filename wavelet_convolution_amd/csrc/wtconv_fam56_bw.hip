// Weight-gradient kernels of the 56x56 members of the stage-plane family
// (plans and entries: wtconv_family.h).
#include "wtconv_family.h"

namespace wtc {

static const BwEntry kFam56Bw[] = {WTC_FAM_56(WTC_FAM_BW)};

const BwEntry* find_fam56_bw(int H, int W, int L, int KB, int K) {
    return fam_find(kFam56Bw, (int)(sizeof(kFam56Bw) / sizeof(kFam56Bw[0])), H, W, L, KB, K);
}

}  // namespace wtc
