// libtgemm registry: the tiled kernel's masked form (element-wise loads and stores, any
// 2-byte alignment and any sizes), every storage of A and B.  Each 2-byte load holds a
// whole register until the LDS write packs it, so the register prefetch of a tile takes
// twice the registers of the 16-byte loads: 128x128 tiles fit, 256x256 ones would spill.
#include "launch.hpp"

namespace tgemm_reg {
namespace {
#define MASKED_ALL(DT, AL, L)                                                              \
    MASKED_TILED(DT, AL, L, 128, 128, 64, 2, 2, 8), MASKED_TILED(DT, AL, L, 64, 64, 64, 2, 2, 8)
const Variant kList[] = {
    MASKED_ALL(0, 0, 0), MASKED_ALL(1, 0, 0), MASKED_ALL(0, 0, 1), MASKED_ALL(1, 0, 1),
    MASKED_ALL(0, 1, 0), MASKED_ALL(1, 1, 0), MASKED_ALL(0, 1, 1), MASKED_ALL(1, 1, 1),
};
}  // namespace
VariantList variants_masked() { return {kList, (int)(sizeof(kList) / sizeof(kList[0]))}; }
}  // namespace tgemm_reg
