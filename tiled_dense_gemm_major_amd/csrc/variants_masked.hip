// libtgemm registry: the tiled kernel's masked form (any 2-byte alignment and any sizes)
// for A [M,K] with B [K,N], and for A [K,M] with either B.  Operands stored with K as the
// row index are read as 2-byte elements, each held in a whole register until its LDS
// write: 128x128 tiles fit, larger ones would spill.
#include "launch.hpp"

namespace tgemm_reg {
namespace {
#define MASKED_SMALL(DT, AL, L)                                                            \
    MASKED_TILED(DT, AL, L, 128, 128, 64, 2, 2, 8), MASKED_TILED(DT, AL, L, 64, 64, 64, 2, 2, 8)
const Variant kList[] = {
    MASKED_SMALL(0, 0, 1), MASKED_SMALL(1, 0, 1), MASKED_SMALL(0, 1, 0),
    MASKED_SMALL(1, 1, 0), MASKED_SMALL(0, 1, 1), MASKED_SMALL(1, 1, 1),
};
}  // namespace
VariantList variants_masked() { return {kList, (int)(sizeof(kList) / sizeof(kList[0]))}; }
}  // namespace tgemm_reg
