// libtgemm registry: the quadrant kernel in split-K and stream-K modes (A [M,K]; B [N,K]
// with 16x16x32 MFMAs, B [K,N] with 32x32x16, the forms the table picks for the large
// products of each storage).
#include "launch.hpp"

namespace tgemm_reg {
namespace {
const Variant kList[] = {
    QUAD_SPLIT(0, 16, 0, 4), QUAD_SPLIT(1, 16, 0, 4),
    QUAD_SPLIT(0, 32, 1, 4), QUAD_SPLIT(1, 32, 1, 4),
    QUAD_SK(0, 16, 0, 4),    QUAD_SK(1, 16, 0, 4),
    QUAD_SK(0, 32, 1, 4),    QUAD_SK(1, 32, 1, 4),
};
}  // namespace
VariantList variants_quad_split() { return {kList, (int)(sizeof(kList) / sizeof(kList[0]))}; }
}  // namespace tgemm_reg
