// libtgemm registry: the quadrant kernel's compiled configurations for A [M,K], B [K,N].
#include "launch.hpp"

namespace tgemm_reg {
namespace {
const Variant kList[] = {
    QUAD_KN(0, 16, 4), QUAD_KN(0, 32, 4),
    QUAD_KN(1, 16, 4), QUAD_KN(1, 32, 4),
    QUAD192(0, 16, 1, 4), QUAD192(0, 32, 1, 4),
    QUAD192(1, 16, 1, 4), QUAD192(1, 32, 1, 4),
};
}  // namespace
VariantList variants_quad_kn() {
    return {kList, (int)(sizeof(kList) / sizeof(kList[0]))};
}
}  // namespace tgemm_reg
