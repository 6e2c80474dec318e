// libtgemm registry: the quadrant kernel's compiled configurations for A [K,M] (32x32x16
// MFMAs: the 16x16x32 form needs more registers than a wave has and spills).
#include "launch.hpp"

namespace tgemm_reg {
namespace {
const Variant kList[] = {
    QUAD_KM(0, 32, 0, 4), QUAD_KM(1, 32, 0, 4),
    QUAD_KM(0, 32, 1, 4), QUAD_KM(1, 32, 1, 4),
};
}  // namespace
VariantList variants_quad_km() {
    return {kList, (int)(sizeof(kList) / sizeof(kList[0]))};
}
}  // namespace tgemm_reg
