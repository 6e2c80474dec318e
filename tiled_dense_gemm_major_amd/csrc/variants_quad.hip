// libtgemm registry: the quadrant kernel's compiled configurations for A [M,K], B [N,K].
#include "launch.hpp"

namespace tgemm_reg {
namespace {
const Variant kList[] = {
    QUAD(0, 16, 4), QUAD(0, 32, 4),
    QUAD(1, 16, 4), QUAD(1, 32, 4),
    QUAD192(0, 16, 0, 4), QUAD192(0, 32, 0, 4),
    QUAD192(1, 16, 0, 4), QUAD192(1, 32, 0, 4),
};
}  // namespace
VariantList variants_quad() { return {kList, (int)(sizeof(kList) / sizeof(kList[0]))}; }
}  // namespace tgemm_reg
