// libtgemm registry: the register-staged tiled kernel's compiled configurations, every
// storage of A and B.
#include "launch.hpp"

namespace tgemm_reg {
namespace {
#define TILED_MK(DT, L)                                                                    \
    TILED(DT, 0, L, 256, 256, 64, 2, 2, 4), TILED(DT, 0, L, 256, 128, 64, 2, 2, 8),        \
        TILED(DT, 0, L, 128, 256, 64, 2, 2, 8), TILED(DT, 0, L, 128, 128, 64, 2, 2, 8),    \
        TILED(DT, 0, L, 64, 64, 64, 2, 2, 8)
#define TILED_KM(DT, L)                                                                    \
    TILED(DT, 1, L, 128, 128, 64, 2, 2, 8), TILED(DT, 1, L, 64, 64, 64, 2, 2, 8)
const Variant kList[] = {
    TILED_MK(0, 0), TILED_MK(1, 0), TILED_MK(0, 1), TILED_MK(1, 1),
    TILED_KM(0, 0), TILED_KM(1, 0), TILED_KM(0, 1), TILED_KM(1, 1),
};
}  // namespace
VariantList variants_tiled() { return {kList, (int)(sizeof(kList) / sizeof(kList[0]))}; }
}  // namespace tgemm_reg
