// libtgemm registry: the ping-pong kernel's compiled configurations for B [K,N] and for
// A [K,M] (transposing LDS reads).
#include "launch.hpp"

namespace tgemm_reg {
namespace {
#define PP_MK_KN(DT)                                                                       \
    PINGPONG(DT, 0, 1, 256, 256, 64, 2, 4), PINGPONG(DT, 0, 1, 256, 256, 32, 5, 4)
#define PP_KM(DT, L) PINGPONG(DT, 1, L, 256, 256, 32, 4, 4)
const Variant kList[] = {
    PP_MK_KN(0), PP_MK_KN(1),
    PP_KM(0, 0), PP_KM(1, 0), PP_KM(0, 1), PP_KM(1, 1),
};
}  // namespace
VariantList variants_pingpong_other() {
    return {kList, (int)(sizeof(kList) / sizeof(kList[0]))};
}
}  // namespace tgemm_reg
