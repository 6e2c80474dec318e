// libtgemm registry: the ping-pong kernel's compiled configurations for A [M,K], B [N,K].
#include "launch.hpp"

namespace tgemm_reg {
namespace {
#define PP_MK_NK(DT)                                                                       \
    PINGPONG(DT, 0, 0, 256, 256, 64, 2, 4), PINGPONG(DT, 0, 0, 256, 256, 32, 4, 4),        \
        PINGPONG(DT, 0, 0, 256, 256, 32, 5, 4)
const Variant kList[] = {PP_MK_NK(0), PP_MK_NK(1)};
}  // namespace
VariantList variants_pingpong_nk() {
    return {kList, (int)(sizeof(kList) / sizeof(kList[0]))};
}
}  // namespace tgemm_reg
