// libtgemm registry: the any-alignment kernel (every storage), for A [M,K] with B [N,K]
// the deep direct-to-LDS ring, the skinny kernel and split-K over workgroups, and the
// skinny kernel for B [K,N].
#include "launch.hpp"

namespace tgemm_reg {
namespace {
#define SMALL_MK_NK(DT)                                                                    \
    GENERIC(DT, 0, 0), DMA(DT, 256, 256, 32, 2, 2, 4, 4), DMA(DT, 256, 256, 32, 2, 2, 5, 4), \
        DMA(DT, 64, 128, 64, 1, 4, 4, 2), DMA(DT, 64, 256, 64, 1, 4, 4, 2),               \
        SKINNY(DT, 1, 4), SKINNY(DT, 2, 3), SKINNY(DT, 4, 1), SKINNY_WIDE(DT, 1, 1),       \
        SKINNY_WIDE4(DT, 2, 1), SKINNY_N64(DT, 1, 64, 8, 2), SKINNY_N64(DT, 2, 64, 8, 1),  \
        SPLITK(DT, 64, 256, 32, 1, 4, 5, 1), SPLITK(DT, 64, 128, 32, 1, 4, 5, 1),          \
        SPLITK(DT, 64, 256, 64, 1, 4, 4, 1), SPLITK(DT, 64, 128, 64, 1, 4, 4, 1),          \
        SPLITK(DT, 64, 128, 64, 1, 4, 6, 1)
const Variant kList[] = {
    SMALL_MK_NK(0), SMALL_MK_NK(1),
    SKINNY_KN(0, 1, 4), SKINNY_KN(0, 2, 3), SKINNY_KN(0, 4, 1),
    SKINNY_KN(1, 1, 4), SKINNY_KN(1, 2, 3), SKINNY_KN(1, 4, 1),
    GENERIC(0, 0, 1), GENERIC(1, 0, 1),
    GENERIC(0, 1, 0), GENERIC(1, 1, 0), GENERIC(0, 1, 1), GENERIC(1, 1, 1),
};
}  // namespace
VariantList variants_small() { return {kList, (int)(sizeof(kList) / sizeof(kList[0]))}; }
}  // namespace tgemm_reg
