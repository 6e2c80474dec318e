// libtgemm registry: the tiled kernel's masked form for A [M,K] with B [N,K], both read
// as the aligned 16-byte blocks around each tile-row piece and realigned in registers.
// The 256x256 tile keeps one register in scratch memory, stored once before the K loop
// and reloaded after it.
#include "launch.hpp"

namespace tgemm_reg {
namespace {
#define MASKED_NK(DT)                                                                      \
    MASKED_TILED(DT, 0, 0, 256, 256, 64, 2, 2, 4), MASKED_TILED(DT, 0, 0, 128, 256, 64, 2, 2, 8), \
        MASKED_TILED(DT, 0, 0, 256, 128, 64, 2, 2, 8),                                     \
        MASKED_TILED(DT, 0, 0, 128, 128, 64, 2, 2, 8), MASKED_TILED(DT, 0, 0, 64, 64, 64, 2, 2, 8)
const Variant kList[] = {MASKED_NK(0), MASKED_NK(1)};
}  // namespace
VariantList variants_masked_nk() { return {kList, (int)(sizeof(kList) / sizeof(kList[0]))}; }
}  // namespace tgemm_reg
