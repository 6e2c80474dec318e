// libtgemm registry: the direct kernel's compiled configurations (A [M,K], B [N,K]).
#include "direct.hpp"
#include "launch.hpp"

namespace tgemm_reg {
namespace {
template <int DT, int G>
hipError_t launch_direct(const void* A, const void* B, void* C, int M, int N, int K, int lda,
                         int ldb, int ldc, int group_m, hipStream_t s) {
    const int gm = cdiv(M, 32), gn = cdiv(N, 32);
    hipLaunchKernelGGL((tgemm::gemm_direct<DT, G>), dim3((unsigned)(gm * gn)), dim3(256), 0, s,
                       KARGS, gm, gn, group_m);
    return hipGetLastError();
}
// 32 x 32 C tiles, four waves splitting K in 16-wide blocks, two batches of G = 8 blocks
// in flight per wave.
#define DIRECT(DT)                                                                         \
    Variant {                                                                              \
        DT, 0, 0, tgemm_config{TGEMM_KERNEL_DIRECT, 32, 32, 16, 1, 1, 2, 8, 4, 32},        \
            &launch_direct<DT, 8>                                                          \
    }
const Variant kList[] = {DIRECT(0), DIRECT(1)};
}  // namespace
VariantList variants_direct() { return {kList, (int)(sizeof(kList) / sizeof(kList[0]))}; }
}  // namespace tgemm_reg
