// libtgemm: the registry of compiled kernel configurations.  The variants live in
// several translation units (variants_*.hip, compiled in parallel); each exports its
// list, and the host code (tgemm.hip) merges them in a fixed order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tgemm.h"

namespace tgemm_reg {

// Leading dimensions are in elements: A[m*lda + k] ([M,K]) or A[k*lda + m] ([K,M]);
// B[n*ldb + k] ([N,K]) or B[k*ldb + n] ([K,N]); C[m*ldc + n].
typedef hipError_t (*launch_fn)(const void* A, const void* B, void* C, int M, int N, int K,
                                int lda, int ldb, int ldc, int group_m, hipStream_t s);
// Split-K launches also take the number of K splits and the caller's workspace.
typedef hipError_t (*splitk_fn)(const void* A, const void* B, void* C, int M, int N, int K,
                                int lda, int ldb, int ldc, int group_m, int splits, void* ws,
                                hipStream_t s);

// Split-K bounds: at least 2 and at most kMaxSplits workgroups per C tile.
constexpr int kMaxSplits = 64;

struct Variant {
    int dtype;
    int a_layout;
    int layout;
    tgemm_config cfg;
    launch_fn launch;              // every kernel but the split-K ones
    splitk_fn split_launch;        // SPLITK and QUAD_SPLITK only
};

struct VariantList {
    const Variant* v;
    int n;
};

// One list per translation unit.
VariantList variants_quad();
VariantList variants_quad_kn();
VariantList variants_quad_km();
VariantList variants_direct();
VariantList variants_quad_split();
VariantList variants_pingpong_nk();
VariantList variants_pingpong_other();
VariantList variants_tiled();
VariantList variants_masked();
VariantList variants_masked_nk();
VariantList variants_small();

}  // namespace tgemm_reg
