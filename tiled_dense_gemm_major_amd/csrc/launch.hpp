// libtgemm: the launchers of every kernel family and the macros that name one compiled
// configuration of the registry.  Included by the variants_*.hip translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"
#include "registry.hpp"

namespace tgemm_reg {

using tgemm::u16;

inline int cdiv(int a, int b) { return (a + b - 1) / b; }

#define KARGS                                                                              \
    static_cast<const u16*>(A), static_cast<const u16*>(B), static_cast<u16*>(C), M, N, K, \
        lda, ldb, ldc

template <int DT, int AL, int LAYOUT, int BM, int BN, int BK, int WM, int WN,
          bool MASKED = false>
hipError_t launch_tiled(const void* A, const void* B, void* C, int M, int N, int K, int lda,
                        int ldb, int ldc, int group_m, hipStream_t s) {
    const int gm = cdiv(M, BM), gn = cdiv(N, BN);
    hipLaunchKernelGGL((tgemm::gemm_tiled<DT, AL, LAYOUT, BM, BN, BK, WM, WN, MASKED>),
                       dim3((unsigned)(gm * gn)), dim3(WM * WN * 64), 0, s, KARGS, gm, gn,
                       group_m);
    return hipGetLastError();
}

template <int DT, int BM, int BN, int BK, int WM, int WN, int STAGES>
hipError_t launch_dma(const void* A, const void* B, void* C, int M, int N, int K, int lda,
                      int ldb, int ldc, int group_m, hipStream_t s) {
    const int gm = cdiv(M, BM), gn = cdiv(N, BN);
    hipLaunchKernelGGL((tgemm::gemm_dma<DT, BM, BN, BK, WM, WN, STAGES, false>),
                       dim3((unsigned)(gm * gn)), dim3(WM * WN * 64), 0, s, KARGS, gm, gn,
                       group_m, static_cast<float*>(nullptr), 0);
    return hipGetLastError();
}

// Split-K: splits workgroups per C tile, each over a whole number of K steps, write fp32
// partial tiles to the workspace ([splits][M][N]); a second kernel sums them in split
// order and writes C.
template <int DT, int BM, int BN, int BK, int WM, int WN, int STAGES>
hipError_t launch_splitk(const void* A, const void* B, void* C, int M, int N, int K, int lda,
                         int ldb, int ldc, int group_m, int splits, void* ws, hipStream_t s) {
    const int gm = cdiv(M, BM), gn = cdiv(N, BN);
    const int kc = cdiv(cdiv(K, splits), BK) * BK;
    float* W = static_cast<float*>(ws);
    hipLaunchKernelGGL((tgemm::gemm_dma<DT, BM, BN, BK, WM, WN, STAGES, true>),
                       dim3((unsigned)(gm * gn), (unsigned)splits), dim3(WM * WN * 64), 0, s,
                       KARGS, gm, gn, group_m, W, kc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((tgemm::splitk_reduce<DT>), dim3((unsigned)cdiv(M * (N / 8), 256)),
                       dim3(256), 0, s, static_cast<const float*>(W), static_cast<u16*>(C), M,
                       N, ldc, splits);
    return hipGetLastError();
}

template <int DT, int AL, int LAYOUT, int BM, int BN, int BK, int S>
hipError_t launch_pingpong(const void* A, const void* B, void* C, int M, int N, int K, int lda,
                           int ldb, int ldc, int group_m, hipStream_t s) {
    const int gm = cdiv(M, BM), gn = cdiv(N, BN);
    hipLaunchKernelGGL((tgemm::gemm_pingpong<DT, AL, LAYOUT, BM, BN, BK, S>),
                       dim3((unsigned)(gm * gn)), dim3(512), 0, s, KARGS, gm, gn, group_m);
    return hipGetLastError();
}

template <int DT, int MF, int PRE, int SPA, int SPB, int STAG, int POL, int L = 0,
          int BM = 256, int AL = 0>
hipError_t launch_quad(const void* A, const void* B, void* C, int M, int N, int K, int lda,
                       int ldb, int ldc, int group_m, hipStream_t s) {
    const int gm = cdiv(M, BM), gn = cdiv(N, 256);
    // the instruction-offset form of the loads needs rows of at least 64 elements (an
    // operand stored [K,*]: 256, its loads' rows being only two apart)
    if (lda >= (AL == 0 ? 64 : 256) && ldb >= (L == 0 ? 64 : 256))
        hipLaunchKernelGGL(
            (tgemm::gemm_quad<DT, MF, PRE, SPA, SPB, STAG, POL, true, L, BM, AL>),
            dim3((unsigned)(gm * gn)), dim3(256), 0, s, KARGS, gm, gn, group_m);
    else
        hipLaunchKernelGGL(
            (tgemm::gemm_quad<DT, MF, PRE, SPA, SPB, STAG, POL, false, L, BM, AL>),
            dim3((unsigned)(gm * gn)), dim3(256), 0, s, KARGS, gm, gn, group_m);
    return hipGetLastError();
}

// The quad kernel in split-K mode: grid (tiles, splits), each split a whole number of
// 64-wide K steps (the last one what remains), then the fixed-order reduction.
template <int DT, int MF, int PRE, int SPA, int SPB, int STAG, int POL, int L = 0>
hipError_t launch_quad_split(const void* A, const void* B, void* C, int M, int N, int K,
                             int lda, int ldb, int ldc, int group_m, int splits, void* ws,
                             hipStream_t s) {
    const int gm = cdiv(M, 256), gn = cdiv(N, 256);
    const int kc = cdiv(cdiv(K, splits), 64) * 64;
    float* W = static_cast<float*>(ws);
    const auto a = static_cast<const tgemm::u16*>(A);
    const auto b = static_cast<const tgemm::u16*>(B);
    const dim3 grid((unsigned)(gm * gn), (unsigned)splits);
    if (lda >= 64 && ldb >= (L == 0 ? 64 : 256))
        hipLaunchKernelGGL((tgemm::gemm_quad_split<DT, MF, PRE, SPA, SPB, STAG, POL, true, L>),
                           grid, dim3(256), 0, s, a, b, M, N, K, lda, ldb, gm, gn, group_m, W,
                           kc);
    else
        hipLaunchKernelGGL((tgemm::gemm_quad_split<DT, MF, PRE, SPA, SPB, STAG, POL, false, L>),
                           grid, dim3(256), 0, s, a, b, M, N, K, lda, ldb, gm, gn, group_m, W,
                           kc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((tgemm::splitk_reduce<DT>), dim3((unsigned)cdiv(M * (N / 8), 256)),
                       dim3(256), 0, s, static_cast<const float*>(W), static_cast<tgemm::u16*>(C),
                       M, N, ldc, splits);
    return hipGetLastError();
}

// Stream-K over the last partial wave, in one launch: the leading tile rows that fill
// whole waves of the 256 compute units as whole tiles, the remaining rows dealt to 256
// stream-K workgroups (dispatched first) in equal shares of their tiles' K steps, then
// the reduction of their partial tiles.  Without a partial wave (or with K = 0, or more
// than 256 remaining tiles) the product runs as the plain quad kernel.
constexpr int kStreamKGroups = 256;
template <int DT, int MF, int PRE, int SPA, int SPB, int STAG, int POL, int L = 0>
hipError_t launch_quad_sk(const void* A, const void* B, void* C, int M, int N, int K, int lda,
                          int ldb, int ldc, int group_m, int, void* ws, hipStream_t s) {
    const int gm = cdiv(M, 256), gn = cdiv(N, 256), nk = cdiv(K, 64);
    const int dp_rows = (gm * gn / kStreamKGroups) * kStreamKGroups / gn;
    const int m_dp = dp_rows * 256 < M ? dp_rows * 256 : M;
    const int rows_sk = M - m_dp;
    const int tiles_sk = cdiv(rows_sk, 256) * gn;
    if (nk == 0 || rows_sk == 0 || tiles_sk > kStreamKGroups)
        return launch_quad<DT, MF, PRE, SPA, SPB, STAG, POL, L>(A, B, C, M, N, K, lda, ldb, ldc,
                                                               group_m, s);
    const auto a = static_cast<const tgemm::u16*>(A);
    const auto b = static_cast<const tgemm::u16*>(B);
    const auto c = static_cast<tgemm::u16*>(C);
    float* W = static_cast<float*>(ws);
    const dim3 grid((unsigned)(kStreamKGroups + dp_rows * gn));
    if (lda >= 64 && ldb >= (L == 0 ? 64 : 256))
        hipLaunchKernelGGL((tgemm::gemm_quad_sk<DT, MF, PRE, SPA, SPB, STAG, POL, true, L>),
                           grid, dim3(256), 0, s, a, b, c, M, N, K, lda, ldb, ldc, gn, group_m,
                           dp_rows, nk, tiles_sk, kStreamKGroups, W);
    else
        hipLaunchKernelGGL((tgemm::gemm_quad_sk<DT, MF, PRE, SPA, SPB, STAG, POL, false, L>),
                           grid, dim3(256), 0, s, a, b, c, M, N, K, lda, ldb, ldc, gn, group_m,
                           dp_rows, nk, tiles_sk, kStreamKGroups, W);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((tgemm::sk_reduce<DT>), dim3((unsigned)cdiv(rows_sk * (N / 8), 256)),
                       dim3(256), 0, s, static_cast<const float*>(W), c + (size_t)m_dp * ldc,
                       rows_sk, N, ldc, gn, nk, tiles_sk, kStreamKGroups);
    return hipGetLastError();
}

template <int DT, int MT, int D, int CK = 64, int NW = 8, int NB = 1>
hipError_t launch_skinny(const void* A, const void* B, void* C, int M, int N, int K, int lda,
                         int ldb, int ldc, int, hipStream_t s) {
    hipLaunchKernelGGL((tgemm::gemm_skinny<DT, MT, D, CK, NW, NB>),
                       dim3((unsigned)cdiv(N, 32 * NB), (unsigned)cdiv(M, MT * 32)),
                       dim3(NW * 64),
                       0, s,
                       KARGS);
    return hipGetLastError();
}

template <int DT, int MT, int D>
hipError_t launch_skinny_kn(const void* A, const void* B, void* C, int M, int N, int K, int lda,
                            int ldb, int ldc, int, hipStream_t s) {
    hipLaunchKernelGGL((tgemm::gemm_skinny_kn<DT, MT, D>),
                       dim3((unsigned)cdiv(N, 32), (unsigned)cdiv(M, MT * 32)), dim3(512), 0, s,
                       KARGS);
    return hipGetLastError();
}

template <int DT, int AL, int LAYOUT>
hipError_t launch_generic(const void* A, const void* B, void* C, int M, int N, int K, int lda,
                          int ldb, int ldc, int group_m, hipStream_t s) {
    const int gm = cdiv(M, 64), gn = cdiv(N, 64);
    hipLaunchKernelGGL((tgemm::gemm_generic<DT, AL, LAYOUT>), dim3((unsigned)(gm * gn)),
                       dim3(256), 0, s, KARGS, gm, gn, group_m);
    return hipGetLastError();
}

#define TILED(DT, AL, L, BM, BN, BK, WM, WN, G)                                           \
    Variant {                                                                              \
        DT, AL, L, tgemm_config{TGEMM_KERNEL_TILED, BM, BN, BK, WM, WN, 2, G, 1, 32},          \
            &launch_tiled<DT, AL, L, BM, BN, BK, WM, WN>                                   \
    }
#define MASKED_TILED(DT, AL, L, BM, BN, BK, WM, WN, G)                                    \
    Variant {                                                                              \
        DT, AL, L, tgemm_config{TGEMM_KERNEL_MASKED, BM, BN, BK, WM, WN, 2, G, 1, 32},         \
            &launch_tiled<DT, AL, L, BM, BN, BK, WM, WN, true>                             \
    }
#define GENERIC(DT, AL, L)                                                                 \
    Variant {                                                                              \
        DT, AL, L, tgemm_config{TGEMM_KERNEL_GENERIC, 64, 64, 16, 2, 2, 1, 8, 1, 32},      \
            &launch_generic<DT, AL, L>                                                     \
    }
#define DMA(DT, BM, BN, BK, WM, WN, ST, G)                                                 \
    Variant {                                                                              \
        DT, 0, 0, tgemm_config{TGEMM_KERNEL_DMA, BM, BN, BK, WM, WN, ST, G, 1, 32},            \
            &launch_dma<DT, BM, BN, BK, WM, WN, ST>                                        \
    }
#define PINGPONG(DT, AL, L, BM, BN, BK, S, G)                                              \
    Variant {                                                                              \
        DT, AL, L, tgemm_config{TGEMM_KERNEL_PINGPONG, BM, BN, BK, 2, 4, S, G, 1, 32},         \
            &launch_pingpong<DT, AL, L, BM, BN, BK, S>                                     \
    }
// Quad kernel schedules (pre-barrier MFMAs, A-load and read spreads), from the sweep;
// K walks staggered per XCD, loads with the sc0 cache policy.
#define QUAD(DT, MF, G)                                                                    \
    Variant {                                                                              \
        DT, 0, 0, tgemm_config{TGEMM_KERNEL_QUAD, 256, 256, 64, 2, 2, 5, G, 1, MF},        \
            &launch_quad<DT, MF, (MF == 16 ? 2 : 1), (MF == 16 ? 56 : 40),                 \
                         (MF == 16 ? 40 : 12), 1, 2>                                       \
    }
// The quad kernel for B [K,N] (transposing B reads), with the schedules above.
#define QUAD_KN(DT, MF, G)                                                                 \
    Variant {                                                                              \
        DT, 0, 1, tgemm_config{TGEMM_KERNEL_QUAD, 256, 256, 64, 2, 2, 5, G, 1, MF},        \
            &launch_quad<DT, MF, (MF == 16 ? 2 : 1), (MF == 16 ? 56 : 40),                 \
                         (MF == 16 ? 40 : 12), 1, 2, 1>                                    \
    }
// The quad kernel with 192-row tiles (waves of 96 x 128), either B storage L: for grids
// that 256 x 256 tiles would leave short of the 256 compute units.
#define QUAD192(DT, MF, L, G)                                                              \
    Variant {                                                                              \
        DT, 0, L, tgemm_config{TGEMM_KERNEL_QUAD, 192, 256, 64, 2, 2, 5, G, 1, MF},        \
            &launch_quad<DT, MF, (MF == 16 ? 2 : 1), (MF == 16 ? 56 : 40),                 \
                         (MF == 16 ? 40 : 12), 1, 2, L, 192>                               \
    }
// The quad kernel for A stored [K,M] (transposing A reads), either B storage L.
#define QUAD_KM(DT, MF, L, G)                                                              \
    Variant {                                                                              \
        DT, 1, L, tgemm_config{TGEMM_KERNEL_QUAD, 256, 256, 64, 2, 2, 5, G, 1, MF},        \
            &launch_quad<DT, MF, (MF == 16 ? 2 : 1), (MF == 16 ? 56 : 40),                 \
                         (MF == 16 ? 40 : 12), 1, 2, L, 256, 1>                            \
    }
// Split-K over workgroups (registry entries carry split_k = 2; a call gives its own count).
#define SPLITK(DT, BM, BN, BK, WM, WN, ST, G)                                              \
    Variant {                                                                              \
        DT, 0, 0, tgemm_config{TGEMM_KERNEL_SPLITK, BM, BN, BK, WM, WN, ST, G, 2, 32},         \
            nullptr, &launch_splitk<DT, BM, BN, BK, WM, WN, ST>                            \
    }
// The quad kernel in split-K mode, either B storage L, with the schedules of QUAD.
#define QUAD_SPLIT(DT, MF, L, G)                                                           \
    Variant {                                                                              \
        DT, 0, L, tgemm_config{TGEMM_KERNEL_QUAD_SPLITK, 256, 256, 64, 2, 2, 5, G, 2, MF}, \
            nullptr,                                                                       \
            &launch_quad_split<DT, MF, (MF == 16 ? 2 : 1), (MF == 16 ? 56 : 40),           \
                               (MF == 16 ? 40 : 12), 1, 2, L>                              \
    }
// Stream-K over the last partial wave with the quad kernel, either B storage L.
#define QUAD_SK(DT, MF, L, G)                                                              \
    Variant {                                                                              \
        DT, 0, L, tgemm_config{TGEMM_KERNEL_QUAD_STREAMK, 256, 256, 64, 2, 2, 5, G, 1, MF},\
            nullptr,                                                                       \
            &launch_quad_sk<DT, MF, (MF == 16 ? 2 : 1), (MF == 16 ? 56 : 40),              \
                            (MF == 16 ? 40 : 12), 1, 2, L>                                 \
    }
#define SKINNY(DT, MT, D)                                                                  \
    Variant {                                                                              \
        DT, 0, 0, tgemm_config{TGEMM_KERNEL_SKINNY, MT * 32, 32, 64, 1, 8, D, 1, 8, 32},       \
            &launch_skinny<DT, MT, D>                                                      \
    }
// The skinny kernel with 128-wide k chunks (block_k 128): 256-byte row segments per load;
// 64-row blocks with four waves (waves_n and split_k 4).
#define SKINNY_WIDE(DT, MT, D)                                                             \
    Variant {                                                                              \
        DT, 0, 0, tgemm_config{TGEMM_KERNEL_SKINNY, MT * 32, 32, 128, 1, 8, D, 1, 8, 32},      \
            &launch_skinny<DT, MT, D, 128>                                                 \
    }
// The skinny kernel for B [K,N] (64-wide k chunks, transposing B reads).
#define SKINNY_KN(DT, MT, D)                                                               \
    Variant {                                                                              \
        DT, 0, 1, tgemm_config{TGEMM_KERNEL_SKINNY, MT * 32, 32, 64, 1, 8, D, 1, 8, 32},       \
            &launch_skinny_kn<DT, MT, D>                                                   \
    }
#define SKINNY_WIDE4(DT, MT, D)                                                            \
    Variant {                                                                              \
        DT, 0, 0, tgemm_config{TGEMM_KERNEL_SKINNY, MT * 32, 32, 128, 1, 4, D, 1, 4, 32},      \
            &launch_skinny<DT, MT, D, 128, 4>                                              \
    }
// The skinny kernel with 64 columns per workgroup (two 32-column blocks): half the
// workgroups of the 32-column form, each reading A once for twice the columns.
#define SKINNY_N64(DT, MT, CK, NW, D)                                                      \
    Variant {                                                                              \
        DT, 0, 0, tgemm_config{TGEMM_KERNEL_SKINNY, MT * 32, 64, CK, 1, NW, D, 1, NW, 32},     \
            &launch_skinny<DT, MT, D, CK, NW, 2>                                           \
    }
}  // namespace tgemm_reg
