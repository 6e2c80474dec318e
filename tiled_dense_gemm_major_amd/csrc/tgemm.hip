// libtgemm: the C ABI, argument checks, the compiled-configuration registry, the
// per-shape configuration table and the launches.  Declarations and conventions are in
// include/tgemm.h.
#include "tgemm.h"

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kernels.hpp"

namespace {

using tgemm::u16;

constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;
constexpr int kLdsBytes = 160 * 1024;

typedef hipError_t (*launch_fn)(const void* A, const void* B, void* C, int M, int N, int K,
                                int group_m, hipStream_t s);

struct Variant {
    int dtype;
    int layout;
    tgemm_config cfg;
    launch_fn launch;
};

int cdiv(int a, int b) { return (a + b - 1) / b; }

template <int DT, int LAYOUT, int BM, int BN, int BK, int WM, int WN>
hipError_t launch_tiled(const void* A, const void* B, void* C, int M, int N, int K,
                        int group_m, hipStream_t s) {
    const int gm = cdiv(M, BM), gn = cdiv(N, BN);
    hipLaunchKernelGGL((tgemm::gemm_tiled<DT, LAYOUT, BM, BN, BK, WM, WN>),
                       dim3((unsigned)(gm * gn)), dim3(WM * WN * 64), 0, s,
                       static_cast<const u16*>(A), static_cast<const u16*>(B),
                       static_cast<u16*>(C), M, N, K, gm, gn, group_m);
    return hipGetLastError();
}

template <int DT, int BM, int BN, int BK, int WM, int WN, int STAGES>
hipError_t launch_dma(const void* A, const void* B, void* C, int M, int N, int K, int group_m,
                      hipStream_t s) {
    const int gm = cdiv(M, BM), gn = cdiv(N, BN);
    hipLaunchKernelGGL((tgemm::gemm_dma<DT, BM, BN, BK, WM, WN, STAGES>),
                       dim3((unsigned)(gm * gn)), dim3(WM * WN * 64), 0, s,
                       static_cast<const u16*>(A), static_cast<const u16*>(B),
                       static_cast<u16*>(C), M, N, K, gm, gn, group_m);
    return hipGetLastError();
}

template <int DT, int LAYOUT, int BM, int BN, int BK, int S>
hipError_t launch_pingpong(const void* A, const void* B, void* C, int M, int N, int K,
                           int group_m, hipStream_t s) {
    const int gm = cdiv(M, BM), gn = cdiv(N, BN);
    hipLaunchKernelGGL((tgemm::gemm_pingpong<DT, LAYOUT, BM, BN, BK, S>), dim3((unsigned)(gm * gn)),
                       dim3(512), 0, s, static_cast<const u16*>(A), static_cast<const u16*>(B),
                       static_cast<u16*>(C), M, N, K, gm, gn, group_m);
    return hipGetLastError();
}

template <int DT, int MT, int D>
hipError_t launch_skinny(const void* A, const void* B, void* C, int M, int N, int K, int,
                         hipStream_t s) {
    hipLaunchKernelGGL((tgemm::gemm_skinny<DT, MT, D>),
                       dim3((unsigned)cdiv(N, 32), (unsigned)cdiv(M, MT * 32)), dim3(512), 0, s,
                       static_cast<const u16*>(A), static_cast<const u16*>(B),
                       static_cast<u16*>(C), M, N, K);
    return hipGetLastError();
}

template <int DT, int LAYOUT>
hipError_t launch_generic(const void* A, const void* B, void* C, int M, int N, int K,
                          int group_m, hipStream_t s) {
    const int gm = cdiv(M, 64), gn = cdiv(N, 64);
    hipLaunchKernelGGL((tgemm::gemm_generic<DT, LAYOUT>), dim3((unsigned)(gm * gn)), dim3(256),
                       0, s, static_cast<const u16*>(A), static_cast<const u16*>(B),
                       static_cast<u16*>(C), M, N, K, gm, gn, group_m);
    return hipGetLastError();
}

#define TILED(DT, L, BM, BN, BK, WM, WN, G)                                               \
    Variant {                                                                              \
        DT, L, tgemm_config{TGEMM_KERNEL_TILED, BM, BN, BK, WM, WN, 2, G, 1},              \
            &launch_tiled<DT, L, BM, BN, BK, WM, WN>                                       \
    }
#define GENERIC(DT, L)                                                                     \
    Variant {                                                                              \
        DT, L, tgemm_config{TGEMM_KERNEL_GENERIC, 64, 64, 16, 2, 2, 1, 8, 1},              \
            &launch_generic<DT, L>                                                         \
    }
#define DMA(DT, BM, BN, BK, WM, WN, ST, G)                                                 \
    Variant {                                                                              \
        DT, 0, tgemm_config{TGEMM_KERNEL_DMA, BM, BN, BK, WM, WN, ST, G, 1},               \
            &launch_dma<DT, BM, BN, BK, WM, WN, ST>                                        \
    }
#define PINGPONG(DT, L, BM, BN, BK, S, G)                                                  \
    Variant {                                                                              \
        DT, L, tgemm_config{TGEMM_KERNEL_PINGPONG, BM, BN, BK, 2, 4, S, G, 1},             \
            &launch_pingpong<DT, L, BM, BN, BK, S>                                         \
    }
#define SKINNY(DT, MT, D)                                                                  \
    Variant {                                                                              \
        DT, 0, tgemm_config{TGEMM_KERNEL_SKINNY, MT * 32, 32, 64, 1, 8, D, 1, 8},          \
            &launch_skinny<DT, MT, D>                                                      \
    }
#define ALL_DMA(DT)                                                                        \
    DMA(DT, 256, 256, 32, 2, 2, 4, 4), DMA(DT, 256, 256, 32, 2, 2, 5, 4),                  \
        PINGPONG(DT, 0, 256, 256, 64, 2, 4), PINGPONG(DT, 0, 256, 256, 32, 4, 4), \
        PINGPONG(DT, 0, 256, 256, 32, 5, 4), SKINNY(DT, 1, 4), SKINNY(DT, 2, 3), SKINNY(DT, 4, 1)
#define ALL_SHAPES(DT, L)                                                                  \
    GENERIC(DT, L), TILED(DT, L, 256, 256, 64, 2, 2, 4), TILED(DT, L, 128, 128, 64, 2, 2, 8), \
        TILED(DT, L, 64, 64, 64, 2, 2, 8)

const Variant kVariants[] = {
    ALL_DMA(0),
    ALL_DMA(1),
    ALL_SHAPES(0, 0),
    ALL_SHAPES(0, 1),
    PINGPONG(0, 1, 256, 256, 64, 2, 4),
    PINGPONG(1, 1, 256, 256, 64, 2, 4),
    PINGPONG(0, 1, 256, 256, 32, 5, 4),
    PINGPONG(1, 1, 256, 256, 32, 5, 4),
    ALL_SHAPES(1, 0),
    ALL_SHAPES(1, 1),
};
constexpr int kNumVariants = (int)(sizeof(kVariants) / sizeof(kVariants[0]));

bool same_shape(const tgemm_config& a, const tgemm_config& b) {
    return a.kernel == b.kernel && a.block_m == b.block_m && a.block_n == b.block_n &&
           a.block_k == b.block_k && a.waves_m == b.waves_m && a.waves_n == b.waves_n &&
           a.stages == b.stages && a.split_k == b.split_k;
}

const Variant* find_variant(int dtype, int layout, const tgemm_config& cfg) {
    for (int i = 0; i < kNumVariants; ++i) {
        const Variant& v = kVariants[i];
        if (v.dtype == dtype && v.layout == layout && same_shape(v.cfg, cfg))
            return &v;
    }
    return nullptr;
}

// The table: fast configurations by how many workgroups they give, so that the chip
// (256 compute units) is filled with the largest tile that still fills it.
tgemm_config choose(int dtype, int layout, int64_t m, int64_t n, int64_t k, bool aligned) {
    (void)dtype;
    tgemm_config c;
    if (!aligned) {
        c = tgemm_config{TGEMM_KERNEL_GENERIC, 64, 64, 16, 2, 2, 1, 8, 1};
        return c;
    }
    if (layout == TGEMM_B_NK && m <= 128 && k >= 1024) {
        const int mt = m <= 32 ? 1 : (m <= 64 ? 2 : 4);
        const int depth = mt == 1 ? 4 : (mt == 2 ? 3 : 1);
        return tgemm_config{TGEMM_KERNEL_SKINNY, mt * 32, 32, 64, 1, 8, depth, 1, 8};
    }
    const int64_t t256 = ((m + 255) / 256) * ((n + 255) / 256);
    const int64_t t128 = ((m + 127) / 128) * ((n + 127) / 128);
    if (t256 >= 192)
        return tgemm_config{TGEMM_KERNEL_PINGPONG, 256, 256, 64, 2, 4, 2, 4, 1};
    if (t128 >= 128)
        return tgemm_config{TGEMM_KERNEL_TILED, 128, 128, 64, 2, 2, 2, 8, 1};
    return tgemm_config{TGEMM_KERNEL_TILED, 64, 64, 64, 2, 2, 2, 8, 1};
}

int check_problem(int dtype, int64_t m, int64_t n, int64_t k, int b_layout) {
    if (dtype != TGEMM_F16 && dtype != TGEMM_BF16)
        return TGEMM_ERR_INVALID_VALUE;
    if (b_layout != TGEMM_B_NK && b_layout != TGEMM_B_KN)
        return TGEMM_ERR_INVALID_VALUE;
    if (m < 0 || n < 0 || k < 0)
        return TGEMM_ERR_INVALID_VALUE;
    if (m > kMaxElems || n > kMaxElems || k > kMaxElems)
        return TGEMM_ERR_UNSUPPORTED;
    if ((k > 0 && (m > kMaxElems / k || n > kMaxElems / k)) || (n > 0 && m > kMaxElems / n))
        return TGEMM_ERR_UNSUPPORTED;
    return TGEMM_OK;
}

bool overlaps(const void* p, int64_t pbytes, const void* q, int64_t qbytes) {
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return pbytes > 0 && qbytes > 0 && a < b + (uintptr_t)qbytes && b < a + (uintptr_t)pbytes;
}

// The fast kernels read A and B through buffer resources whose range check rejects any
// offset with bit 31 set, which holds only for operands of at most 2^31 bytes.
constexpr int64_t kMaxFastOperandBytes = int64_t(1) << 31;

bool fast_aligned(int64_t m, int64_t n, int64_t k, const void* A, const void* B,
                  const void* C) {
    return k % 8 == 0 && n % 8 == 0 && ((uintptr_t)A % 16) == 0 && ((uintptr_t)B % 16) == 0 &&
           ((uintptr_t)C % 16) == 0 && 2 * m * k <= kMaxFastOperandBytes &&
           2 * n * k <= kMaxFastOperandBytes;
}

int run(int dtype, int64_t m, int64_t n, int64_t k, const void* A, const void* B, void* C,
        int b_layout, const tgemm_config* cfg, void* stream) {
    int rc = check_problem(dtype, m, n, k, b_layout);
    if (rc != TGEMM_OK)
        return rc;
    if (m == 0 || n == 0)
        return TGEMM_OK;
    if (!C || (k > 0 && (!A || !B)))
        return TGEMM_ERR_NULL_POINTER;
    if (((uintptr_t)C & 1) || ((uintptr_t)A & 1) || ((uintptr_t)B & 1))
        return TGEMM_ERR_ALIGNMENT;
    if (overlaps(C, 2 * m * n, A, 2 * m * k) || overlaps(C, 2 * m * n, B, 2 * n * k))
        return TGEMM_ERR_ALIASING;
    const bool aligned = fast_aligned(m, n, k, A, B, C);
    tgemm_config use = cfg ? *cfg : choose(dtype, b_layout, m, n, k, aligned);
    const Variant* v = find_variant(dtype, b_layout, use);
    if (!v)
        return TGEMM_ERR_UNSUPPORTED;
    if (use.kernel != TGEMM_KERNEL_GENERIC && !aligned)
        return TGEMM_ERR_ALIGNMENT;
    const int group_m = use.group_m > 0 ? use.group_m : v->cfg.group_m;
    (void)hipGetLastError();   // start from a clean error state for this launch
    const hipError_t e = v->launch(A, B, C, (int)m, (int)n, (int)k, group_m,
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TGEMM_OK : TGEMM_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int gemm_f16(int64_t m, int64_t n, int64_t k, const void* A, const void* B, void* C,
             int b_layout, void* stream) {
    return run(TGEMM_F16, m, n, k, A, B, C, b_layout, nullptr, stream);
}

int gemm_bf16(int64_t m, int64_t n, int64_t k, const void* A, const void* B, void* C,
              int b_layout, void* stream) {
    return run(TGEMM_BF16, m, n, k, A, B, C, b_layout, nullptr, stream);
}

int gemm_ex(int dtype, int64_t m, int64_t n, int64_t k, const void* A, const void* B, void* C,
            int b_layout, const tgemm_config* cfg, void* stream) {
    return run(dtype, m, n, k, A, B, C, b_layout, cfg, stream);
}

int tgemm_query_config(int dtype, int64_t m, int64_t n, int64_t k, int b_layout, int aligned,
                       tgemm_config* out) {
    int rc = check_problem(dtype, m, n, k, b_layout);
    if (rc != TGEMM_OK)
        return rc;
    if (!out)
        return TGEMM_ERR_NULL_POINTER;
    *out = choose(dtype, b_layout, m, n, k, aligned != 0);
    const Variant* v = find_variant(dtype, b_layout, *out);
    if (v)
        out->group_m = v->cfg.group_m;
    return TGEMM_OK;
}

int tgemm_list_configs(int dtype, int b_layout, tgemm_config* out, int capacity) {
    if (dtype != TGEMM_F16 && dtype != TGEMM_BF16)
        return TGEMM_ERR_INVALID_VALUE;
    if (b_layout != TGEMM_B_NK && b_layout != TGEMM_B_KN)
        return TGEMM_ERR_INVALID_VALUE;
    if (capacity < 0 || (capacity > 0 && !out))
        return TGEMM_ERR_INVALID_VALUE;
    int count = 0;
    for (int i = 0; i < kNumVariants; ++i) {
        const Variant& v = kVariants[i];
        if (v.dtype != dtype || v.layout != b_layout)
            continue;
        if (count < capacity)
            out[count] = v.cfg;
        ++count;
    }
    return count;
}

const char* tgemm_status_string(int status) {
    switch (status) {
    case TGEMM_OK: return "TGEMM_OK";
    case TGEMM_ERR_INVALID_VALUE: return "TGEMM_ERR_INVALID_VALUE: bad size, dtype or layout";
    case TGEMM_ERR_NULL_POINTER: return "TGEMM_ERR_NULL_POINTER: NULL operand";
    case TGEMM_ERR_ALIGNMENT: return "TGEMM_ERR_ALIGNMENT: operand alignment not supported";
    case TGEMM_ERR_ALIASING: return "TGEMM_ERR_ALIASING: C overlaps A or B";
    case TGEMM_ERR_UNSUPPORTED: return "TGEMM_ERR_UNSUPPORTED: size or configuration not supported";
    case TGEMM_ERR_LAUNCH: return "TGEMM_ERR_LAUNCH: kernel launch failed";
    case TGEMM_ERR_DEVICE: return "TGEMM_ERR_DEVICE: device query failed";
    default: return "unknown tgemm status";
    }
}

int tgemm_version(void) { return 100; }

}  // extern "C"
