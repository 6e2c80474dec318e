// The direct kernel of libtgemm: products with few output tiles and a short K walk
// (A [M,K], B [N,K]).
//
// A small product is latency-bound rather than bound by the matrix cores or HBM ("Tiling
// a matmul", section "Where it breaks": small shapes leave compute units idle, and split-K
// gives them work).  Here each workgroup owns a 32 x 32 tile of C (a 512 x 512 C gives
// 256 workgroups, one per compute unit) and its four waves split the tile's K range: wave
// w takes the w-th quarter of its 16-wide k blocks (consecutive blocks, so a wave's
// consecutive loads complete whole cache lines).  A lane's MFMA operands are loaded
// straight from global memory into registers, with no LDS staging: for the 32x32x16
// MFMA, lane l holds 8 consecutive k (8 * (l / 32) .. +7) of row l % 32 of A and of B,
// one 16-byte buffer load per operand per k block.  Loads go out in batches of G blocks,
// the next batch while the current one is multiplied, so a wave with at most G blocks
// waits for one memory round trip.  Rows past M or N and k blocks past K read as zeros
// (out-of-range offsets).  The four partial tiles are added in LDS in wave order (a fixed
// order: every launch gives the same bits); each wave adds, casts and stores a quarter of
// the tile.
#pragma once

#include "kernels.hpp"

namespace tgemm {

template <int DT, int G>
__global__ void __launch_bounds__(256)
gemm_direct(const u16* __restrict__ A, const u16* __restrict__ B, u16* __restrict__ C, int M,
            int N, int K, int lda, int ldb, int ldc, int grid_m, int grid_n, int group_m) {
    __shared__ f32x4 part[4][4][64];           // the partial tiles, [wave][quarter][lane]
    int tm, tn;
    tile_of((int)blockIdx.x, grid_m, grid_n, group_m, tm, tn);
    const int m0 = tm * 32, n0 = tn * 32;
    const int lane = (int)threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const rsrc_t ra = make_rsrc(A, span_bytes(M, K, lda));
    const rsrc_t rb = make_rsrc(B, span_bytes(N, K, ldb));
    const int r = lane & 31, kh = (lane >> 5) * 8;
    // the lane's row and k half as a byte offset; the k block goes in the scalar offset
    const uint32_t a_at = m0 + r < M ? (uint32_t)((m0 + r) * lda + kh) * 2u : kOutOfRange;
    const uint32_t b_at = n0 + r < N ? (uint32_t)((n0 + r) * ldb + kh) * 2u : kOutOfRange;
    const int nkb = (K + 15) / 16;             // 16-wide k blocks of the walk
    const int first = (nkb * wave) >> 2;       // this wave's blocks: [first, first + mine)
    const int mine = ((nkb * (wave + 1)) >> 2) - first;
    const int batches = (mine + G - 1) / G;

    u32x4 fa[2][G], fb[2][G];
    // batch j of this wave's blocks into buffer buf; a block's k half past K (K is a
    // multiple of 8) or a block past the wave's list reads zeros
    auto load = [&](auto bufc, int j) {
        constexpr int buf = decltype(bufc)::value;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int i = j * G + g;
            const int kb = first + i;
            const bool listed = i < mine;                  // the same for every lane
            const uint32_t soff = listed ? (uint32_t)kb * 32u : 0u;
            const bool live = listed && kb * 16 + kh < K;  // per lane (its k half)
            fa[buf][g] = load16(ra, live ? a_at : kOutOfRange, soff);
            fb[buf][g] = load16(rb, live ? b_at : kOutOfRange, soff);
        }
    };
    f32x16 acc = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    auto mul = [&](auto bufc) {
        constexpr int buf = decltype(bufc)::value;
#pragma unroll
        for (int g = 0; g < G; ++g)
            acc = mfma_32x32x16<DT>(fb[buf][g], fa[buf][g], acc);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // Pairs of batches with no branch inside (a branch there makes the compiler copy the
    // accumulators out of and back into their registers every pass); a batch past the
    // wave's list loads zeros without touching memory.
    load(I0{}, 0);
    int j = 0;
    for (; j + 2 <= batches; j += 2) {
        load(I1{}, j + 1);
        mul(I0{});
        load(I0{}, j + 2);
        mul(I1{});
    }
    if (j < batches)                           // an odd last batch, in buffer 0
        mul(I0{});

    // lane l holds C row m0 + l % 32 and, for element v, column
    // n0 + 8 (v / 4) + 4 (l / 32) + v % 4: four runs of 4 consecutive columns, the g-th
    // in elements 4g .. 4g + 3.  Wave w adds the four waves' run w in wave order.
#pragma unroll
    for (int g = 0; g < 4; ++g)
        part[wave][g][lane] = f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
    __syncthreads();
    f32x4 sum = part[0][wave][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w)
        sum += part[w][wave][lane];
    const int m = m0 + r;
    const int n = n0 + 8 * wave + 4 * (lane >> 5);
    u32x2 v;
    v[0] = pack2<DT>(sum[0], sum[1]);
    v[1] = pack2<DT>(sum[2], sum[3]);
    if (m < M && n < N)
        *reinterpret_cast<u32x2*>(C + (size_t)m * ldc + n) = v;
}

}  // namespace tgemm
