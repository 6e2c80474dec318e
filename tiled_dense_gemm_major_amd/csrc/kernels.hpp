// gfx950 kernels of libtgemm: C[M,N] = sum_k A[M,K] * b(n,k), fp16/bf16 in, fp32 sums,
// one round-to-nearest-even cast to the 16-bit output.
//
// Block tiling ("0. A Minimal Hopper Matmul", section "Block Tiling"; "Tiling a matmul",
// sections "The idea in one minute" and "The levels of tiling"): a workgroup owns one
// BM x BN tile of C and walks K in steps of BK; each step stages an A tile [BM,BK] and a
// B tile [BN,BK] in LDS, every wavefront reads its rows and columns from there into
// MFMA operand registers, and the fp32 accumulators stay in (accumulation) registers
// until the epilogue casts and stores them.  The loads of the next steps overlap the
// matrix-core work of the current one (section "Pipelining" of the tiling page), and the
// tiles are launched in a grouped order so that neighbours share A rows and B columns
// in cache (section "The levels of tiling").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tgemm {

typedef uint16_t u16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

enum { DT_F16 = 0, DT_BF16 = 1 };
enum { LAYOUT_NK = 0, LAYOUT_KN = 1 };

// ------------------------------------------------------------------------------------
// Matrix-core step: D(32x32, fp32) += S0(32 x 16) * S1(16 x 32).  Lane l supplies, for
// both sources, the 8 consecutive-k values k = 8*(l/32) .. 8*(l/32)+7 of row (l % 32)
// of S0 and of column (l % 32) of S1.  Lane l receives D column (l % 32), rows
// 8*(v/4) + 4*(l/32) + (v%4) in element v of the 16-float result.
// ------------------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 s0, u32x4 s1, f32x16 acc) {
    if constexpr (DT == DT_F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, s0),
                                                      __builtin_bit_cast(f16x8, s1), acc, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, s0),
                                                       __builtin_bit_cast(bf16x8, s1), acc, 0, 0, 0);
}

// fp32 -> 16-bit output with round-to-nearest-even (the hardware conversions in the
// default rounding mode), two values packed low | high << 16.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    if constexpr (DT == DT_F16) {
        const _Float16 l = (_Float16)lo, h = (_Float16)hi;
        return (uint32_t)__builtin_bit_cast(u16, l) | ((uint32_t)__builtin_bit_cast(u16, h) << 16);
    } else {
        const __bf16 l = (__bf16)lo, h = (__bf16)hi;
        return (uint32_t)__builtin_bit_cast(u16, l) | ((uint32_t)__builtin_bit_cast(u16, h) << 16);
    }
}

template <int DT>
__device__ __forceinline__ u16 cvt1(float x) {
    if constexpr (DT == DT_F16)
        return __builtin_bit_cast(u16, (_Float16)x);
    else
        return __builtin_bit_cast(u16, (__bf16)x);
}

// ------------------------------------------------------------------------------------
// Launch order.  Workgroup ids are handed to the 8 XCDs (each with its own L2) in turn:
// id w runs on XCD w % 8.  The ids are first renumbered so that each XCD receives one
// contiguous range of logical tiles, then the logical index walks the tiles in groups of
// group_m tile-rows, column by column inside a group, so the workgroups one XCD runs at
// the same time cover a compact block of C and share its A rows and B columns in L2.
// ------------------------------------------------------------------------------------
__device__ __forceinline__ void tile_of(int wg, int grid_m, int grid_n, int group_m, int& tm,
                                        int& tn) {
    const int nwg = grid_m * grid_n;
    const int per_xcd = nwg >> 3, extra = nwg & 7;
    const int xcd = wg & 7, slot = wg >> 3;
    const int L = xcd * per_xcd + (xcd < extra ? xcd : extra) + slot;
    const int per_group = group_m * grid_n;
    const int g = L / per_group;
    const int first_m = g * group_m;
    const int rows = (grid_m - first_m) < group_m ? (grid_m - first_m) : group_m;
    const int within = L - g * per_group;
    tm = first_m + within % rows;
    tn = within / rows;
}

// LDS swizzle.  A tile row holds KC 16-byte chunks.  Chunk c of row r is stored at chunk
// c ^ swz(r), so the 8 rows read by 8 neighbouring lanes (one 128-byte bank sweep) land
// in 8 different 16-byte bank groups, for both the 128-bit writes and the 128-bit reads.
template <int KC>
__device__ __forceinline__ int swz(int row) {
    if constexpr (KC >= 8)
        return row & 7;
    else
        return (row / (8 / KC)) & (KC - 1);
}

__device__ __forceinline__ void block_sync_lds() {
    // Wait for this wave's LDS traffic, then meet the other waves.  Outstanding global
    // loads into registers are deliberately not waited for (they are the prefetch).
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ------------------------------------------------------------------------------------
// Buffer loads.  A buffer resource covers one operand ([rows x K] or [K x N] halves);
// the hardware checks each lane's VGPR offset against its size and returns zeros,
// without touching memory, for offsets at or past the end.  The SGPR offset (used for
// the K position) is not part of that check.
// ------------------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw 32-bit data format, gfx9 family
constexpr uint32_t kOutOfRange = 0x80000000u;  // OR-ed into an offset: past any operand

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes,
                                             (int)kRsrcWord3);
}

__device__ __forceinline__ u32x4 load16(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// ------------------------------------------------------------------------------------
// The tiled kernel.
//   Template: DT (fp16/bf16), LAYOUT (B as [N,K] or [K,N]), BM x BN x BK tile, WM x WN
//   waves (each owns a (BM/WM) x (BN/WN) block of the tile, in 32 x 32 MFMA blocks).
//   Host-checked requirements: K % 8 == 0, N % 8 == 0, 16-byte aligned A, B, C, and
//   A and B each at most 2^31 bytes (so an offset with the top bit set is out of range).
//   Edges: rows of A past M and of B past N read as zero through the buffer range check
//   (their results fall outside C and are not stored anyway); chunks with k >= K get an
//   out-of-range offset and read as zero; stores outside [M,N] are skipped.
// Pipeline: two LDS stages plus one register stage.  While the MFMAs run on the tile in
// stage t%2, tile t+1 (already in registers) is written to the other stage and the
// global loads of tile t+2 are issued, so every global load has a whole step to arrive.
// ------------------------------------------------------------------------------------
template <int DT, int LAYOUT, int BM, int BN, int BK, int WM, int WN>
__global__ void __attribute__((amdgpu_flat_work_group_size(WM * WN * 64, WM * WN * 64),
                               amdgpu_waves_per_eu(1, 1)))
gemm_tiled(const u16* __restrict__ A, const u16* __restrict__ B, u16* __restrict__ C, int M,
           int N, int K, int grid_m, int grid_n, int group_m) {
    constexpr int NT = WM * WN * 64;
    constexpr int KC = BK / 8;              // 16-byte chunks in one tile row
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int KS = BK / 16;             // MFMA k-steps per tile
    constexpr int A_ELEMS = BM * BK;
    constexpr int STAGE = (BM + BN) * BK;   // elements of one LDS stage (A then B)
    constexpr int RS = NT / KC;             // rows between the chunks one thread loads
    constexpr int A_LD = BM / RS;           // A chunks per thread
    constexpr int B_LD = (LAYOUT == LAYOUT_NK) ? BN / RS : 1;
    // [K,N] B: a thread loads 8x8 blocks (8 k-rows of 8 n); KN_BLK blocks per tile.
    constexpr int KN_BLK = KC * (BN / 8);
    constexpr int KN_LD = (KN_BLK + NT - 1) / NT;
    constexpr int B_REGS = (LAYOUT == LAYOUT_NK) ? B_LD : 8 * KN_LD;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(BK % 16 == 0 && NT % KC == 0 && RS % 8 == 0, "bad BK");
    static_assert(BM % RS == 0 && (LAYOUT == LAYOUT_KN || BN % RS == 0), "bad load split");

    __shared__ __attribute__((aligned(16))) u16 lds[2 * STAGE];

    int tm, tn;
    tile_of((int)blockIdx.x, grid_m, grid_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    const rsrc_t ra = make_rsrc(A, (uint32_t)M * (uint32_t)K * 2u);
    const rsrc_t rb = make_rsrc(B, (uint32_t)N * (uint32_t)K * 2u);

    // ---- global -> register addressing (byte offsets; K position goes in soffset) ----
    const int lc = tid % KC;                 // this thread's chunk column (row-major loads)
    const int lr = tid / KC;                 // its first row; the others follow every RS
    // Every offset that must not be read carries kOutOfRange, OR-ed in after all
    // additions, so the range check rejects it whatever the SGPR offset adds.
    uint32_t a_off[A_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int r = m0 + lr + i * RS;
        a_off[i] = r < M ? (uint32_t)(r * K + lc * 8) * 2u : kOutOfRange;
    }
    // The LDS slot of chunk (row, lc): rows lr + i*RS share one swizzle (RS % 8 == 0).
    const int a_lds = lr * BK + ((lc ^ swz<KC>(lr)) * 8);

    uint32_t b_off[LAYOUT == LAYOUT_NK ? B_LD : KN_LD];
    int b_lds = 0, kn_kb = 0, kn_nb = 0;
    if constexpr (LAYOUT == LAYOUT_NK) {
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int r = n0 + lr + i * RS;
            b_off[i] = r < N ? (uint32_t)(r * K + lc * 8) * 2u : kOutOfRange;
        }
        b_lds = A_ELEMS + lr * BK + ((lc ^ swz<KC>(lr)) * 8);
    } else {
        static_assert(LAYOUT == LAYOUT_NK || KN_LD == 1, "one 8x8 block per thread");
        kn_kb = tid % KC;
        kn_nb = tid / KC;
        // Offset of row k = 8*kb (the K position goes in soffset); only meaningful for
        // a live block whose 8 columns are inside [0, N) (N % 8 == 0).
        b_off[0] = ((uint32_t)(kn_kb * 8) * (uint32_t)N + (uint32_t)(n0 + kn_nb * 8)) * 2u;
        b_lds = A_ELEMS + (kn_nb * 8) * BK;
    }
    const bool kn_live = ((KN_BLK % NT == 0) || (tid < KN_BLK)) && (n0 + kn_nb * 8 < N);

    u32x4 a_reg[A_LD];
    u32x4 b_reg[B_REGS];

    auto gload = [&](int kt) {
        const int k0 = kt * BK;
        const uint32_t kbad = (k0 + lc * 8 < K) ? 0u : kOutOfRange;
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            a_reg[i] = load16(ra, a_off[i] | kbad, (uint32_t)k0 * 2u);
        if constexpr (LAYOUT == LAYOUT_NK) {
#pragma unroll
            for (int i = 0; i < B_LD; ++i)
                b_reg[i] = load16(rb, b_off[i] | kbad, (uint32_t)k0 * 2u);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bool ok = kn_live && (k0 + kn_kb * 8 + j < K);
                b_reg[j] = load16(rb, (b_off[0] + (uint32_t)j * (uint32_t)N * 2u) | (ok ? 0u : kOutOfRange),
                                  (uint32_t)k0 * (uint32_t)N * 2u);
            }
        }
    };

    auto swrite = [&](u16* st) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            *reinterpret_cast<u32x4*>(st + a_lds + i * RS * BK) = a_reg[i];
        if constexpr (LAYOUT == LAYOUT_NK) {
#pragma unroll
            for (int i = 0; i < B_LD; ++i)
                *reinterpret_cast<u32x4*>(st + b_lds + i * RS * BK) = b_reg[i];
        } else {
            {
                // 8x8 transpose (a dead block holds zeros and lands in rows never stored): b_reg[j] holds n = 0..7 at k = j; row n gets k = 0..7.
#pragma unroll
                for (int n = 0; n < 8; ++n) {
                    const int p = n >> 1;
                    const uint32_t sel = (n & 1) ? 0x07060302u : 0x05040100u;
                    u32x4 o;
                    o[0] = __builtin_amdgcn_perm(b_reg[1][p], b_reg[0][p], sel);
                    o[1] = __builtin_amdgcn_perm(b_reg[3][p], b_reg[2][p], sel);
                    o[2] = __builtin_amdgcn_perm(b_reg[5][p], b_reg[4][p], sel);
                    o[3] = __builtin_amdgcn_perm(b_reg[7][p], b_reg[6][p], sel);
                    *reinterpret_cast<u32x4*>(st + b_lds + n * BK +
                                              ((kn_kb ^ swz<KC>(kn_nb * 8 + n)) * 8)) = o;
                }
            }
        }
    };

    // ---- LDS -> MFMA operands ---------------------------------------------------------
    const int xr = swz<KC>(lane & 31);       // swizzle of this lane's rows (bases are x8)
    const int half = lane >> 5;               // which 8 of the 16 k of an MFMA step
    const int a_row0 = (wm * WTM + (lane & 31)) * BK;
    const int b_row0 = A_ELEMS + (wn * WTN + (lane & 31)) * BK;

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

    auto compute = [&](const u16* st) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int koff = (((2 * s) | half) ^ xr) * 8;
            u32x4 af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = *reinterpret_cast<const u32x4*>(st + a_row0 + i * 32 * BK + koff);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bf[j] = *reinterpret_cast<const u32x4*>(st + b_row0 + j * 32 * BK + koff);
            // S0 = B rows (n), S1 = A rows (m): lane l then holds C row m = l % 32 and
            // four consecutive columns n per group of four results.
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = mfma_32x32x16<DT>(bf[j], af[i], acc[i][j]);
        }
    };

    const int nk = (K + BK - 1) / BK;
    if (nk > 0) {
        gload(0);
        swrite(lds);
        if (nk > 1)
            gload(1);
        block_sync_lds();
        for (int kt = 0; kt < nk; ++kt) {
            u16* cur = lds + (kt & 1) * STAGE;
            u16* nxt = lds + ((kt & 1) ^ 1) * STAGE;
            compute(cur);
            if (kt + 1 < nk) {
                swrite(nxt);
                if (kt + 2 < nk)
                    gload(kt + 2);
            }
            block_sync_lds();
        }
    }

    // ---- epilogue: cast once, store 4 consecutive columns (8 bytes) per group ----------
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int m = m0 + wm * WTM + i * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * WTN + j * 32 + 8 * g + 4 * half;
                u32x2 v;
                v[0] = pack2<DT>(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
                v[1] = pack2<DT>(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
                if (m < M && n < N)
                    *reinterpret_cast<u32x2*>(C + (size_t)m * N + n) = v;
            }
        }
    }
}

// ------------------------------------------------------------------------------------
// The generic kernel: any alignment, any M, N, K.  64 x 64 tile, K step 16, 4 waves each
// owning one 32 x 32 MFMA block; element-by-element masked loads into one LDS stage.
// ------------------------------------------------------------------------------------
template <int DT, int LAYOUT>
__global__ void __launch_bounds__(256)
gemm_generic(const u16* __restrict__ A, const u16* __restrict__ B, u16* __restrict__ C, int M,
             int N, int K, int grid_m, int grid_n, int group_m) {
    __shared__ __attribute__((aligned(16))) u16 As[64 * 16];
    __shared__ __attribute__((aligned(16))) u16 Bs[64 * 16];
    int tm, tn;
    tile_of((int)blockIdx.x, grid_m, grid_n, group_m, tm, tn);
    const int m0 = tm * 64, n0 = tn * 64;
    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    f32x16 acc = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + 256 * i;
            {   // A: consecutive threads walk k (contiguous in memory)
                const int r = e >> 4, kk = e & 15;
                const int gm = m0 + r, gk = k0 + kk;
                As[r * 16 + kk] = (gm < M && gk < K) ? A[(size_t)gm * K + gk] : (u16)0;
            }
            if constexpr (LAYOUT == LAYOUT_NK) {
                const int r = e >> 4, kk = e & 15;
                const int gn = n0 + r, gk = k0 + kk;
                Bs[r * 16 + kk] = (gn < N && gk < K) ? B[(size_t)gn * K + gk] : (u16)0;
            } else {   // consecutive threads walk n (contiguous in memory)
                const int r = e & 63, kk = e >> 6;
                const int gn = n0 + r, gk = k0 + kk;
                Bs[r * 16 + kk] = (gn < N && gk < K) ? B[(size_t)gk * N + gn] : (u16)0;
            }
        }
        __syncthreads();
        const u32x4 af = *reinterpret_cast<const u32x4*>(&As[(wm * 32 + (lane & 31)) * 16 + (lane >> 5) * 8]);
        const u32x4 bf = *reinterpret_cast<const u32x4*>(&Bs[(wn * 32 + (lane & 31)) * 16 + (lane >> 5) * 8]);
        acc = mfma_32x32x16<DT>(bf, af, acc);
        __syncthreads();
    }
    const int m = m0 + wm * 32 + (lane & 31);
    if (m < M) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int n = n0 + wn * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (n < N)
                C[(size_t)m * N + n] = cvt1<DT>(acc[v]);
        }
    }
}

}  // namespace tgemm
