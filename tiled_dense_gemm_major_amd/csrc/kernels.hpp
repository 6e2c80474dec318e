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

#include <type_traits>
#include <utility>

namespace tgemm {

typedef uint16_t u16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

enum { DT_F16 = 0, DT_BF16 = 1 };
enum { LAYOUT_NK = 0, LAYOUT_KN = 1 };   // B stored [N,K] (K contiguous) or [K,N]
enum { LAYOUT_MK = 0, LAYOUT_KM = 1 };   // A stored [M,K] (K contiguous) or [K,M]

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

// Matrix-core step: D(16x16, fp32) += S0(16 x 32) * S1(32 x 16).  Lane l supplies, for
// both sources, 8 consecutive-k values k = 8*(l/16) .. 8*(l/16)+7 of row (l % 16) of S0
// and of column (l % 16) of S1 (the same k for both, whatever order the unit sums them
// in).  Lane l receives D column (l % 16), rows 4*(l/16) + v in element v of the result.
template <int DT>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 s0, u32x4 s1, f32x4 acc) {
    if constexpr (DT == DT_F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, s0),
                                                      __builtin_bit_cast(f16x8, s1), acc, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, s0),
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

// LDS swizzle.  A tile row holds KC 16-byte chunks.  The LDS serves a 128-bit access 16
// lanes at a time from a 256-byte window of banks, and neighbouring lanes read or write
// neighbouring tile rows at the same logical chunk.  Chunk c of row r is stored at chunk
// c ^ swz(r), where swz changes every R = 16/KC rows (the rows sharing one 256-byte
// window), so the 16 rows touched by 16 neighbouring lanes land in 16 different 16-byte
// bank groups: conflict-free 128-bit writes (row-major loads) and fragment reads.
template <int KC>
__device__ __forceinline__ int swz(int row) {
    constexpr int R = KC >= 16 ? 1 : 16 / KC;
    return (row / R) & (KC - 1);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
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

// Bytes spanned by an operand stored as `rows` rows of `cols` elements, `ld` elements
// apart (the host keeps this within 2^31).
__device__ __forceinline__ uint32_t span_bytes(int rows, int cols, int ld) {
    return rows > 0 && cols > 0 ? ((uint32_t)(rows - 1) * (uint32_t)ld + (uint32_t)cols) * 2u
                                : 0u;
}

__device__ __forceinline__ u32x4 load16(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// One 2-byte element, for operands with no alignment beyond the element's own; an
// offset of kOutOfRange reads zero.
__device__ __forceinline__ u16 load2(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

// Sixteen bytes starting `sh` bytes (even, 0..14) into the 32 bytes lo:hi (two aligned
// 16-byte blocks loaded back to back): a two-stage select of the five words from
// sh / 4 on, written as bit operations (a select between array elements could become a
// dynamic index, which the compiler would place in memory), then a funnel shift by
// (sh % 4) bytes.
__device__ __forceinline__ u32x4 realign16(u32x4 lo, u32x4 hi, uint32_t sh) {
    const uint32_t w0 = lo[0], w1 = lo[1], w2 = lo[2], w3 = lo[3];
    const uint32_t w4 = hi[0], w5 = hi[1], w6 = hi[2], w7 = hi[3];
    const uint32_t m8 = 0u - ((sh >> 3) & 1u), m4 = 0u - ((sh >> 2) & 1u);
    const uint32_t bits = (sh & 2u) * 8u;
    const auto pick = [](uint32_t m, uint32_t a, uint32_t b) { return (a & m) | (b & ~m); };
    const uint32_t s0 = pick(m8, w2, w0), s1 = pick(m8, w3, w1), s2 = pick(m8, w4, w2),
                   s3 = pick(m8, w5, w3), s4 = pick(m8, w6, w4), s5 = pick(m8, w7, w5);
    const uint32_t t0 = pick(m4, s1, s0), t1 = pick(m4, s2, s1), t2 = pick(m4, s3, s2),
                   t3 = pick(m4, s4, s3), t4 = pick(m4, s5, s4);
    return u32x4{__builtin_amdgcn_alignbit(t1, t0, bits), __builtin_amdgcn_alignbit(t2, t1, bits),
                 __builtin_amdgcn_alignbit(t3, t2, bits), __builtin_amdgcn_alignbit(t4, t3, bits)};
}

// Word masks keeping the first `left` 2-byte elements of an 8-element chunk (left <= 0:
// none, >= 8: all).
__device__ __forceinline__ u32x4 first_elems_mask(int left) {
    u32x4 m;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        m[j] = 2 * j + 1 < left ? 0xffffffffu : (2 * j < left ? 0x0000ffffu : 0u);
    return m;
}

// ------------------------------------------------------------------------------------
// The tiled kernel.
//   Template: DT (fp16/bf16), LAYOUT (B as [N,K] or [K,N]), BM x BN x BK tile, WM x WN
//   waves (each owns a (BM/WM) x (BN/WN) block of the tile, in 32 x 32 MFMA blocks).
//   Host-checked requirements: K % 8 == 0, N % 8 == 0, 16-byte aligned A, B, C, and
//   A and B each at most 2^31 bytes.
//   Edges: a load that must not happen (a row of A past M, of B past N, a chunk with
//   k >= K, a tile past the last) gets the offset kOutOfRange, which the buffer range
//   check turns into zeros without a memory access; stores outside [M,N] are skipped.
//   MASKED: the same tiles and pipeline for operands of any 2-byte alignment and any
//   sizes (A and B each at most 2^31 - 32 bytes), and C stored one element at a time.
//     K contiguous ([M,K] A, [N,K] B): each 16-byte chunk of a tile row is read as the
//       two aligned 16-byte blocks around it, through a buffer whose base is the
//       operand's address rounded down to 16 bytes and whose size is rounded up to 16
//       (so no block reaches past the operand's last 16-byte block), with the whole
//       offset in the range-checked vector offset; the chunk's shift within the blocks
//       is fixed per row (chunks start 16 bytes apart), and the chunk is realigned in
//       registers and, in the last K tile, masked to the elements below K;
//     K as the row index ([K,M] A, [K,N] B): 2-byte loads, each masked by its own k
//       and column: lane l reads column 64h + l of 8 consecutive k rows (one load
//       instruction reads 128 contiguous bytes), which are the 8 k of one 16-byte LDS
//       chunk of tile row 64h + l, written whole (neighbouring lanes, neighbouring
//       rows: no conflicts); the row and k positions common to the wave go into the
//       scalar offset.
//
// Pipeline (two LDS stages, one register stage, double-buffered MFMA operands).  Step t
// computes tile t from LDS stage t%2 in KS k-substeps of 16.  Alongside its MFMAs:
//   substep 0      : tile t+1 (A part) from registers to the other stage, then the
//                    global loads of tile t+2 (A part) into the freed registers;
//   substep 1      : the same for the B part;
// so every global load has a whole step to arrive; and in every substep the operands of
// the next substep are read from LDS.  The one
// barrier per step sits before the last substep: by then every wave has written tile
// t+1 and has read its last operands of tile t, so the last substep can read the first
// operands of tile t+1 while its MFMAs run, and the next step begins with them in hand.
// Steps past the last tile run with out-of-range loads (zeros), so the loop body has
// no branches.
// ------------------------------------------------------------------------------------
// Epilogue through LDS for the 32x32x16 accumulator layout (a lane holds row lane % 32
// of each 32-row block and columns 8g + 4 (lane / 32) .. +3, g = 0..3, of each 32-column
// block: 16-byte pieces of 32 rows per store if written directly).  Each of the NW waves
// stages its WTM x WTN block in LDS, WTM/NP rows per pass (rows padded by 16 bytes, so
// the 8-byte writes of 16 rows fall in distinct banks), and stores it back as whole row
// segments of WTN columns, 16 bytes per lane.  The caller has freed the first CAP
// elements of LDS for all waves (a barrier after the last operand reads); a wave's LDS
// accesses complete in order, so a pass's writes follow the previous pass's reads.
template <int TM, int WTM, int SRS, int NW, int CAP>
constexpr int staged_passes() {
    for (int np = 1; np <= TM; ++np)
        if (TM % np == 0 && (WTM / np) * SRS * NW <= CAP)
            return np;
    return -1;
}
// MASKED: C may have any 2-byte alignment and N any value, so each lane stores its eight
// elements one by one, those at n < N only.
template <int DT, int WTM, int WTN, int NW, int CAP, bool MASKED = false>
__device__ __forceinline__ void store_c_staged(const f32x16 (&acc)[WTM / 32][WTN / 32],
                                               u16* lds, int wave, int lane, u16* C, int M,
                                               int N, int ldc, int mrow0, int ncol0) {
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int SRS = WTN + 8;                   // staged row stride in elements
    constexpr int NP = staged_passes<TM, WTM, SRS, NW, CAP>();
    static_assert(NP > 0, "C staging fits the LDS ring");
    constexpr int HR = WTM / NP;                   // rows staged per pass
    constexpr int LPR = WTN / 8;                   // lanes per staged row
    constexpr int RPR = 64 / LPR;                  // rows per 64-lane read
    static_assert(64 % LPR == 0 && HR % RPR == 0, "staging split");
    u16* stg = lds + wave * HR * SRS;
    const int half = lane >> 5;
    const int sr = lane / LPR, sc = (lane % LPR) * 8;
    const int n = ncol0 + sc;
#pragma unroll
    for (int ps = 0; ps < NP; ++ps) {
#pragma unroll
        for (int i = ps * (TM / NP); i < (ps + 1) * (TM / NP); ++i) {
            const int r = (i - ps * (TM / NP)) * 32 + (lane & 31);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 v;
                    v[0] = pack2<DT>(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
                    v[1] = pack2<DT>(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
                    *reinterpret_cast<u32x2*>(stg + r * SRS + j * 32 + 8 * g + 4 * half) = v;
                }
            }
        }
#pragma unroll
        for (int q = 0; q < HR / RPR; ++q) {
            const int r = q * RPR + sr;
            const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * SRS + sc);
            const int m = mrow0 + ps * HR + r;
            if constexpr (MASKED) {
                if (m < M) {
                    u16* row = C + (size_t)m * ldc + n;
                    const u16x8 h = __builtin_bit_cast(u16x8, v);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (n + e < N)
                            row[e] = h[e];
                }
            } else if (m < M && n < N) {
                *reinterpret_cast<u32x4*>(C + (size_t)m * ldc + n) = v;
            }
        }
    }
}

template <int DT, int ALAYOUT, int LAYOUT, int BM, int BN, int BK, int WM, int WN,
          bool MASKED = false>
__global__ void __attribute__((amdgpu_flat_work_group_size(WM * WN * 64, WM * WN * 64),
                               amdgpu_waves_per_eu(1, 1)))
gemm_tiled(const u16* __restrict__ A, const u16* __restrict__ B, u16* __restrict__ C, int M,
           int N, int K, int lda, int ldb, int ldc, int grid_m, int grid_n, int group_m) {
    constexpr int NT = WM * WN * 64;
    constexpr int KC = BK / 8;              // 16-byte chunks in one tile row
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int KS = BK / 16;             // MFMA k-substeps per tile
    constexpr int A_ELEMS = BM * BK;
    constexpr int STAGE = (BM + BN) * BK;   // elements of one LDS stage (A then B)
    constexpr int RS = NT / KC;             // rows between the chunks one thread loads
    // Per thread: A_LD / B_LD 16-byte chunks of a K-contiguous operand, or the 8 rows of
    // one 8x8 block of an operand stored with K as its row index ([K,M] A, [K,N] B).
    constexpr int A_LD = (ALAYOUT == LAYOUT_MK) ? BM / RS : 8;
    constexpr int B_LD = (LAYOUT == LAYOUT_NK) ? BN / RS : 8;
    constexpr int KM_BLK = KC * (BM / 8);   // 8x8 blocks of a [K,M] A tile
    constexpr int KN_BLK = KC * (BN / 8);   // 8x8 blocks of a [K,N] B tile
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(BK % 32 == 0 && NT % KC == 0, "BK must give an even number of substeps");
    static_assert((NT / 16) % KC == 0, "a thread's rows must share one swizzle");
    static_assert((ALAYOUT == LAYOUT_KM || BM % RS == 0) &&
                  (LAYOUT == LAYOUT_KN || BN % RS == 0), "bad load split");
    static_assert(ALAYOUT == LAYOUT_MK || KM_BLK <= NT, "one 8x8 [K,M] block per thread");
    static_assert(LAYOUT == LAYOUT_NK || KN_BLK <= NT, "one 8x8 [K,N] block per thread");
    // MASKED parts: 8 tile rows of a wave (K contiguous), or one 64-column x 8-k block of
    // a wave (K as the row index); else the 16-byte loads above.
    constexpr int NW = WM * WN;
    constexpr int A_PARTS = !MASKED || ALAYOUT == LAYOUT_MK ? A_LD : BM / 64 * KC / NW;
    constexpr int B_PARTS = !MASKED || LAYOUT == LAYOUT_NK ? B_LD : BN / 64 * KC / NW;
    static_assert(!MASKED || (BK == 64 && BM % 64 == 0 && BN % 64 == 0 &&
                              (BM / 64 * KC) % NW == 0 && (BN / 64 * KC) % NW == 0),
                  "masked parts: 64 k per tile row, whole parts per wave");

    __shared__ __attribute__((aligned(16))) u16 lds[2 * STAGE];

    int tm, tn;
    tile_of((int)blockIdx.x, grid_m, grid_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int nk = (K + BK - 1) / BK;

    // MASKED, K contiguous: a_d / b_d is the operand's byte offset past 16-byte alignment;
    // its buffer starts that many bytes lower and ends at the next 16-byte boundary.
    constexpr bool A_RA = MASKED && ALAYOUT == LAYOUT_MK, B_RA = MASKED && LAYOUT == LAYOUT_NK;
    const uint32_t a_d = A_RA ? (uint32_t)((uintptr_t)A & 15u) : 0u;
    const uint32_t b_d = B_RA ? (uint32_t)((uintptr_t)B & 15u) : 0u;
    const auto round16 = [](uint32_t x) { return (x + 15u) & ~15u; };
    const rsrc_t ra =
        A_RA ? make_rsrc(reinterpret_cast<const char*>(A) - a_d,
                         round16(a_d + span_bytes(M, K, lda)))
             : (ALAYOUT == LAYOUT_MK ? make_rsrc(A, span_bytes(M, K, lda))
                                     : make_rsrc(A, span_bytes(K, M, lda)));
    const rsrc_t rb =
        B_RA ? make_rsrc(reinterpret_cast<const char*>(B) - b_d,
                         round16(b_d + span_bytes(N, K, ldb)))
             : (LAYOUT == LAYOUT_NK ? make_rsrc(B, span_bytes(N, K, ldb))
                                    : make_rsrc(B, span_bytes(K, N, ldb)));

    // ---- global -> register addressing (byte offsets; the K position goes in soffset) --
    const int lc = tid % KC;                 // this thread's chunk column (row-major loads)
    const int lr = tid / KC;                 // its first row; the others follow every RS
    // For an operand stored with K as its row index, thread tid loads the 8x8 block
    // (k = 8*kb .. +7, row r0 + 8*rb .. +7); its 8 rows of the tile lie inside the
    // operand or outside it together (the row count is a multiple of 8).
    const int t_kb = tid % KC, t_rb = tid / KC;

    uint32_t a_off[ALAYOUT == LAYOUT_MK ? A_LD : 1];
    int a_lds;
    bool km_live = true;
    uint32_t a_sh[A_RA ? A_LD : 1];      // MASKED: each row's chunk shift in bytes
    if constexpr (ALAYOUT == LAYOUT_MK) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int r = m0 + lr + i * RS;
            if constexpr (A_RA) {
                const uint32_t at = a_d + (uint32_t)(r * lda + lc * 8) * 2u;
                a_off[i] = r < M ? at & ~15u : kOutOfRange;
                a_sh[i] = at & 15u;
            } else {
                a_off[i] = r < M ? (uint32_t)(r * lda + lc * 8) * 2u : kOutOfRange;
            }
        }
        a_lds = lr * BK + ((lc ^ swz<KC>(lr)) * 8);
    } else {
        km_live = (tid < KM_BLK) && (m0 + t_rb * 8 < M);
        a_off[0] = ((uint32_t)(t_kb * 8) * (uint32_t)lda + (uint32_t)(m0 + t_rb * 8)) * 2u;
        a_lds = (t_rb * 8) * BK;
    }

    uint32_t b_off[LAYOUT == LAYOUT_NK ? B_LD : 1];
    int b_lds;
    bool kn_live = true;
    uint32_t b_sh[B_RA ? B_LD : 1];
    if constexpr (LAYOUT == LAYOUT_NK) {
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int r = n0 + lr + i * RS;
            if constexpr (B_RA) {
                const uint32_t at = b_d + (uint32_t)(r * ldb + lc * 8) * 2u;
                b_off[i] = r < N ? at & ~15u : kOutOfRange;
                b_sh[i] = at & 15u;
            } else {
                b_off[i] = r < N ? (uint32_t)(r * ldb + lc * 8) * 2u : kOutOfRange;
            }
        }
        b_lds = A_ELEMS + lr * BK + ((lc ^ swz<KC>(lr)) * 8);
    } else {
        kn_live = (tid < KN_BLK) && (n0 + t_rb * 8 < N);
        b_off[0] = ((uint32_t)(t_kb * 8) * (uint32_t)ldb + (uint32_t)(n0 + t_rb * 8)) * 2u;
        b_lds = A_ELEMS + (t_rb * 8) * BK;
    }

    u32x4 a_reg[MASKED && !A_RA ? 1 : A_LD];
    u32x4 b_reg[MASKED && !B_RA ? 1 : B_LD];
    u32x4 a_hi[A_RA ? A_LD : 1];          // MASKED, K contiguous: the second block
    u32x4 b_hi[B_RA ? B_LD : 1];
    u16 a_el[MASKED && !A_RA ? A_PARTS : 1][8];
    u16 b_el[MASKED && !B_RA ? B_PARTS : 1][8];
    // MASKED, K as the row index: the wave index as a scalar (it feeds scalar offsets)
    // and each operand's per-lane byte offset (column m0 + lane, n0 + lane).
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t a_lane = (uint32_t)(m0 + lane) * 2u;
    const uint32_t b_lane = (uint32_t)(n0 + lane) * 2u;

    // MASKED, K as the row index: part i of an operand (`rows` columns inside it from
    // column r0 on) of tile kt: column 64h + lane of k rows 8 kb .. 8 kb + 7, with
    // (h, kb) = block NW * i + wv; then its 16-byte LDS write into tile row 64h + lane.
    auto mload_part = [&](u16 (&el)[8], rsrc_t rs, uint32_t lane_off, int r0, int rows,
                          int ld, int kt, auto ic) {
        constexpr int i = decltype(ic)::value;
        const bool live = kt < nk;
        const int k0 = live ? kt * BK : 0;
        const int q = NW * i + wv, h = q / KC, kb = q % KC;
        const bool cok = r0 + 64 * h + lane < rows;
        // (the range check sees the vector offset only: an element out of range needs no
        // particular scalar offset; & rather than && and an unconditional scalar offset
        // keep these selects, not branches)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int kr = k0 + 8 * kb + j;
            const bool kok = live & (kr < K);
            const uint32_t so = ((uint32_t)kr * (uint32_t)ld + (uint32_t)(64 * h)) * 2u;
            el[j] = load2(rs, (kok & cok) ? lane_off : kOutOfRange, so);
        }
    };
    auto mwrite_part = [&](u16* st, const u16 (&el)[8], auto ic) {
        constexpr int i = decltype(ic)::value;
        const int q = NW * i + wv, h = q / KC, kb = q % KC;
        const int rt = 64 * h + lane;
        u16x8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            v[j] = el[j];
        *reinterpret_cast<u32x4*>(st + rt * BK + ((kb ^ swz<KC>(rt)) * 8)) =
            __builtin_bit_cast(u32x4, v);
    };

    // One part of an operand's loads of tile kt: chunk i (K contiguous) or k row i of the
    // thread's 8x8 block (K as the row index).
    auto gload_part = [&](u32x4* reg, rsrc_t rs, const uint32_t* off, bool kmajor,
                          bool t_live, int ld, int kt, auto ic) {
        constexpr int i = decltype(ic)::value;
        const bool live = kt < nk;
        const int k0 = live ? kt * BK : 0;
        if (kmajor) {
            const bool ok = live && (k0 + lc * 8 < K);
            reg[i] = load16(rs, ok ? off[i] : kOutOfRange, (uint32_t)k0 * 2u);
        } else {
            const bool ok = live && t_live && (k0 + t_kb * 8 + i < K);
            reg[i] = load16(rs, ok ? off[0] + (uint32_t)i * (uint32_t)ld * 2u : kOutOfRange,
                            (uint32_t)k0 * (uint32_t)ld * 2u);
        }
    };
    // MASKED, K contiguous: chunk i's two aligned blocks of tile kt, the whole offset in
    // the vector offset (range-checked), out of range for a chunk at or past K.
    auto rload_part = [&](u32x4* lo, u32x4* hi, rsrc_t rs, const uint32_t* off, int kt,
                          auto ic) {
        constexpr int i = decltype(ic)::value;
        const bool live = kt < nk;
        const int k0 = live ? kt * BK : 0;
        // (a row past the edge has off[i] = kOutOfRange, which stays out of range with
        // the K offset added; & rather than && keeps this a select, not a branch)
        const uint32_t at = off[i] + (uint32_t)k0 * 2u;
        const uint32_t vo = (live & (k0 + lc * 8 < K)) ? at : kOutOfRange;
        lo[i] = load16(rs, vo, 0u);
        hi[i] = load16(rs, vo + 16u, 0u);
    };
    auto gload_a_part = [&](int kt, auto ic) {
        if constexpr (A_RA)
            rload_part(a_reg, a_hi, ra, a_off, kt, ic);
        else if constexpr (MASKED)
            mload_part(a_el[decltype(ic)::value], ra, a_lane, m0, M, lda, kt, ic);
        else
            gload_part(a_reg, ra, a_off, ALAYOUT == LAYOUT_MK, km_live, lda, kt, ic);
    };
    auto gload_b_part = [&](int kt, auto ic) {
        if constexpr (B_RA)
            rload_part(b_reg, b_hi, rb, b_off, kt, ic);
        else if constexpr (MASKED)
            mload_part(b_el[decltype(ic)::value], rb, b_lane, n0, N, ldb, kt, ic);
        else
            gload_part(b_reg, rb, b_off, LAYOUT == LAYOUT_NK, kn_live, ldb, kt, ic);
    };
    auto gload_a = [&](int kt) {
        static_for<0, A_PARTS>([&](auto i) { gload_a_part(kt, i); });
    };
    auto gload_b = [&](int kt) {
        static_for<0, B_PARTS>([&](auto i) { gload_b_part(kt, i); });
    };
    // One part of an operand tile's LDS write: chunk i (K contiguous), or tile row
    // 8*rb + i of the transposed 8x8 block (reg[j] holds rows 0..7 at k = j; row i
    // receives k = 0..7).
    auto swrite_part = [&](u16* st, const u32x4* reg, int lds_at, bool kmajor, int blocks,
                           auto ic) {
        constexpr int i = decltype(ic)::value;
        if (kmajor) {
            *reinterpret_cast<u32x4*>(st + lds_at + i * RS * BK) = reg[i];
        } else if (tid < blocks) {
            constexpr int p = i >> 1;
            constexpr uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
            u32x4 o;
            o[0] = __builtin_amdgcn_perm(reg[1][p], reg[0][p], sel);
            o[1] = __builtin_amdgcn_perm(reg[3][p], reg[2][p], sel);
            o[2] = __builtin_amdgcn_perm(reg[5][p], reg[4][p], sel);
            o[3] = __builtin_amdgcn_perm(reg[7][p], reg[6][p], sel);
            *reinterpret_cast<u32x4*>(st + lds_at + i * BK +
                                      ((t_kb ^ swz<KC>(t_rb * 8 + i)) * 8)) = o;
        }
    };
    // MASKED, K contiguous: chunk i of tile kt realigned and, in the last K tile, cut to
    // the elements below K (tail_keep: this lane's chunk mask there), in place, ready for
    // the plain chunk write.  Branch-free: other tiles OR the mask with all ones.
    const u32x4 tail_keep =
        A_RA || B_RA ? first_elems_mask(K - ((nk > 0 ? nk - 1 : 0) * BK + lc * 8)) : u32x4{};
    auto realign_part = [&](u32x4* lo, const u32x4* hi, const uint32_t* sh, int kt, auto ic) {
        constexpr int i = decltype(ic)::value;
        const uint32_t keep_all = kt * BK + BK > K ? 0u : 0xffffffffu;
        lo[i] = realign16(lo[i], hi[i], sh[i]) & (tail_keep | keep_all);
    };
    auto swrite_a_part = [&](u16* st, int kt, auto ic) {
        if constexpr (A_RA) {
            realign_part(a_reg, a_hi, a_sh, kt, ic);
            swrite_part(st, a_reg, a_lds, true, KM_BLK, ic);
        } else if constexpr (MASKED) {
            mwrite_part(st, a_el[decltype(ic)::value], ic);
        } else {
            swrite_part(st, a_reg, a_lds, ALAYOUT == LAYOUT_MK, KM_BLK, ic);
        }
    };
    auto swrite_b_part = [&](u16* st, int kt, auto ic) {
        if constexpr (B_RA) {
            realign_part(b_reg, b_hi, b_sh, kt, ic);
            swrite_part(st, b_reg, b_lds, true, KN_BLK, ic);
        } else if constexpr (MASKED) {
            mwrite_part(st + A_ELEMS, b_el[decltype(ic)::value], ic);
        } else {
            swrite_part(st, b_reg, b_lds, LAYOUT == LAYOUT_NK, KN_BLK, ic);
        }
    };
    auto swrite_a = [&](u16* st, int kt) {
        static_for<0, A_PARTS>([&](auto i) { swrite_a_part(st, kt, i); });
    };
    auto swrite_b = [&](u16* st, int kt) {
        static_for<0, B_PARTS>([&](auto i) { swrite_b_part(st, kt, i); });
    };

    // ---- LDS -> MFMA operands ---------------------------------------------------------
    const int xr = swz<KC>(lane & 31);       // swizzle of this lane's rows (bases are x32)
    const int half = lane >> 5;               // which 8 of the 16 k of an MFMA step
    const int a_row0 = (wm * WTM + (lane & 31)) * BK;
    const int b_row0 = A_ELEMS + (wn * WTN + (lane & 31)) * BK;

    u32x4 fa[2][TM], fb[2][TN];
    auto read_frag = [&](const u16* st, int s, int buf, auto idx) {
        constexpr int I = decltype(idx)::value;
        const int koff = (((2 * s) | half) ^ xr) * 8;
        if constexpr (I < TM)
            fa[buf][I] = *reinterpret_cast<const u32x4*>(st + a_row0 + I * 32 * BK + koff);
        else
            fb[buf][I - TM] =
                *reinterpret_cast<const u32x4*>(st + b_row0 + (I - TM) * 32 * BK + koff);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

    if (nk > 0) {
        gload_a(0);
        gload_b(0);
        swrite_a(lds, 0);
        swrite_b(lds, 0);
        gload_a(1);
        gload_b(1);
        block_sync_lds();
        static_for<0, TM + TN>([&](auto i) { read_frag(lds, 0, 0, i); });

        // Memory operations of substep S, in issue order: the TM + TN operand reads of
        // the next substep, then (substep 0) the A part of tile t+1 to LDS and the A
        // loads of tile t+2, then (substep WB) the same for B.  They are dealt out over
        // the substep's TM*TN MFMA slots, front-loaded, one MFMA per slot.
        constexpr int WB = KS > 2 ? 1 : 0;
        constexpr int NR = TM + TN;
        for (int kt = 0; kt < nk; ++kt) {
            u16* cur = lds + (kt & 1) * STAGE;
            u16* nxt = lds + ((kt & 1) ^ 1) * STAGE;
            const int kt2 = kt + 2;
            static_for<0, KS>([&](auto sc) {
                constexpr int S = decltype(sc)::value;
                constexpr int NWA = (S == 0) ? A_PARTS : 0;
                constexpr int NWB = (S == WB) ? B_PARTS : 0;
                constexpr int NOPS = NR + 2 * NWA + 2 * NWB;
                constexpr int SLOTS = TM * TN;
                auto mem_op = [&](auto oc) {
                    constexpr int O = decltype(oc)::value;
                    if constexpr (O < NR) {
                        if constexpr (S + 1 < KS)
                            read_frag(cur, S + 1, (S + 1) & 1, std::integral_constant<int, O>{});
                        else
                            read_frag(nxt, 0, 0, std::integral_constant<int, O>{});
                    } else if constexpr (O < NR + NWA) {
                        constexpr int i = O - NR;
                        swrite_a_part(nxt, kt + 1, std::integral_constant<int, i>{});
                    } else if constexpr (O < NR + 2 * NWA) {
                        constexpr int i = O - NR - NWA;
                        gload_a_part(kt2, std::integral_constant<int, i>{});
                    } else if constexpr (O < NR + 2 * NWA + NWB) {
                        constexpr int i = O - NR - 2 * NWA;
                        swrite_b_part(nxt, kt + 1, std::integral_constant<int, i>{});
                    } else {
                        constexpr int i = O - NR - 2 * NWA - NWB;
                        gload_b_part(kt2, std::integral_constant<int, i>{});
                    }
                };
                static_for<0, SLOTS>([&](auto jc) {
                    constexpr int J = decltype(jc)::value;
                    constexpr int i = J / TN, j = J % TN;
                    // S0 = B rows (n), S1 = A rows (m): lane l then holds C row m = l % 32
                    // and four consecutive columns n per group of four results.
                    acc[i][j] = mfma_32x32x16<DT>(fb[S & 1][j], fa[S & 1][i], acc[i][j]);
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (S == KS - 1 && J == 0) {
                        block_sync_lds();
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    constexpr int lo = (J * NOPS + SLOTS - 1) / SLOTS;
                    constexpr int hi = ((J + 1) * NOPS + SLOTS - 1) / SLOTS;
                    static_for<lo, hi>([&](auto oc) {
                        mem_op(oc);
                        __builtin_amdgcn_sched_barrier(0);
                    });
                });
            });
        }
    }

    // ---- epilogue: cast once, stage through LDS, store whole row segments ----------------
    __syncthreads();
    store_c_staged<DT, WTM, WTN, WM * WN, 2 * STAGE, MASKED>(acc, lds, wave, lane, C, M, N,
                                                             ldc, m0 + wm * WTM,
                                                             n0 + wn * WTN);
}

// ------------------------------------------------------------------------------------
// Direct-to-LDS kernel (B as [N,K] only).
//   The global loads write LDS themselves (buffer_load_dwordx4 ... lds): one instruction
//   moves 64 lanes x 16 bytes into 1 KiB of consecutive LDS bytes starting at an address
//   held in M0, lane l filling bytes [16l, 16l+16).  No register staging and no LDS-write
//   instructions, so the tile ring can be deep: STAGES buffers of BK = 32 (two MFMA
//   k-substeps each), the loads of tile t+STAGES-1 issued while tile t is computed.
//   Swizzle: a 1 KiB block holds 64/KC consecutive tile rows; lane l lands in row
//   l / KC of the block at physical chunk l % KC, so it loads the logical chunk
//   (l % KC) ^ swz(row) of that row -- the placement the fragment reads expect.
//   Requirements as for gemm_tiled.  A chunk past K or a row past M/N is read out of
//   range, which the hardware turns into zeros written to LDS.
// Per step t (compute tile t from stage t % STAGES, BK / 16 substeps, an even number):
//   substep 0     : MFMAs; read the operands of substep 1; issue tile t+STAGES-1's loads
//                   into the stage tile t-1 used (free since the previous step's barrier);
//   substep s     : MFMAs; read the operands of substep s+1;
//   last substep  : one MFMA; wait until this wave's loads of tile t+1 have landed and
//                   meet the other waves (tile t+1 complete, tile t no longer read); the
//                   remaining MFMAs with the reads of tile t+1's first operands.
// BK = 64 makes every row segment a whole 128-byte line (one request per line).
// SPLIT: split-K over workgroups ("Tiling a matmul", section "Where it breaks": a grid of
// few output tiles leaves compute units idle; splitting K gives each of them work).
// Workgroup (tile, z) sums k in [z*kc, min(K, (z+1)*kc)) (kc a multiple of BK) and
// writes its fp32 partial tile to W[z][m][n] (packed [M,N] per split) instead of C;
// splitk_reduce, the next kernel on the stream, adds the partials in split order, casts
// once and stores C.  (Summing in the last workgroup of each tile instead, behind a
// device-scope arrival counter, measured slower on gfx950: the partials then have to be
// made coherent across the XCDs inside the kernel.)
// ------------------------------------------------------------------------------------
// The same buffer resource as four dwords (base address low/high, size, format), for the
// direct-to-LDS loads below.
typedef u32x4 rsrc4_t;
__device__ __forceinline__ rsrc4_t make_rsrc4(const void* base, uint32_t bytes) {
    const uint64_t p = (uint64_t)(uintptr_t)base;
    return rsrc4_t{(uint32_t)p, (uint32_t)(p >> 32) & 0xffffu, bytes, kRsrcWord3};
}

// One direct-to-LDS load: 64 lanes x 16 bytes to lds_dst (M0) + 16 * lane.  Issued from
// inline assembly so that the compiler does not track it: it would otherwise wait for
// every such load in flight before each transposing LDS read (it cannot tell that they
// touch different stages).  The kernels order these loads themselves, with explicit
// vmcnt waits and barriers, and never read a stage before their own waits say it landed.
__device__ __forceinline__ void dma16(rsrc4_t r, u16* lds_dst, uint32_t voff, uint32_t soff) {
    // the destination and the K offset are the same for every lane of the wave
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_dst);
    const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 ::"v"(voff), "s"(r), "s"(so), "s"(m0v)
                 : "memory", "m0");
}

// The same load with the destination given as an LDS byte address (wave-uniform), so
// that the address arithmetic stays in scalar registers.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// POL selects the cache policy of the load (0: default, 1: nt, 2: sc0, 3: sc1,
// 4: sc0 sc1, 5: sc0 nt, 6: sc1 nt).
template <int POL = 0>
__device__ __forceinline__ void dma16_at(rsrc4_t r, uint32_t lds_byte, uint32_t voff,
                                         uint32_t soff) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_byte);
    const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
#define TGEMM_DMA_ASM(SUFFIX)                                                              \
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen" SUFFIX " lds" \
                 ::"v"(voff), "s"(r), "s"(so), "s"(m0v)                                      \
                 : "memory", "m0")
    if constexpr (POL == 0) TGEMM_DMA_ASM("");
    else if constexpr (POL == 1) TGEMM_DMA_ASM(" nt");
    else if constexpr (POL == 2) TGEMM_DMA_ASM(" sc0");
    else if constexpr (POL == 3) TGEMM_DMA_ASM(" sc1");
    else if constexpr (POL == 4) TGEMM_DMA_ASM(" sc0 sc1");
    else if constexpr (POL == 5) TGEMM_DMA_ASM(" sc0 nt");
    else TGEMM_DMA_ASM(" sc1 nt");
#undef TGEMM_DMA_ASM
}

// Direct-to-LDS loads that walk M0 themselves: set_m0 points M0 at the first 1 KiB
// destination, and each dma16_next writes the next 1 KiB block and advances M0 by 1 KiB,
// so consecutive blocks need no M0 set-up of their own.  An M0 write needs one
// instruction before the next LDS-DMA load: NOP emits it where nothing else intervenes.
// The M0 increment also writes SCC, which the asm declares (a condition the compiler
// keeps in SCC across the load would otherwise be lost).
__device__ __forceinline__ void set_m0(uint32_t lds_byte) {
    asm volatile("s_mov_b32 m0, %0" ::"s"(__builtin_amdgcn_readfirstlane(lds_byte)) : "m0");
}
template <int POL, bool NOP>
__device__ __forceinline__ void dma16_next(rsrc4_t r, uint32_t voff, uint32_t soff) {
    const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
    if constexpr (NOP) {
        if constexpr (POL == 2)
            asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen sc0 lds\n\ts_add_u32 m0, m0, 0x400"
                         ::"v"(voff), "s"(r), "s"(so) : "memory", "m0", "scc");
        else
            asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds\n\ts_add_u32 m0, m0, 0x400"
                         ::"v"(voff), "s"(r), "s"(so) : "memory", "m0", "scc");
    } else {
        if constexpr (POL == 2)
            asm volatile("buffer_load_dwordx4 %0, %1, %2 offen sc0 lds\n\ts_add_u32 m0, m0, 0x400"
                         ::"v"(voff), "s"(r), "s"(so) : "memory", "m0", "scc");
        else
            asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds\n\ts_add_u32 m0, m0, 0x400"
                         ::"v"(voff), "s"(r), "s"(so) : "memory", "m0", "scc");
    }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_lgkm() {
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm_then_sync() {
    // This wave's global->LDS loads down to N outstanding, its LDS traffic drained, then
    // the workgroup barrier.
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int DT, int BM, int BN, int BK, int WM, int WN, int STAGES, bool SPLIT>
__global__ void __attribute__((amdgpu_flat_work_group_size(WM * WN * 64, WM * WN * 64),
                               amdgpu_waves_per_eu(1, 1)))
gemm_dma(const u16* __restrict__ A, const u16* __restrict__ B, u16* __restrict__ C, int M,
         int N, int K, int lda, int ldb, int ldc, int grid_m, int grid_n, int group_m,
         float* __restrict__ W, int kc) {
    constexpr int NW = WM * WN;
    constexpr int KC = BK / 8;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int KS = BK / 16;
    constexpr int A_ELEMS = BM * BK;
    constexpr int STAGE = (BM + BN) * BK;
    constexpr int ROWS = 64 / KC;                 // tile rows per 1 KiB load
    constexpr int A_LD = BM / ROWS / NW;          // A loads per wave per tile
    constexpr int B_LD = BN / ROWS / NW;
    constexpr int LD = A_LD + B_LD;
    static_assert(KS % 2 == 0, "an even number of k-substeps per tile");
    static_assert((BM / ROWS) % NW == 0 && (BN / ROWS) % NW == 0, "bad load split");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(STAGES >= 3 && LD * (STAGES - 2) <= 63, "vmcnt range");
    static_assert(STAGES * STAGE * 2 <= 160 * 1024, "LDS");

    __shared__ __attribute__((aligned(1024))) u16 lds[STAGES * STAGE];

    int tm, tn;
    tile_of((int)blockIdx.x, grid_m, grid_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    // this workgroup's K range [kb, ke)
    const int kb = SPLIT ? (int)blockIdx.y * kc : 0;
    const int ke = SPLIT ? (K - kb < kc ? K : kb + kc) : K;
    const int nk = ke > kb ? (ke - kb + BK - 1) / BK : 0;

    const rsrc4_t ra = make_rsrc4(A, span_bytes(M, K, lda));
    const rsrc4_t rb = make_rsrc4(B, span_bytes(N, K, ldb));

    // Lane l lands in row l / KC of a 1 KiB block at physical chunk l % KC; it fetches
    // the logical chunk that the swizzle of that row (block base + l / KC) puts there.
    const int prow = lane / KC;
    uint32_t a_off[A_LD], b_off[B_LD];
    int a_kc[A_LD], b_kc[B_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int row = (wave * A_LD + i) * ROWS + prow;
        a_kc[i] = ((lane % KC) ^ swz<KC>(row)) * 8;
        a_off[i] = m0 + row < M ? (uint32_t)((m0 + row) * lda + a_kc[i]) * 2u : kOutOfRange;
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int row = (wave * B_LD + i) * ROWS + prow;
        b_kc[i] = ((lane % KC) ^ swz<KC>(row)) * 8;
        b_off[i] = n0 + row < N ? (uint32_t)((n0 + row) * ldb + b_kc[i]) * 2u : kOutOfRange;
    }
    auto stage_ptr = [&](int t) { return lds + (t % STAGES) * STAGE; };
    // Load i (< LD) of tile kt into its stage.
    auto dma = [&](int kt, auto ic) {
        constexpr int i = decltype(ic)::value;
        const bool live = kt < nk;
        const int k0 = live ? kb + kt * BK : 0;
        u16* st = stage_ptr(kt);
        if constexpr (i < A_LD)
            dma16(ra, st + (wave * A_LD + i) * ROWS * BK,
                     live && k0 + a_kc[i] < ke ? a_off[i] : kOutOfRange, (uint32_t)k0 * 2u);
        else
            dma16(rb, st + A_ELEMS + (wave * B_LD + (i - A_LD)) * ROWS * BK,
                     live && k0 + b_kc[i - A_LD] < ke ? b_off[i - A_LD] : kOutOfRange,
                     (uint32_t)k0 * 2u);
    };

    const int xr = swz<KC>(lane & 31);
    const int half = lane >> 5;
    const int a_row0 = (wm * WTM + (lane & 31)) * BK;
    const int b_row0 = A_ELEMS + (wn * WTN + (lane & 31)) * BK;
    u32x4 fa[2][TM], fb[2][TN];
    auto read_frag = [&](const u16* st, int s, int buf, auto idx) {
        constexpr int I = decltype(idx)::value;
        const int koff = (((2 * s) | half) ^ xr) * 8;
        if constexpr (I < TM)
            fa[buf][I] = *reinterpret_cast<const u32x4*>(st + a_row0 + I * 32 * BK + koff);
        else
            fb[buf][I - TM] =
                *reinterpret_cast<const u32x4*>(st + b_row0 + (I - TM) * 32 * BK + koff);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

    if (nk > 0) {
        for (int p = 0; p < STAGES - 1; ++p)
            static_for<0, LD>([&](auto i) { dma(p, i); });
        wait_vm_then_sync<LD * (STAGES - 2)>();
        static_for<0, TM + TN>([&](auto i) { read_frag(lds, 0, 0, i); });
        constexpr int NR = TM + TN;
        constexpr int SLOTS = TM * TN;
        for (int kt = 0; kt < nk; ++kt) {
            const u16* cur = stage_ptr(kt);
            const u16* nxt = stage_ptr(kt + 1);
            const int kl = kt + STAGES - 1;
            static_for<0, KS>([&](auto sc) {
                constexpr int S = decltype(sc)::value;
                constexpr int NOPS = NR + (S == 0 ? LD : 0);
                static_for<0, SLOTS>([&](auto jc) {
                    constexpr int J = decltype(jc)::value;
                    constexpr int i = J / TN, j = J % TN;
                    acc[i][j] = mfma_32x32x16<DT>(fb[S & 1][j], fa[S & 1][i], acc[i][j]);
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (S == KS - 1 && J == 0) {
                        wait_vm_then_sync<LD * (STAGES - 2)>();
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    constexpr int lo = (J * NOPS + SLOTS - 1) / SLOTS;
                    constexpr int hi = ((J + 1) * NOPS + SLOTS - 1) / SLOTS;
                    static_for<lo, hi>([&](auto oc) {
                        constexpr int O = decltype(oc)::value;
                        if constexpr (O < NR) {
                            if constexpr (S + 1 < KS)
                                read_frag(cur, S + 1, (S + 1) & 1,
                                          std::integral_constant<int, O>{});
                            else
                                read_frag(nxt, 0, 0, std::integral_constant<int, O>{});
                        } else {
                            dma(kl, std::integral_constant<int, O - NR>{});
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    });
                });
            });
        }
    }

    wait_vm<0>();                                  // the trailing loads into LDS

    // a lane's C elements: row m(i), four consecutive columns n(j, g)
    auto m_of = [&](int i) { return m0 + wm * WTM + i * 32 + (lane & 31); };
    auto n_of = [&](int j, int g) { return n0 + wn * WTN + j * 32 + 8 * g + 4 * half; };
    auto quad = [&](int i, int j, int g) {
        return f32x4{acc[i][j][4 * g + 0], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                     acc[i][j][4 * g + 3]};
    };
    auto store_c = [&](int m, int n, f32x4 v) {
        u32x2 p;
        p[0] = pack2<DT>(v[0], v[1]);
        p[1] = pack2<DT>(v[2], v[3]);
        if (m < M && n < N)
            *reinterpret_cast<u32x2*>(C + (size_t)m * ldc + n) = p;
    };
    if constexpr (!SPLIT) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    store_c(m_of(i), n_of(j, g), quad(i, j, g));
    } else {
        const size_t plane = (size_t)M * (size_t)N;
        float* wz = W + (size_t)blockIdx.y * plane;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int m = m_of(i), n = n_of(j, g);
                    if (m < M && n < N)
                        *reinterpret_cast<f32x4*>(wz + (size_t)m * N + n) = quad(i, j, g);
                }
    }
}

// C = cast(sum over z of W[z]), the partial tiles of a split-K product summed in split
// order (a fixed order: repeated calls give the same bits).  One thread per 8
// consecutive columns of a row of C (N is a multiple of 8).  The partials are fetched
// eight splits at a time, all loads in flight before the first add.
template <int DT>
__global__ void __launch_bounds__(256)
splitk_reduce(const float* __restrict__ W, u16* __restrict__ C, int M, int N, int ldc,
              int S) {
    constexpr int U = 8;
    const int per_row = N >> 3;
    const int idx = (int)blockIdx.x * 256 + (int)threadIdx.x;
    if (idx >= M * per_row)
        return;
    const int m = idx / per_row, n = (idx - m * per_row) * 8;
    const size_t plane = (size_t)M * (size_t)N;
    const float* p = W + (size_t)m * (size_t)N + n;
    f32x4 lo = {0.0f, 0.0f, 0.0f, 0.0f}, hi = lo;
    for (int z0 = 0; z0 < S; z0 += U) {
        f32x4 a[U], b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (z0 + u < S) {
                a[u] = *reinterpret_cast<const f32x4*>(p + (size_t)(z0 + u) * plane);
                b[u] = *reinterpret_cast<const f32x4*>(p + (size_t)(z0 + u) * plane + 4);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (z0 + u < S) {
                lo += a[u];
                hi += b[u];
            }
        }
    }
    u32x4 v;
    v[0] = pack2<DT>(lo[0], lo[1]);
    v[1] = pack2<DT>(lo[2], lo[3]);
    v[2] = pack2<DT>(hi[0], hi[1]);
    v[3] = pack2<DT>(hi[2], hi[3]);
    *reinterpret_cast<u32x4*>(C + (size_t)m * ldc + n) = v;
}


// The stream-K partials (gemm_quad_sk): each element of C, eight consecutive columns per
// thread, is the sum of its tile's segments in workgroup order (their K ranges in
// order), read from the slots the workgroups wrote, cast once.  Workgroups with an
// empty range wrote nothing and are skipped.
template <int DT>
__global__ void __launch_bounds__(256)
sk_reduce(const float* __restrict__ W, u16* __restrict__ C, int M, int N, int ldc, int grid_n,
          int nk, int tiles, int G) {
    const int per_row = N >> 3;
    const int idx = (int)blockIdx.x * 256 + (int)threadIdx.x;
    if (idx >= M * per_row)
        return;
    const int m = idx / per_row, n = (idx - m * per_row) * 8;
    const int tm = m >> 8, tn = n >> 8;
    const int64_t I = (int64_t)tiles * nk;
    const int64_t i0 = (int64_t)(tm * grid_n + tn) * nk, i1 = i0 + nk - 1;
    // the workgroup whose range holds iteration i: the last w with w I / G <= i
    const int w_lo = (int)(((i0 + 1) * G - 1) / I), w_hi = (int)(((i1 + 1) * G - 1) / I);
    const size_t off = (size_t)(m - tm * 256) * 256 + (size_t)(n - tn * 256);
    f32x4 lo = {0.0f, 0.0f, 0.0f, 0.0f}, hi = lo;
    for (int w = w_lo; w <= w_hi; ++w) {
        const int64_t bw = (int64_t)w * I / G, bw1 = (int64_t)(w + 1) * I / G;
        if (bw1 <= bw)
            continue;
        // the tile is the workgroup's first segment if its range starts inside the tile
        const float* p = W + (size_t)(2 * w + (bw >= i0 ? 0 : 1)) * 65536 + off;
        lo += *reinterpret_cast<const f32x4*>(p);
        hi += *reinterpret_cast<const f32x4*>(p + 4);
    }
    u32x4 v;
    v[0] = pack2<DT>(lo[0], lo[1]);
    v[1] = pack2<DT>(lo[2], lo[3]);
    v[2] = pack2<DT>(hi[0], hi[1]);
    v[3] = pack2<DT>(hi[2], hi[3]);
    *reinterpret_cast<u32x4*>(C + (size_t)m * ldc + n) = v;
}

// ------------------------------------------------------------------------------------
// Ping-pong kernel.
//   8 waves, two per SIMD, in two groups: group 0 (waves 0-3) owns C rows [0, BM/2) of the
//   tile, group 1 (waves 4-7) rows [BM/2, BM); inside a group wave c owns a BN/4-wide
//   column block, so each wave holds a (BM/2) x (BN/4) block of accumulators.  Waves w
//   and w+4 share a SIMD.  Each wave alternates a memory phase (read all MFMA operands of
//   one K step from LDS; issue direct-to-LDS loads) and a compute phase (the K step's
//   MFMAs back to back, at raised issue priority), and the two groups run half a period
//   apart, so on every SIMD one wave feeds the matrix core while the other fetches.
//   Phases end at workgroup barriers:
//     phase 2t   : group 0 reads tile t,   group 1 computes tile t-1
//     phase 2t+1 : group 0 computes tile t, group 1 reads tile t
//   Tiles rotate through STAGES LDS stages.  A rows [0, BM/2) of a tile are read only by
//   group 0 (in phase 2t), so they are free one phase earlier than the rest: group 1
//   loads them for tile t+STAGES in its memory phase 2t+1; group 0 loads A rows
//   [BM/2, BM) and B of tile t+STAGES in its memory phase 2t+2.  No loads are issued in
//   compute phases.  Each wave waits for its own part of tile t+1 before the barrier
//   that ends phase 2t+1, so a load has 2*STAGES-2 phases to land; with BK = 32 the
//   phases are half as long and the ring twice as deep (4-5 stages in 160 KiB), which
//   hides a longer memory latency at the cost of twice as many barriers.
// ------------------------------------------------------------------------------------
template <int DT, int ALAYOUT, int LAYOUT, int BM, int BN, int BK, int STAGES>
__global__ void __attribute__((amdgpu_flat_work_group_size(512, 512),
                               amdgpu_waves_per_eu(2, 2)))
gemm_pingpong(const u16* __restrict__ A, const u16* __restrict__ B, u16* __restrict__ C, int M,
              int N, int K, int lda, int ldb, int ldc, int grid_m, int grid_n, int group_m) {
    constexpr int KC = BK / 8;
    constexpr int WTM = BM / 2, WTN = BN / 4;     // one wave's block of C
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int KS = BK / 16;
    constexpr int A_ELEMS = BM * BK;
    constexpr int STAGE = (BM + BN) * BK;
    constexpr int ROWS = 64 / KC;                  // tile rows per 1 KiB load
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave block must be whole 32x32 tiles");
    static_assert((BM / 8) % ROWS == 0 && (BN / 4) % ROWS == 0, "bad load split");
    static_assert(STAGES >= 2 && STAGES * STAGE * 2 <= 160 * 1024, "LDS");
    static_assert(LAYOUT == LAYOUT_NK || BN == 256, "B [K,N] path: 256 columns");
    static_assert(ALAYOUT == LAYOUT_MK || BM == 256, "A [K,M] path: 256 rows");

    __shared__ __attribute__((aligned(1024))) u16 lds[STAGES * STAGE];

    int tm, tn;
    tile_of((int)blockIdx.x, grid_m, grid_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = (int)threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, wc = wave & 3;
    const int nk = (K + BK - 1) / BK;

    const rsrc4_t ra = ALAYOUT == LAYOUT_MK ? make_rsrc4(A, span_bytes(M, K, lda))
                                            : make_rsrc4(A, span_bytes(K, M, lda));
    const rsrc4_t rb = LAYOUT == LAYOUT_NK ? make_rsrc4(B, span_bytes(N, K, ldb))
                                           : make_rsrc4(B, span_bytes(K, N, ldb));

    // The rows this wave loads: group 1 wave c the A rows [c*BM/8, (c+1)*BM/8); group 0
    // wave c the A rows [BM/2 + c*BM/8, ...) and the B rows [c*BN/4, (c+1)*BN/4).  They
    // come in 1 KiB blocks of ROWS consecutive rows; lane l lands in row l / KC of a
    // block at physical chunk l % KC and fetches the logical chunk the swizzle puts there,
    // which (blocks start at multiples of ROWS) depends only on the block's parity.
    constexpr int A_BLK = (BM / 8) / ROWS;         // A blocks per wave
    constexpr int B_BLK = (BN * BK / 512) / 4;     // B blocks (1 KiB) per group-0 wave
    static_assert(KC == 4 || KC == 8, "the swizzle repeats every two blocks for 4 or 8 chunks");
    const int prow = lane / KC;
    const int a_row = (grp ? 0 : BM / 2) + wc * (BM / 8);   // first A row of this wave
    const int b_row = wc * (BN / 4);                          // first B row (group 0)
    const int kc_even = ((lane % KC) ^ swz<KC>(prow)) * 8;
    const int kc_odd = ((lane % KC) ^ swz<KC>(ROWS + prow)) * 8;
    // A tile past the end is loaded as zeros (every lane out of range) into a stage no
    // one reads again, which keeps the number of loads in flight static.
    // A [K,M] tiles are kept as two halves, rows [0, BM/2) and [BM/2, BM) of the tile,
    // each BK k rows of BM/2 columns (256-byte rows) with 16-byte chunks swizzled by
    // 4*(k % 4); group 1 loads the first half, group 0 the second, 4 k rows per load.
    constexpr int HALF = (BM / 2) * BK;
    const int a_half = grp ? 0 : 1;
    auto dma_a = [&](int kt, auto ic) {            // block i of this wave's A rows
        constexpr int i = decltype(ic)::value;
        const bool live = kt < nk;
        const int k0 = live ? kt * BK : 0;
        u16* st = lds + (kt % STAGES) * STAGE;
        if constexpr (ALAYOUT == LAYOUT_MK) {
            const int kc = (i & 1) ? kc_odd : kc_even;
            const int r = m0 + a_row + i * ROWS + prow;
            const bool ok = live && r < M && k0 + kc < K;
            dma16(ra, st + (a_row + i * ROWS) * BK,
                     ok ? (uint32_t)(r * lda + kc) * 2u : kOutOfRange, (uint32_t)k0 * 2u);
        } else {
            const int kr = wc * (BK / 4) + 4 * i + (lane >> 4);
            const int cl = (lane & 15) ^ (4 * (kr & 3));
            const int m = m0 + a_half * (BM / 2) + 8 * cl;
            const bool ok = live && m < M && k0 + kr < K;
            dma16(ra, st + a_half * HALF + (wc * (BK / 4) + 4 * i) * (BM / 2),
                     ok ? (uint32_t)(kr * lda + m) * 2u : kOutOfRange,
                     (uint32_t)k0 * (uint32_t)lda * 2u);
        }
    };
    // B [N,K]: the BN/4 rows of wave c's columns are read only by wave c of each group,
    // so each of the two waves loads half of them: group 0 the upper half in its memory
    // phase, group 1 the lower half in its own memory phase, once its reads of the stage
    // have completed.  B [K,N]: every k row holds all waves' columns, so group 0 loads
    // all of B.
    auto dma_b = [&](int kt, auto ic) {            // block i of this wave's B share
        constexpr int i = decltype(ic)::value;
        const bool live = kt < nk;
        const int k0 = live ? kt * BK : 0;
        u16* st = lds + (kt % STAGES) * STAGE;
        if constexpr (LAYOUT == LAYOUT_NK) {
            const int r0 = b_row + (grp == 0 ? B_BLK / 2 : 0) * ROWS;
            const int kc = (i & 1) ? kc_odd : kc_even;
            const int r = n0 + r0 + i * ROWS + prow;
            const bool ok = live && r < N && k0 + kc < K;
            dma16(rb, st + A_ELEMS + (r0 + i * ROWS) * BK,
                     ok ? (uint32_t)(r * ldb + kc) * 2u : kOutOfRange, (uint32_t)k0 * 2u);
        } else {
            // the stage holds k rows of BN columns; a 1 KiB load fills two rows, lane l
            // row l / 32 at physical chunk l % 32, fetching the logical chunk that the
            // row's swizzle (chunk ^ 4*(k % 4)) puts there.
            const int kr = wc * (BK / 4) + 2 * i + (lane >> 5);
            const int cl = (lane & 31) ^ (4 * (kr & 3));
            const int n = n0 + 8 * cl;
            const bool ok = live && n < N && k0 + kr < K;
            dma16(rb, st + A_ELEMS + (wc * (BK / 4) + 2 * i) * BN,
                     ok ? (uint32_t)(kr * ldb + n) * 2u : kOutOfRange,
                     (uint32_t)k0 * (uint32_t)ldb * 2u);
        }
    };
    static_assert(B_BLK % 2 == 0 && (B_BLK / 2) % 2 == 0, "B halves keep the block parity");
    constexpr bool SPLIT_B = LAYOUT == LAYOUT_NK;
    constexpr int B0 = SPLIT_B ? B_BLK / 2 : B_BLK;   // B blocks per group-0 wave
    constexpr int B1 = SPLIT_B ? B_BLK / 2 : 0;       // B blocks per group-1 wave
    constexpr int LD0 = A_BLK + B0, LD1 = A_BLK + B1; // loads per wave per tile
    // load q of a group's share of tile kt: its A blocks, then its B blocks
    auto load_q = [&](int kt, auto qc) {
        constexpr int q = decltype(qc)::value;
        if constexpr (q < A_BLK)
            dma_a(kt, std::integral_constant<int, q>{});
        else
            dma_b(kt, std::integral_constant<int, q - A_BLK>{});
    };


    const int xr = swz<KC>(lane & 31);
    const int half = lane >> 5;
    const int a_row0 = (grp * WTM + (lane & 31)) * BK;
    const int b_row0 = A_ELEMS + (wc * WTN + (lane & 31)) * BK;
    // B [K,N] operands come from two transposing reads (ds_read_b64_tr_b16): in each
    // 16-lane group, lane s points at the 4 columns [4(s%4), 4(s%4)+4) of k row s/4 of a
    // 4 x 16 block, and lane i receives column i of those 4 rows; lane groups 0/1 cover
    // columns 0-15/16-31 and groups 2/3 the same for the upper 8 k, so two reads (k and
    // k+4) give each lane its column's 8 consecutive k in MFMA operand order.
    // The same reads serve an A [K,M] half (rows of BM/2 columns).
    int kn_base[TN], km_base[TM];
    {
        const int g = lane >> 4, sl = lane & 15;
        const int kl = 8 * (g >> 1) + (sl >> 2);
        if constexpr (LAYOUT == LAYOUT_KN) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n = wc * WTN + 32 * j + 16 * (g & 1) + 4 * (sl & 3);
                kn_base[j] = A_ELEMS + kl * BN + (((n >> 3) ^ (4 * (kl & 3))) << 3) + (n & 7);
            }
        }
        if constexpr (ALAYOUT == LAYOUT_KM) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int m = 32 * i + 16 * (g & 1) + 4 * (sl & 3);   // inside the half
                km_base[i] = grp * HALF + kl * (BM / 2) +
                             (((m >> 3) ^ (4 * (kl & 3))) << 3) + (m & 7);
            }
        }
    }
    // two transposing reads, k rows kr and kr + 4 (row length RL), as one MFMA operand
    auto read_tr = [&](const u16* p0, auto rlc) {
        constexpr int RL = decltype(rlc)::value;
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 4 * RL));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
    };
    u32x4 fa[KS][TM], fb[KS][TN];
    // Operand read r of tile kt: the B operands first (group 1 frees its B rows as soon
    // as they are read), then A.
    constexpr int NRB = KS * TN, NR = KS * (TN + TM);
    auto read_r = [&](int kt, auto rc) {
        constexpr int r = decltype(rc)::value;
        const u16* st = lds + (kt % STAGES) * STAGE;
        if constexpr (r < NRB) {
            constexpr int S = r / TN, j = r % TN;
            const int koff = (((2 * S) | half) ^ xr) * 8;
            if constexpr (LAYOUT == LAYOUT_NK) {
                fb[S][j] = *reinterpret_cast<const u32x4*>(st + b_row0 + j * 32 * BK + koff);
            } else {
                fb[S][j] = read_tr(st + kn_base[j] + (16 * S) * BN,
                                   std::integral_constant<int, BN>{});
            }
        } else {
            constexpr int S = (r - NRB) / TM, i = (r - NRB) % TM;
            if constexpr (ALAYOUT == LAYOUT_MK) {
                const int koff = (((2 * S) | half) ^ xr) * 8;
                fa[S][i] = *reinterpret_cast<const u32x4*>(st + a_row0 + i * 32 * BK + koff);
            } else {
                fa[S][i] = read_tr(st + km_base[i] + (16 * S) * (BM / 2),
                                   std::integral_constant<int, BM / 2>{});
            }
        }
    };
    // A memory phase: the operand reads of tile kt with the first NL loads of this
    // group's share of tile lt spread evenly among them (load q goes before read
    // q * NR / NL), so the load path and the LDS work side by side.
    auto mem_phase = [&](int kt, int lt, auto nlc) {
        constexpr int NL = decltype(nlc)::value;
        static_for<0, NR>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            static_for<0, NL>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                if constexpr (q * NR / NL == r) {
                    load_q(lt, qc);
                    __builtin_amdgcn_sched_barrier(0);
                }
            });
            read_r(kt, rc);
        });
        __builtin_amdgcn_sched_barrier(0);
    };
    // LDS reads a wave issues per tile for the A operands, capped at the 15 the counter
    // can name: LDS instructions complete in order, so once at most this many are
    // outstanding the B reads (issued first) are done
    constexpr int A_READS = KS * TM < 15 ? KS * TM : 15;

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

    if (nk > 0) {
        // Group 1 loads the A rows [0, BM/2) of tile kt + STAGES in its memory phase
        // 2kt+1 (group 0 finished reading them in phase 2kt); group 0 loads the rest of
        // tile kt + STAGES - 1 in its memory phase 2kt (group 1 finished reading that
        // stage in phase 2kt-1).  Before the loop: the first STAGES (group 1) or
        // STAGES - 1 (group 0) tiles.
        for (int u = 0; u < STAGES - (grp == 0 ? 1 : 0); ++u) {
            if (grp == 0) {
                static_for<0, LD0>([&](auto qc) { load_q(u, qc); });
            } else {
                static_for<0, LD1>([&](auto qc) { load_q(u, qc); });
            }
        }
        if (grp == 0)
            wait_vm<(STAGES - 2) * LD0>();         // tile 0 landed (this wave's part)
        else
            wait_vm<(STAGES - 1) * LD1>();
        wait_lgkm_sync();                          // end of phase -1
        if (grp == 1)
            wait_lgkm_sync();                      // group 1 sits out phase 0
        for (int kt = 0; kt < nk; ++kt) {
            // memory phase (2kt for group 0, 2kt+1 for group 1): this group's loads of
            // the next free stage part (loads first: they have the longest way to go),
            // then the operands of tile kt
            if (grp == 0) {
                mem_phase(kt, kt + STAGES - 1, std::integral_constant<int, LD0>{});
                wait_lgkm_sync();                  // end of phase 2kt
            } else {
                mem_phase(kt, kt + STAGES, std::integral_constant<int, A_BLK>{});
                if constexpr (SPLIT_B) {
                    wait_lgkm<A_READS>();          // this wave's B reads of tile kt done
                    static_for<0, B1>([&](auto qc) {
                        dma_b(kt + STAGES, qc);
                    });
                }
                wait_vm<(STAGES - 1) * LD1>();     // tile kt+1 landed (this wave's part)
                wait_lgkm_sync();                  // end of phase 2kt+1
            }
            // compute phase: the K step's MFMAs back to back
            __builtin_amdgcn_s_setprio(1);
            static_for<0, KS * TM * TN>([&](auto qc) {
                constexpr int Q = decltype(qc)::value;
                constexpr int S = Q / (TM * TN), i = (Q / TN) % TM, j = Q % TN;
                acc[i][j] = mfma_32x32x16<DT>(fb[S][j], fa[S][i], acc[i][j]);
            });
            __builtin_amdgcn_s_setprio(0);
            if (grp == 0) {
                wait_vm<(STAGES - 2) * LD0>();     // tile kt+1 landed (this wave's part)
                wait_lgkm_sync();                  // end of phase 2kt+1
            } else if (kt + 1 < nk) {
                wait_lgkm_sync();                  // end of phase 2kt+2
            }
        }
        wait_vm<0>();                              // the trailing zero loads
    }

    // Epilogue: one cast per value, staged through LDS into whole row segments (see
    // store_c_staged); the ring is free once every wave has read its last operands.
    __syncthreads();
    store_c_staged<DT, WTM, WTN, 8, STAGES * STAGE>(acc, lds, wave, lane, C, M, N, ldc,
                                                    m0 + grp * WTM, n0 + wc * WTN);
}

// Direct-to-LDS load into the 1 KiB block OFF bytes past M0.  The instruction offset is
// added to the global address as well, so the caller's offset is OFF lower than the
// element's.  NOP: an s_nop first (M0 was written by the instruction before).  STEP: M0
// moves on by 4 KiB after the load (the instruction offset reaches 3 KiB at most).
template <int POL, int OFF, bool NOP, bool STEP>
__device__ __forceinline__ void dma16_off(rsrc4_t r, uint32_t voff, uint32_t soff) {
    static_assert(OFF >= 0 && OFF < 4096, "12-bit instruction offset");
    const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
    static_assert(POL == 0 || POL == 2, "default or sc0 policy");
    if constexpr (POL == 2) {
        if constexpr (NOP && STEP)
            asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen offset:%3 sc0 lds\n\ts_add_u32 m0, m0, 0x1000"
                         ::"v"(voff), "s"(r), "s"(so), "i"(OFF) : "memory", "m0", "scc");
        else if constexpr (NOP)
            asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen offset:%3 sc0 lds"
                         ::"v"(voff), "s"(r), "s"(so), "i"(OFF) : "memory");
        else if constexpr (STEP)
            asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:%3 sc0 lds\n\ts_add_u32 m0, m0, 0x1000"
                         ::"v"(voff), "s"(r), "s"(so), "i"(OFF) : "memory", "m0", "scc");
        else
            asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:%3 sc0 lds"
                         ::"v"(voff), "s"(r), "s"(so), "i"(OFF) : "memory");
    } else {
        if constexpr (NOP && STEP)
            asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen offset:%3 lds\n\ts_add_u32 m0, m0, 0x1000"
                         ::"v"(voff), "s"(r), "s"(so), "i"(OFF) : "memory", "m0", "scc");
        else if constexpr (NOP)
            asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen offset:%3 lds"
                         ::"v"(voff), "s"(r), "s"(so), "i"(OFF) : "memory");
        else if constexpr (STEP)
            asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:%3 lds\n\ts_add_u32 m0, m0, 0x1000"
                         ::"v"(voff), "s"(r), "s"(so), "i"(OFF) : "memory", "m0", "scc");
        else
            asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:%3 lds"
                         ::"v"(voff), "s"(r), "s"(so), "i"(OFF) : "memory");
    }
}

// ------------------------------------------------------------------------------------
// Quadrant kernel (A [M,K]; B [N,K], or B [K,N] with LAYOUT_KN).
//   One wave per SIMD: 4 waves in 2 x 2, each owning a 128 x 128 quadrant of the
//   256 x 256 tile with all of its accumulators in registers (BMT = 192: a 192 x 256
//   tile of 96 x 128 quadrants, for grids that 256-row tiles leave short of the compute
//   units; its A slots hold 192 rows, each wave loading 48 of them in 6 loads).  A
//   stored [K,M] (ALAY = LAYOUT_KM, 256-row tiles): A slots of 64 k rows of 256 columns,
//   loaded and read exactly as B [K,N] below (k rows, the same swizzle, transposing
//   reads), the A operand of a lane being 8 consecutive k of one row m.  Per MFMA this reads a
//   third fewer operand bytes from LDS than 8 waves of 128 x 64 (4 x 256 instead of
//   8 x 192 tile rows per K step).  MF picks the matrix instruction: 16 (16x16x32,
//   8 x 8 blocks per wave) or 32 (32x32x16, 4 x 4 blocks per wave).
//   Tiles of BK = 64 k (128-byte row segments: every load request is a whole cache
//   line) arrive by direct-to-LDS loads; wave w loads rows [64w, 64w + 64) of each
//   operand tile, 8 loads per operand.  The 160 KiB of LDS hold three A slots and two B
//   slots (32 KiB each), so the A part of a tile can be fetched a step earlier than
//   the B part and the two halves of a tile's loads go out in different halves of a
//   step: the load stream stays even instead of leaving each barrier in one burst.
// Step t computes tile t in KS sub-steps (BK / k per MFMA).  Each sub-step's MFMAs run
// back to back with its memory operations dealt out among them:
//   sub-steps s < KS-1 : the operand reads of sub-step s+1 (registers double-buffered),
//                        and the A loads of tile t+2 (its slot held tile t-1);
//   sub-step KS-1      : after PRE MFMAs, each wave waits for its own loads of tile t+1
//                        and meets the others at the step's one barrier (tile t+1 is
//                        then in LDS and every wave has read all of tile t), then the
//                        reads of tile t+1's first operands and the B loads of tile t+2
//                        into the B slot tile t used.
// An A load has a step and a half to land, a B load one step.  The K walk takes the
// tail tile (the last K % 64 columns, masked) first, then the whole tiles; loads past
// the end of the walk continue it into a slot no step reads, so every step has the same
// number of loads in flight.  STAG starts the whole-tile walk of the workgroups of XCD x
// at x/8 of K (wrapping), so that the eight XCDs do not stream the same addresses at
// once; POL is the cache policy of the loads; OFFS places each load's 1 KiB LDS block
// by its instruction offset (one M0 update per four loads).  The steps run as
// (tiles mod 6) single steps, then groups of six with constant ring slots (3 A slots,
// 2 B slots), so a grouped step's LDS addresses are constant offsets and no scalar
// bookkeeping sits between two steps' MFMAs.
// B [K,N] ("TileLang: a tile language one level below Triton", section "The first kernel:
// GEMM": B given as a (K, N) tensor): a B slot holds the tile's 64 k rows of 256 columns
// (512 bytes each), filled by the same 1 KiB direct-to-LDS loads (two k rows per load,
// wave w the rows [16w, 16w + 16)).  The 16-byte chunk holding column n of row k sits at
// chunk (n / 8) ^ kn_swz(k) (below).  The MFMA operand of a lane (8
// consecutive k of one column) comes from two transposing reads (ds_read_b64_tr_b16): in
// each 16-lane group, lane s points at 4 columns of k row s / 4 of a 4 x 16 block and
// receives its column's 4 values.  A wave's read covers the rows k0 + 8g + (0..3) of lane
// group g for 16 columns (32x32x16: rows k0 + 8(g/2) + (0..3), 16 columns per group):
// with the swizzle the 8 row pieces that lanes 0-31 read together land in 8 different
// 32-byte bank slots, as do those of lanes 32-63.  With B [K,N] the two B slots come
// first in LDS.
// ------------------------------------------------------------------------------------
template <int NOPS, int SLOTS, int J>
struct deal {   // ops [lo, hi) follow slot J when NOPS ops are dealt over SLOTS slots
    static constexpr int lo = J >= SLOTS ? NOPS : (J * NOPS + SLOTS - 1) / SLOTS;
    static constexpr int hi = J >= SLOTS ? NOPS : ((J + 1) * NOPS + SLOTS - 1) / SLOTS;
};
// Op o of a sequence of NL loads and NR reads with the loads spaced evenly among the
// reads: the load index, or -1 - (read index).
template <int NL, int NR>
constexpr int op_kind(int o) {
    int loads = 0;
    for (int p = 0; p <= o; ++p) {
        const bool is_load = loads < NL && p == loads * (NL + NR) / (NL > 0 ? NL : 1);
        if (p == o)
            return is_load ? loads : -1 - (o - loads);
        loads += is_load;
    }
    return 0;
}

// Chunk swizzle of row k of a B [K,N] slot (see above): for 16x16x32 operands the rows
// read together are k0 + (0..3) and k0 + 8 + (0..3) at the same 16 columns; for
// 32x32x16 operands k0 + (0..3) at 32 columns.
template <int MF>
__device__ __forceinline__ int kn_swz(int k) {
    return MF == 16 ? 2 * ((k & 3) + 4 * ((k >> 3) & 1)) : 4 * (k & 3);
}

// The body of the quad kernels: C tile (tm, tn).  MODE 0: the whole K walk, cast to C.
// MODE 1 (partial): the K range [k0, k0 + klen) only (k0 a multiple of 64) and the fp32
// partial tile stored to P, element (m, n) at P[(m - pm0) * ldp + (n - pn0)], instead of
// the cast to C.  MODE 2: MODE 1 where `partial` holds, else MODE 0 (one body, so one LDS
// ring, for a kernel that does both).
template <int DT, int MF, int PRE, int SPA, int SPB, int STAG, int POL, bool OFFS, int LAYOUT,
          int BMT, int ALAY, int MODE>
__device__ __attribute__((always_inline)) inline void
quad_body(const u16* __restrict__ A, const u16* __restrict__ B, u16* __restrict__ C, int M,
          int N, int K, int lda, int ldb, int ldc, int tm, int tn, int k0, int klen,
          float* __restrict__ P, int ldp, int pm0, int pn0, bool partial = false) {
    constexpr int BM = BMT, BN = 256, BK = 64;
    constexpr int KC = BK / 8;                 // 16-byte chunks per tile row
    constexpr int ROWS = 64 / KC;              // tile rows per 1 KiB load (8)
    constexpr int SLOTA = BM * BK;             // elements of one A slot (32 or 24 KiB)
    constexpr int SLOTB = BN * BK;             // elements of one B slot (32 KiB)
    constexpr int SA = 3, SB = 2;              // A and B slots
    constexpr int NBA = BM / 4 / ROWS;         // A loads per wave per tile (8 or 6)
    constexpr int NBB = 64 / ROWS;             // B loads per wave per tile (8)
    constexpr int KM = MF == 16 ? 32 : 16;     // k per MFMA
    constexpr int KS = BK / KM;                // sub-steps per tile
    constexpr int CPS = KM / 8;                // 16-byte chunks per sub-step
    constexpr int WTM = BM / 2;                // a wave's rows of C (128 or 96)
    constexpr int TM = WTM / MF, TN = 128 / MF;
    constexpr int NR = TM + TN;                // operand reads per sub-step
    constexpr int NM = TM * TN;                // MFMAs per sub-step
    using acc_t = std::conditional_t<MF == 16, f32x4, f32x16>;
    static_assert(MF == 16 || MF == 32, "MFMA 16x16x32 or 32x32x16");
    static_assert(KS % 2 == 0, "every step starts from operand buffer 0");
    static_assert(BM == 256 || BM == 192, "256 or 192 tile rows");
    static_assert(WTM % MF == 0 && NBA % 2 == 0, "whole MFMA blocks, block pairs");
    static_assert((SA * SLOTA + SB * SLOTB) * 2 <= 160 * 1024, "LDS");
    static_assert(PRE >= 1 && PRE < NM && SPA >= 1 && SPB >= 1, "schedule");
    constexpr bool KN = LAYOUT == LAYOUT_KN;
    constexpr bool AKM = ALAY == LAYOUT_KM;    // A stored [K,M]: A slots of k rows, like B [K,N]
    static_assert(!AKM || BM == 256, "A [K,M]: 256-row tiles (512-byte k rows)");
    // Two loads of one operand can be adjacent (no instruction between them) when the A
    // loads outnumber their MFMA slots, or the B loads outnumber the reads dealt between.
    constexpr bool TIGHT = NBA > (SPA < (KS - 1) * NM ? SPA : (KS - 1) * NM) || NR < NBB;

    __shared__ __attribute__((aligned(1024))) u16 lds[SA * SLOTA + SB * SLOTB];

    static_assert(MODE >= 0 && MODE <= 2, "mode");
    const bool part = MODE == 1 || (MODE == 2 && partial);
    if (MODE != 0 && part) {
        // the K range as a product of its own: the operands start at its first k, and K
        // is its length (a last range may hold a partial tile, or nothing)
        K = klen > 0 ? klen : 0;
        A += AKM ? (size_t)k0 * (size_t)lda : (size_t)k0;
        B += KN ? (size_t)k0 * (size_t)ldb : (size_t)k0;
    }

    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = (int)threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int nk = (K + BK - 1) / BK;

    const rsrc4_t ra = AKM ? make_rsrc4(A, span_bytes(K, M, lda))
                           : make_rsrc4(A, span_bytes(M, K, lda));
    const rsrc4_t rb = KN ? make_rsrc4(B, span_bytes(K, N, ldb))
                          : make_rsrc4(B, span_bytes(N, K, ldb));

    // Lane l lands in row r0 + b*ROWS (r0 = 64w + l/KC) of block b at physical chunk
    // l % KC and fetches the logical chunk that the row's swizzle puts there (the swizzle
    // repeats every 16 rows, i.e. every two blocks).  The byte offset of each block's row
    // and chunk is computed once, out-of-range for rows past M (A) or N (B); a load adds
    // the K position of its tile as the scalar offset.  B [K,N]: lane l of load b lands in
    // k row 16w + 2b + l/32 at physical chunk l % 32, out-of-range for columns past N.
    const int prow = lane / KC, pch = lane % KC;
    const int r0 = (BM / 4) * wave + prow;     // A rows of block 0 of this wave
    const int rb0 = 64 * wave + prow;          // B [N,K] rows of block 0
    int kcol[2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
        kcol[p] = (pch ^ swz<KC>(p * ROWS + prow)) * 8;
    // With OFFS the 1 KiB LDS block of load b comes from the instruction offset
    // (b % 4) KiB, M0 moving on by 4 KiB after the fourth load: one M0 update per four
    // loads instead of one per load.  The offset adds to the global address as well, so
    // the stored offsets are that much lower; rows b * ROWS >= 8 apart keep them
    // non-negative when lda, ldb >= 64 (the launcher's condition for OFFS); with B [K,N],
    // whose rows of load b are 2b apart, when ldb >= 256.
    uint32_t a_vo[NBA], b_vo[NBB];
    auto kn_row = [&](int b) { return 16 * wave + 2 * b + (lane >> 5); };
    auto set_offsets = [&]() {
#pragma unroll
        for (int b = 0; b < NBA; ++b) {
            const int ra = m0 + r0 + b * ROWS;
            const uint32_t lo = OFFS ? (uint32_t)(b & 3) * 1024u : 0u;
            if constexpr (AKM) {
                const int kr = kn_row(b);
                const int m = m0 + 8 * ((lane & 31) ^ kn_swz<MF>(kr));
                a_vo[b] = m < M ? (uint32_t)(kr * lda + m) * 2u - lo : kOutOfRange;
            } else {
                a_vo[b] = ra < M ? (uint32_t)(ra * lda + kcol[b & 1]) * 2u - lo : kOutOfRange;
            }
        }
#pragma unroll
        for (int b = 0; b < NBB; ++b) {
            const int rbn = n0 + rb0 + b * ROWS;
            const uint32_t lo = OFFS ? (uint32_t)(b & 3) * 1024u : 0u;
            if constexpr (KN) {
                const int kr = kn_row(b);
                const int n = n0 + 8 * ((lane & 31) ^ kn_swz<MF>(kr));
                b_vo[b] = n < N ? (uint32_t)(kr * ldb + n) * 2u - lo : kOutOfRange;
            } else {
                b_vo[b] = rbn < N ? (uint32_t)(rbn * ldb + kcol[b & 1]) * 2u - lo : kOutOfRange;
            }
        }
    };
    set_offsets();
    // The K walk: the tail tile holding the last K % BK columns first, if any (its loads
    // go out before the loop, the only masked ones), then the whole tiles, starting kofs
    // tiles in (XCD x starts x/8 of the way along) and wrapping.  Loads past the end of
    // the walk are never read; they continue the wrap (any valid tile would do).
    const int nfull = K / BK;
    const bool tail = nfull < nk;
    const int toff = tail ? 1 : 0;
    const int kofs = STAG ? (((int)blockIdx.x & 7) * nfull) >> 3 : 0;
    const uint32_t lds0 = lds_addr(lds);
    // the wave's first 1 KiB block in an A slot and in a B slot
    const uint32_t wave_a_at = (uint32_t)((BM / 4) * wave * BK * 2);
    const uint32_t wave_b_at = (uint32_t)(64 * wave * BK * 2);
    // index among the whole tiles of walk step u >= toff
    auto full_index = [&](int u) { return nfull > 0 ? (u - toff + kofs) % nfull : 0; };
    // For the tail tile's loads: chunks past K (B [K,N]: k rows past K) get out-of-range
    // offsets (zeros), in place (set_offsets restores them afterwards).
    auto mask_tail = [&]() {
        const int rem = K - nfull * BK;
        const bool ok0 = kcol[0] < rem, ok1 = kcol[1] < rem;
#pragma unroll
        for (int b = 0; b < NBA; ++b) {
            if constexpr (AKM)
                a_vo[b] = kn_row(b) < rem ? a_vo[b] : kOutOfRange;
            else
                a_vo[b] = ((b & 1) ? ok1 : ok0) ? a_vo[b] : kOutOfRange;
        }
#pragma unroll
        for (int b = 0; b < NBB; ++b) {
            const bool ok = (b & 1) ? ok1 : ok0;
            if constexpr (KN)
                b_vo[b] = kn_row(b) < rem ? b_vo[b] : kOutOfRange;
            else
                b_vo[b] = ok ? b_vo[b] : kOutOfRange;
        }
    };
    // Load b (< NBA or NBB) of operand A (is_a) or B of the tile at K position k0, into the 1 KiB
    // block M0 points at (the loads of one operand's tile go out in block order, M0 set to
    // the wave's first block beforehand).  The K position goes in the scalar offset: k0
    // elements along a row ([M,K] and [N,K] operands) or k0 rows of ldb elements (B [K,N]).
    auto load_b = [&](int k0, auto isac, auto bc, auto nopc) {
        constexpr bool is_a = decltype(isac)::value;
        constexpr int b = decltype(bc)::value;
        constexpr bool back_to_back = decltype(nopc)::value;   // no instruction between loads
        constexpr int NBX = is_a ? NBA : NBB;
        const uint32_t soff = (!is_a && KN) ? (uint32_t)k0 * (uint32_t)ldb * 2u
                              : (is_a && AKM) ? (uint32_t)k0 * (uint32_t)lda * 2u
                                              : (uint32_t)k0 * 2u;
        static_assert(b < NBX, "block of the operand's tile");
        uint32_t vo;
        if constexpr (is_a)
            vo = a_vo[b];
        else
            vo = b_vo[b];
        if constexpr (OFFS) {
            // an s_nop after an M0 write: before block 0 of a back-to-back run (M0 was just
            // set), and before block 4 when it may directly follow block 3's M0 step
            constexpr bool nop = back_to_back ? (b & 3) == 0 : (b == 4 && TIGHT);
            dma16_off<POL, (b & 3) * 1024, nop, (b & 3) == 3 && b + 1 < NBX>(
                is_a ? ra : rb, vo, soff);
        } else {
            dma16_next<POL, back_to_back>(is_a ? ra : rb, vo, soff);
        }
    };
    // Slot order in LDS: A slots then B slots; with B [K,N] the B slots come first, so
    // that a transposing read's slot, sub-step and second-read offsets fit the 16-bit
    // offset field on one base register per column block.  a_at / b_at: a slot's first
    // element.
    auto a_at = [&](auto i) { return (KN ? SB * SLOTB : 0) + i * SLOTA; };
    auto b_at = [&](auto j) { return (KN ? 0 : SA * SLOTA) + j * SLOTB; };
    // M0 for the wave's first block of A slot i or B slot j, from bases kept in scalar
    // registers
    const uint32_t m0_a = __builtin_amdgcn_readfirstlane(lds0 + wave_a_at);
    const uint32_t m0_b = __builtin_amdgcn_readfirstlane(lds0 + wave_b_at);
    auto m0_of_a = [&](auto i) { return m0_a + (uint32_t)(a_at(i) * 2); };
    auto m0_of_b = [&](auto j) { return m0_b + (uint32_t)(b_at(j) * 2); };

    // Operand reads: lane l takes row l % MF of an MFMA block, 16-byte chunk
    // s * CPS + l / MF of the sub-step (the swizzle of its row depends on l % 16 only).
    const int lr = lane % MF, kq = lane / MF;
    const int xr = swz<KC>(lr);
    const int a_row0 = (wm * WTM + lr) * BK;
    const int b_row0 = (wn * 128 + lr) * BK;
    // B [K,N]: lane s of 16-lane group g reads 4 columns of one k row of the sub-step
    // (and, in the second read, the row 4 on).  16x16x32: row 8g + s/4, columns
    // 16j + 4(s%4) of the wave's 128; 32x32x16: row 8(g/2) + s/4, columns
    // 32j + 16(g%2) + 4(s%4).  The row's swizzle is the lane's own, so block j sits at a
    // lane-dependent place: one element offset per block; the slot, the sub-step and the
    // second read add constants.
    // The element offset of block j of a [K, 256] slot for the wave half h (wn or wm).
    auto tr_off = [&](int j, int h) {
        const int g = lane >> 4, sl = lane & 15;
        if constexpr (MF == 16) {
            const int p = (sl >> 2) + 4 * (g & 1);
            return (8 * g + (sl >> 2)) * 256 +
                   (16 * h + 2 * (j ^ p) + ((sl & 3) >> 1)) * 8 + 4 * (sl & 1);
        } else {
            const int q = sl >> 2;
            return (8 * (g >> 1) + q) * 256 +
                   (16 * h + 4 * (j ^ q) + 2 * (g & 1) + ((sl & 3) >> 1)) * 8 + 4 * (sl & 1);
        }
    };
    int kn_off[KN ? TN : 1], km_off[AKM ? TM : 1];
    if constexpr (KN) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
            kn_off[j] = tr_off(j, wn);
    }
    if constexpr (AKM) {               // A [K,M]: the same reads over the wave's rows
#pragma unroll
        for (int i = 0; i < TM; ++i)
            km_off[i] = tr_off(i, wm);
    }
    // two transposing reads (k rows and 4 rows on) of a [K, 256] slot, one MFMA operand
    auto read_tr = [&](const u16* p0) {
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 4 * 256));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
    };
    u32x4 fa[2][TM], fb[2][TN];
    auto read_r = [&](const u16* as, const u16* bs, auto sc, auto bufc, auto rc) {
        constexpr int s = decltype(sc)::value;
        constexpr int bf = decltype(bufc)::value;
        constexpr int r = decltype(rc)::value;
        const int koff = ((s * CPS + kq) ^ xr) * 8;
        if constexpr (r < TN) {
            if constexpr (KN)
                fb[bf][r] = read_tr(bs + kn_off[r] + s * KM * BN);
            else
                fb[bf][r] = *reinterpret_cast<const u32x4*>(bs + b_row0 + r * MF * BK + koff);
        } else {
            if constexpr (AKM)
                fa[bf][r - TN] = read_tr(as + km_off[r - TN] + s * KM * BM);
            else
                fa[bf][r - TN] =
                    *reinterpret_cast<const u32x4*>(as + a_row0 + (r - TN) * MF * BK + koff);
        }
    };

    acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = acc_t{};
    // MFMA J of a sub-step from operand buffer bf.  S0 = B rows (n), S1 = A rows (m): a
    // lane then holds one C row and groups of four consecutive columns.  The blocks go
    // row by row, every other row backwards, so that two consecutive MFMAs always share
    // an operand (the A block along a row, the B block at a turn): fewer operand
    // transitions cost less energy on this power-limited chip (measured 0.7-0.8 % faster
    // at 4096^3 and 8192^3, both B storages; columns outermost was 1.8 % slower).
    auto mma = [&](auto bufc, auto jc) {
        constexpr int bf = decltype(bufc)::value;
        constexpr int J = decltype(jc)::value;
        constexpr int i = J / TN, j = (i & 1) ? TN - 1 - J % TN : J % TN;
        if constexpr (MF == 16)
            acc[i][j] = mfma_16x16x32<DT>(fb[bf][j], fa[bf][i], acc[i][j]);
        else
            acc[i][j] = mfma_32x32x16<DT>(fb[bf][j], fa[bf][i], acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);
    };

    // One step: tile t from A slot ia and B slot jb; tile t+1 lies in A slot ia1 and
    // B slot jb1 (= the other B slot); A slot ia2 takes tile t+2, whose K position (in
    // bytes) is k2.  The slots come as ints or as integral constants (then every LDS
    // address of the step is a constant offset).  In a slot without memory operations the
    // step advances the walk: kk, and k2n, the K position of the next step's loads.
    uint32_t kwalk = 0;                // K position (bytes) of the next step's loads
    const uint32_t kwrap = (uint32_t)nfull * (uint32_t)(BK * 2);
    auto step = [&](auto ia, auto ia1, auto ia2, auto jb, auto jb1)
                    __attribute__((always_inline)) {
        const u16* as = lds + a_at(ia);
        const u16* bs = lds + b_at(jb);
        const u16* as1 = lds + a_at(ia1);
        const u16* bs1 = lds + b_at(jb1);
        const uint32_t k2b = kwalk;                   // this step loads tile t+2 from here
        const int k2i = (int)(k2b / 2u);              // load_b takes elements
        static_for<0, KS>([&](auto subc) {
            constexpr int s = decltype(subc)::value;
            constexpr int cb = s & 1, nb = cb ^ 1;
            constexpr bool last = s + 1 == KS;
            constexpr int J0 = last ? PRE : 0;
            // this sub-step's operands were read during the previous one: one wait for
            // all of them (lgkmcnt(0), vmcnt and expcnt left at their maxima) instead of
            // the compiler's wait before each first use
            __builtin_amdgcn_s_waitcnt(0xC07F);
            if constexpr (s == 0) {
                set_m0(m0_of_a(ia2));               // the A loads of tile t+2
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (last) {
                static_for<0, PRE>([&](auto jc) { mma(std::integral_constant<int, cb>{}, jc); });
                wait_vm_then_sync<NBA>();      // tile t+1 landed; the A loads of t+2 may fly
                __builtin_amdgcn_sched_barrier(0);
                set_m0(m0_of_b(jb));                // the B loads of tile t+2
                __builtin_amdgcn_sched_barrier(0);
            }
            // the A loads of tile t+2 are dealt over the first SPA MFMA slots of the
            // sub-steps before the barrier, the reads (and, after the barrier, the B
            // loads of tile t+2) over the first SPB slots of each sub-step
            constexpr int PRE_SLOTS = (KS - 1) * NM;
            constexpr int SA_ = SPA < PRE_SLOTS ? SPA : PRE_SLOTS;
            constexpr int NL = last ? NBB : 0;
            constexpr int NOPS = NR + NL;
            constexpr int SS = SPB < NM - J0 ? SPB : NM - J0;
            static_for<J0, NM>([&](auto jc) {
                constexpr int J = decltype(jc)::value;
                mma(std::integral_constant<int, cb>{}, jc);
                if constexpr (!last) {
                    constexpr int G = s * NM + J;     // slot index over the pre-barrier sub-steps
                    static_for<deal<NBA, SA_, G>::lo, deal<NBA, SA_, G>::hi>([&](auto bc) {
                        load_b(k2i, std::true_type{}, bc, std::false_type{});
                        __builtin_amdgcn_sched_barrier(0);
                    });
                }
                if constexpr (s == 0 && J == NM - 4) {
                    kwalk += (uint32_t)(BK * 2);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if constexpr (s == 0 && J == NM - 3) {
                    kwalk = kwalk >= kwrap ? 0u : kwalk;
                    __builtin_amdgcn_sched_barrier(0);
                }
                static_for<deal<NOPS, SS, J - J0>::lo, deal<NOPS, SS, J - J0>::hi>(
                    [&](auto oc) {
                        constexpr int kind = op_kind<NL, NR>(decltype(oc)::value);
                        if constexpr (kind >= 0)
                            load_b(k2i, std::false_type{}, std::integral_constant<int, kind>{},
                                   std::false_type{});
                        else if constexpr (!last)
                            read_r(as, bs, std::integral_constant<int, s + 1>{},
                                   std::integral_constant<int, nb>{},
                                   std::integral_constant<int, -1 - kind>{});
                        else
                            read_r(as1, bs1, std::integral_constant<int, 0>{},
                                   std::integral_constant<int, nb>{},
                                   std::integral_constant<int, -1 - kind>{});
                        __builtin_amdgcn_sched_barrier(0);
                    });
            });
        });
    };

    if (nk > 0) {
        // The steps run as nk % 6 single steps, then groups of six with constant slots
        // (the A ring has 3 slots, the B ring 2): tile 0 goes into the slots that make
        // the first group start at A slot 0 and B slot 0.
        const int rem = nk % 6;
        const int p0 = (6 - rem) % 6;              // ring phase of tile 0
        // tiles 0 and 1 (A then B each); step 0 issues the A loads of tile 2
        for (int u = 0; u < 2; ++u) {
            const bool tail_tile = tail && u == 0;
            if (tail_tile)
                mask_tail();
            const int ku = tail_tile ? nfull * BK : full_index(u) * BK;
            set_m0(m0_of_a((p0 + u) % SA));
            static_for<0, NBA>([&](auto bc) {
                load_b(ku, std::true_type{}, bc, std::true_type{});
            });
            set_m0(m0_of_b((p0 + u) % SB));
            static_for<0, NBB>([&](auto bc) {
                load_b(ku, std::false_type{}, bc, std::true_type{});
            });
            // with no whole tile the later loads keep the mask: they then never reach
            // past K, whatever the instruction offset adds
            if (tail_tile && nfull > 0)
                set_offsets();
        }
        wait_vm_then_sync<NBA + NBB>();           // tile 0 complete
        static_for<0, NR>([&](auto rc) {
            read_r(lds + a_at(p0 % SA), lds + b_at(p0 % SB),
                   std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, rc);
        });
        kwalk = (uint32_t)full_index(2) * (uint32_t)(BK * 2);
        for (int t = 0; t < rem; ++t) {
            const int p = p0 + t;                  // < 11
            const int ia = p % SA, jb = p % SB;
            const int ia1 = ia == SA - 1 ? 0 : ia + 1;
            const int ia2 = ia1 == SA - 1 ? 0 : ia1 + 1;
            step(ia, ia1, ia2, jb, jb ^ 1);
        }
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        for (int g = nk / 6; g > 0; --g) {
            step(I0{}, I1{}, I2{}, I0{}, I1{});
            step(I1{}, I2{}, I0{}, I1{}, I0{});
            step(I2{}, I0{}, I1{}, I0{}, I1{});
            step(I0{}, I1{}, I2{}, I1{}, I0{});
            step(I1{}, I2{}, I0{}, I0{}, I1{});
            step(I2{}, I0{}, I1{}, I1{}, I0{});
        }
        wait_vm<0>();                              // the trailing zero loads
    }

    if (MODE != 0 && part) {
        // The fp32 partial tile, straight from the accumulators: a lane's four
        // consecutive columns of one row are one 16-byte store (16 rows of 64 bytes per
        // instruction).
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int m = m0 + wm * WTM + i * MF + lr;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
#pragma unroll
                for (int g = 0; g < (MF == 16 ? 1 : 4); ++g) {
                    const int n = n0 + wn * 128 + j * MF + (MF == 16 ? 4 * kq : 8 * g + 4 * kq);
                    const f32x4 v = {acc[i][j][4 * g + 0], acc[i][j][4 * g + 1],
                                     acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                    if (m < M && n < N)
                        *reinterpret_cast<f32x4*>(P + (size_t)(m - pm0) * ldp + (n - pn0)) = v;
                }
            }
        }
        return;
    }

    // Epilogue: one cast per value.  A lane holds groups of four consecutive columns of a
    // row, which would leave each store as 16 scattered 32-byte pieces; instead each wave
    // stages its 128 x 128 block in LDS (the ring is free once every wave's loads have
    // landed and its reads are done) and stores it back as 256-byte row segments, 16
    // bytes per lane, with the non-temporal hint (1-2 % faster than plain stores; storing
    // straight from the accumulators instead was 3 % slower).  Rows are padded to 272
    // bytes, and in rows with bit 3 set the two 8-byte halves of each 16-byte chunk trade
    // places: the 8-byte writes of a lane's 16 rows then use 16 distinct bank pairs when
    // the LDS serves them 16 lanes at a time over 32 banks (rows r and r + 8 would share
    // them otherwise), and stay distinct when it serves 32 lanes over 64 banks.  The
    // reads swap the halves back in registers (the row's bit 3 is known at compile time).
    constexpr int RSE = 128 + 8;                   // staged row stride in elements
    static_assert(4 * WTM * RSE <= SA * SLOTA + SB * SLOTB, "C staging fits the LDS ring");
    wait_vm_then_sync<0>();
    u16* stage = lds + wave * WTM * RSE;
    // the lane's column within an 8-column run, halves traded in rows with bit 3 set
    // (bit 3 of a staged row i * MF + lr is bit 3 of lr); the rest is a constant offset
    const int cx = (4 * kq) ^ (4 * ((lr >> 3) & 1));
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int g = 0; g < (MF == 16 ? 1 : 4); ++g) {
                const int r = i * MF + lr;
                const int c = j * MF + (MF == 16 ? 0 : 8 * g) + cx;
                u32x2 v;
                v[0] = pack2<DT>(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
                v[1] = pack2<DT>(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
                *reinterpret_cast<u32x2*>(stage + r * RSE + c) = v;
            }
        }
    }
    // a wave's LDS accesses complete in order: its reads below see its writes above
    const int sr = lane >> 4, sc = (lane & 15) * 8;
    const int n = n0 + wn * 128 + sc;
#pragma unroll
    for (int q = 0; q < WTM / 4; ++q) {
        const int r = 4 * q + sr;                  // bit 3 of r is bit 1 of q (sr < 4)
        const u32x4 h = *reinterpret_cast<const u32x4*>(stage + r * RSE + sc);
        const u32x4 v = (q & 2) ? u32x4{h[2], h[3], h[0], h[1]} : h;
        const int m = m0 + wm * WTM + r;
        if (m < M && n < N)     // non-temporal: C is written once and not read back here
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(C + (size_t)m * ldc + n));
    }
}

template <int DT, int MF, int PRE, int SPA, int SPB, int STAG, int POL, bool OFFS,
          int LAYOUT = LAYOUT_NK, int BMT = 256, int ALAY = LAYOUT_MK>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256),
                               amdgpu_waves_per_eu(1, 1)))
gemm_quad(const u16* __restrict__ A, const u16* __restrict__ B, u16* __restrict__ C, int M,
          int N, int K, int lda, int ldb, int ldc, int grid_m, int grid_n, int group_m) {
    int tm, tn;
    tile_of((int)blockIdx.x, grid_m, grid_n, group_m, tm, tn);
    quad_body<DT, MF, PRE, SPA, SPB, STAG, POL, OFFS, LAYOUT, BMT, ALAY, 0>(
        A, B, C, M, N, K, lda, ldb, ldc, tm, tn, 0, 0, nullptr, 0, 0, 0);
}

// Split-K over workgroups with the quad kernel ("Tiling a matmul", section "Where it
// breaks": a grid of few tiles with a long K leaves compute units idle; splitting K
// gives them work): grid (tiles, splits), each workgroup one tile over one K range of
// kc, its fp32 partial tile to W[z]; splitk_reduce adds the planes in split order.
template <int DT, int MF, int PRE, int SPA, int SPB, int STAG, int POL, bool OFFS,
          int LAYOUT = LAYOUT_NK>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256),
                               amdgpu_waves_per_eu(1, 1)))
gemm_quad_split(const u16* __restrict__ A, const u16* __restrict__ B, int M, int N, int K,
                int lda, int ldb, int grid_m, int grid_n, int group_m, float* __restrict__ W,
                int kc) {
    int tm, tn;
    tile_of((int)blockIdx.x, grid_m, grid_n, group_m, tm, tn);
    const int z = (int)blockIdx.y, k0 = z * kc;
    const int kend = K < k0 + kc ? K : k0 + kc;
    quad_body<DT, MF, PRE, SPA, SPB, STAG, POL, OFFS, LAYOUT, 256, LAYOUT_MK, 1>(
        A, B, nullptr, M, N, K, lda, ldb, N, tm, tn, k0, kend - k0,
        W + (size_t)z * (size_t)M * (size_t)N, N, 0, 0);
}

// Stream-K for a product whose tiles do not fill whole waves ("Tiling a matmul", section
// "Where it breaks": a last partial wave leaves compute units idle), in one launch of
// G + dp_rows * grid_n workgroups.  The first G take the stream-K rows (tile rows
// dp_rows .. grid_m - 1): their (tile, 64-wide K step) iterations, tile by tile in
// row-major order, dealt in equal contiguous ranges, workgroup w taking iterations
// [w I / G, (w + 1) I / G) of the I = sk_tiles * nk.  With at most G such tiles a range
// spans at most two tiles: each segment runs the quad K walk over its K range and stores
// its fp32 partial tile to slot 2w + (its segment index) of W (256 x 256 floats per
// slot); sk_reduce, the next kernel, adds each tile's segments in workgroup order.  The
// other workgroups, dispatched after them, each take one whole tile of the leading
// dp_rows tile rows (grouped, XCD-aware order) and store it cast, as gemm_quad does.
template <int DT, int MF, int PRE, int SPA, int SPB, int STAG, int POL, bool OFFS,
          int LAYOUT = LAYOUT_NK>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256),
                               amdgpu_waves_per_eu(1, 1)))
gemm_quad_sk(const u16* __restrict__ A, const u16* __restrict__ B, u16* __restrict__ C, int M,
             int N, int K, int lda, int ldb, int ldc, int grid_n, int group_m, int dp_rows,
             int nk, int sk_tiles, int G, float* __restrict__ W) {
    const int wg = (int)blockIdx.x;
    if (wg >= G) {                             // a whole tile of the leading rows
        int tm, tn;
        tile_of(wg - G, dp_rows, grid_n, group_m, tm, tn);
        quad_body<DT, MF, PRE, SPA, SPB, STAG, POL, OFFS, LAYOUT, 256, LAYOUT_MK, 2>(
            A, B, C, M, N, K, lda, ldb, ldc, tm, tn, 0, 0, nullptr, 0, 0, 0, false);
        return;
    }
    const int64_t I = (int64_t)sk_tiles * nk;
    const int64_t b0 = (int64_t)wg * I / G, b1 = (int64_t)(wg + 1) * I / G;
    int64_t it = b0;
#pragma unroll 1
    for (int seg = 0; seg < 2 && it < b1; ++seg) {
        const int t = (int)(it / nk);
        const int s0 = (int)(it - (int64_t)t * nk);
        const int s1 = (int)((int64_t)nk < s0 + (b1 - it) ? (int64_t)nk : s0 + (b1 - it));
        const int tm = dp_rows + t / grid_n, tn = t % grid_n;
        const int k0 = s0 * 64, kend = K < s1 * 64 ? K : s1 * 64;
        if (seg > 0)
            __syncthreads();                   // the first segment's LDS reads are done
        quad_body<DT, MF, PRE, SPA, SPB, STAG, POL, OFFS, LAYOUT, 256, LAYOUT_MK, 2>(
            A, B, nullptr, M, N, K, lda, ldb, N, tm, tn, k0, kend - k0,
            W + (size_t)(2 * wg + seg) * 65536, 256, tm * 256, tn * 256, true);
        it += s1 - s0;
    }
}

// ------------------------------------------------------------------------------------
// Skinny kernel (small M, B as [N,K]): the product is a stream of B with little reuse
// ("Tiling a matmul", section "Where it breaks": small or skinny shapes stay
// memory-bound whatever the tiling; split-K keeps all the compute units busy).
//   One workgroup per 32 columns of C (all MT*32 rows of a row block); its 8 waves (4
//   with 128-wide chunks of 64 rows, whose LDS buffers would not fit eight times) split
//   the K range into as many contiguous parts (split-K inside the workgroup), each wave
//   accumulating a full (MT*32) x 32 partial product.  Per k chunk (64 wide: whole
//   128-byte row segments, 8 lanes per row; or 128 wide: 256-byte segments, 16 lanes
//   per row, longer runs per memory page) a wave loads the chunk D chunks ahead into
//   registers, writes it to its own swizzled LDS buffer and reads it back in MFMA
//   operand layout (a wave's LDS accesses complete in order, so no barrier is needed).
//   At the end the partial products are summed through LDS in a fixed order
//   (deterministic), cast once and stored.  Requirements as for gemm_tiled; rows past
//   M, columns past N and k past K read as zero through the buffer range check.
// ------------------------------------------------------------------------------------
// The skinny kernels' end: the waves' partial products to LDS as red[wave][n][m] (m
// contiguous), summed in wave order (deterministic), cast once and stored.
// acc[h * NB + b]: rows 32h.., columns 32b.. of the workgroup's BM x (32 NB) block.
template <int DT, int MT, int NW, int NB = 1>
__device__ __forceinline__ void skinny_epilogue(u16* lds, const f32x16 (&acc)[MT * NB],
                                                u16* __restrict__ C, int M, int N, int ldc,
                                                int m0, int n0, int tid, int lane, int wave) {
    constexpr int BN = 32 * NB, BM = MT * 32;
    const int half = lane >> 5;
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int h = 0; h < MT; ++h)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int n = 32 * b + 8 * (v >> 2) + 4 * half + (v & 3);
                red[(wave * BN + n) * BM + 32 * h + (lane & 31)] = acc[h * NB + b][v];
            }
    __syncthreads();
    constexpr int OUT_PER_T = BM * BN / (NW * 64);   // consecutive n per thread
    static_assert(OUT_PER_T % 4 == 0 || OUT_PER_T == 2, "store groups");
    const int m = tid % BM;
    const int nb = (tid / BM) * OUT_PER_T;
    float sum[OUT_PER_T];
#pragma unroll
    for (int q = 0; q < OUT_PER_T; ++q) {
        float t = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            t += red[(w * BN + nb + q) * BM + m];
        sum[q] = t;
    }
    // groups of G consecutive columns go out as one store where C's base and row stride
    // keep them G * 2-byte aligned and the group lies inside N, else one element at a
    // time (C may have any 2-byte alignment and any N: the operands alone decide whether
    // this kernel runs)
    constexpr int G = OUT_PER_T >= 4 ? 4 : 2;
    const bool cvec = ((uintptr_t)C % (2 * G)) == 0 && ldc % G == 0;
    const int gm = m0 + m;
    if (gm < M) {
        u16* crow = C + (size_t)gm * ldc + n0 + nb;
#pragma unroll
        for (int q = 0; q < OUT_PER_T; q += G) {
            const int n = n0 + nb + q;
            if (cvec && n + G <= N) {
                if constexpr (G == 4) {
                    u32x2 v;
                    v[0] = pack2<DT>(sum[q], sum[q + 1]);
                    v[1] = pack2<DT>(sum[q + 2], sum[q + 3]);
                    *reinterpret_cast<u32x2*>(crow + q) = v;
                } else {
                    *reinterpret_cast<uint32_t*>(crow + q) = pack2<DT>(sum[q], sum[q + 1]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < G; e += 2) {
                    const uint32_t pr = pack2<DT>(sum[q + e], sum[q + e + 1]);
                    if (n + e < N)
                        crow[q + e] = (u16)(pr & 0xffffu);
                    if (n + e + 1 < N)
                        crow[q + e + 1] = (u16)(pr >> 16);
                }
            }
        }
    }
}

template <int DT, int MT, int D, int CKT = 64, int NWT = 8, int NB = 1>
__global__ void __attribute__((amdgpu_flat_work_group_size(NWT * 64, NWT * 64),
                               amdgpu_waves_per_eu(NWT / 4, NWT / 4)))
gemm_skinny(const u16* __restrict__ A, const u16* __restrict__ B, u16* __restrict__ C, int M,
            int N, int K, int lda, int ldb, int ldc) {
    constexpr int NW = NWT, BN = 32 * NB, CK = CKT, KC = CK / 8;
    static_assert(NW == 4 || NW == 8, "four or eight waves");
    constexpr int RPL = 64 / KC;                   // chunk rows per 1 KiB load
    constexpr int BM = MT * 32;
    constexpr int ROWS = BM + BN;                  // rows of one chunk: A rows, then B rows
    constexpr int LD = ROWS / RPL;                 // 1 KiB loads per chunk per wave
    constexpr int WBUF = ROWS * CK;                // elements of one wave's LDS buffer
    constexpr int RED = NW * BN * BM;              // floats of the final reduction
    constexpr int LDS_ELEMS = (NW * WBUF * 2 > RED * 4) ? NW * WBUF : RED * 2;
    static_assert(CK == 64 || CK == 128, "64- or 128-wide chunks");
    static_assert(ROWS % RPL == 0 && LDS_ELEMS * 2 <= 160 * 1024, "chunk layout and LDS");
    __shared__ __attribute__((aligned(16))) u16 lds[LDS_ELEMS];

    const int n0 = (int)blockIdx.x * BN, m0 = (int)blockIdx.y * BM;
    const int tid = (int)threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;

    const rsrc_t ra = make_rsrc(A, span_bytes(M, K, lda));
    const rsrc_t rb = make_rsrc(B, span_bytes(N, K, ldb));
    // load i covers chunk rows RPL*i .. RPL*(i+1)-1: lane l takes row RPL*i + l/KC, 16-byte
    // piece l%KC (8 lanes per 128-byte row segment, or 16 per 256-byte one)
    const int lrow = lane / KC, lpc = lane % KC;
    uint32_t off[LD];
#pragma unroll
    for (int i = 0; i < LD; ++i) {
        const int r = RPL * i + lrow;
        if (r < BM)
            off[i] = m0 + r < M ? (uint32_t)((m0 + r) * lda + lpc * 8) * 2u : kOutOfRange;
        else
            off[i] = n0 + r - BM < N ? (uint32_t)((n0 + r - BM) * ldb + lpc * 8) * 2u
                                     : kOutOfRange;
    }
    u16* wb = lds + wave * WBUF;
    // LDS slot of load i's piece: chunk row RPL*i + lrow, swizzled by that row
    auto wr_off = [&](int i) {
        return (RPL * i + lrow) * CK + ((lpc ^ swz<KC>(RPL * i + lrow)) * 8);
    };
    // A loads whose RPL rows all lie past M carry nothing but still take a slot of the
    // compute unit's load path (decode products have M of 1-16 in a 32-row block): they
    // are not issued, and the LDS rows they would fill are zeroed once (a wave reads only
    // its own buffer)
    const int a_rows = M - m0;
    auto dead = [&](int i) { return i * RPL < BM && RPL * i >= a_rows; };
#pragma unroll
    for (int i = 0; i < LD; ++i)
        if (dead(i))
            *reinterpret_cast<u32x4*>(wb + wr_off(i)) = u32x4{0u, 0u, 0u, 0u};

    const int nch = (K + CK - 1) / CK;
    const int c_lo = wave * nch / NW, len = (wave + 1) * nch / NW - c_lo;
    // Every workgroup reads the same rows of A.  Each one starts its walk over the chunk
    // range at a different chunk (workgroups on one XCD are 8 apart in blockIdx.x), so the
    // workgroups of an XCD do not request the same A lines at the same moment.
    const int rot = len > 0 ? (int)((blockIdx.x >> 3) % (unsigned)len) : 0;

    u32x4 buf[D][LD];
    auto load_chunk = [&](int t, auto slot) {     // t-th chunk of this wave's walk
        constexpr int S = decltype(slot)::value;
        const bool live = t < len;
        const int p = t + rot < len ? t + rot : t + rot - len;
        const int k0 = live ? (c_lo + p) * CK : 0;
        const bool ok = live && k0 + lpc * 8 < K;
#pragma unroll
        for (int i = 0; i < LD; ++i)
            if (!dead(i))
                buf[S][i] = load16(i * RPL < BM ? ra : rb, ok ? off[i] : kOutOfRange,
                                   (uint32_t)k0 * 2u);
    };

    const int xr = swz<KC>(lane & 31);
    f32x16 acc[MT * NB];
#pragma unroll
    for (int h = 0; h < MT * NB; ++h)
        acc[h] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

    static_for<0, D>([&](auto d) { load_chunk(decltype(d)::value, d); });
    for (int c = 0; c < len; c += D) {
        static_for<0, D>([&](auto dc) {
            constexpr int d = decltype(dc)::value;
#pragma unroll
            for (int i = 0; i < LD; ++i)
                if (!dead(i))
                    *reinterpret_cast<u32x4*>(wb + wr_off(i)) = buf[d][i];
            u32x4 fa[CK / 16][MT], fb[CK / 16][NB];
#pragma unroll
            for (int j = 0; j < CK / 16; ++j) {
                const int koff = (((2 * j) | half) ^ xr) * 8;
#pragma unroll
                for (int h = 0; h < MT; ++h)
                    fa[j][h] = *reinterpret_cast<const u32x4*>(
                        wb + (32 * h + (lane & 31)) * CK + koff);
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    fb[j][b] = *reinterpret_cast<const u32x4*>(
                        wb + (BM + 32 * b + (lane & 31)) * CK + koff);
            }
            load_chunk(c + d + D, dc);
#pragma unroll
            for (int j = 0; j < CK / 16; ++j)
#pragma unroll
                for (int h = 0; h < MT; ++h)
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        acc[h * NB + b] =
                            mfma_32x32x16<DT>(fb[j][b], fa[j][h], acc[h * NB + b]);
        });
    }

    skinny_epilogue<DT, MT, NW, NB>(lds, acc, C, M, N, ldc, m0, n0, tid, lane, wave);
}

// The skinny kernel for B stored [K,N] (N contiguous): the same workgroup, wave split,
// A chunks and epilogue, with the B chunk taken as 64 k rows of the workgroup's 32
// columns (64 bytes per row; 16 rows per 1 KiB load) and stored as it lies.  Its MFMA
// operands come from two transposing LDS reads (ds_read_b64_tr_b16, as in the [K,N]
// forms of the tiled and ping-pong kernels): lane group g covers columns 16(g%2)..+15
// and k rows 8(g/2)..+3 (then +4), so each lane receives its column's 8 consecutive k in
// operand order; the four rows of a group's read are 64 bytes apart, so lanes 0-31 reach
// all 64 banks once.  A B row's 128-byte line holds two workgroups' columns: column
// blocks 2p and 2p+1 go to workgroups 8 ids apart (one XCD, one L2).
template <int DT, int MT, int D>
__global__ void __attribute__((amdgpu_flat_work_group_size(512, 512),
                               amdgpu_waves_per_eu(2, 2)))
gemm_skinny_kn(const u16* __restrict__ A, const u16* __restrict__ B, u16* __restrict__ C,
               int M, int N, int K, int lda, int ldb, int ldc) {
    constexpr int NW = 8, BN = 32, CK = 64, KC = CK / 8;
    constexpr int RPL = 64 / KC;                   // A rows per 1 KiB load (8)
    constexpr int BM = MT * 32;
    constexpr int LA = BM / RPL;                   // A loads per chunk per wave
    constexpr int LB = CK / 16;                    // B loads per chunk: 16 k rows each
    constexpr int ABUF = BM * CK, WBUF = ABUF + CK * BN;
    constexpr int RED = NW * BN * BM;              // floats of the final reduction
    constexpr int LDS_ELEMS = (NW * WBUF * 2 > RED * 4) ? NW * WBUF : RED * 2;
    static_assert(LDS_ELEMS * 2 <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) u16 lds[LDS_ELEMS];

    // column blocks in pairs per XCD; a ragged last group of 16 ids keeps the identity
    const int bid = (int)blockIdx.x, full = (int)gridDim.x & ~15;
    const int nblk = bid < full ? 2 * ((bid >> 4) * 8 + (bid & 7)) + ((bid >> 3) & 1) : bid;
    const int n0 = nblk * BN, m0 = (int)blockIdx.y * BM;
    const int tid = (int)threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;

    const rsrc_t ra = make_rsrc(A, span_bytes(M, K, lda));
    const rsrc_t rb = make_rsrc(B, span_bytes(K, N, ldb));
    // A load i: chunk rows 8i + lane/8, 16-byte piece lane%8 (as in gemm_skinny)
    const int lrow = lane / KC, lpc = lane % KC;
    uint32_t aoff[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int r = RPL * i + lrow;
        aoff[i] = m0 + r < M ? (uint32_t)((m0 + r) * lda + lpc * 8) * 2u : kOutOfRange;
    }
    // B load i: k rows 16i + lane/4 of the chunk, columns n0 + 8(lane%4) .. +7; the chunk's
    // first k row comes in as the scalar offset
    const int bkr = lane >> 2, bpc = lane & 3;
    const bool bcol = n0 + bpc * 8 < N;
    uint32_t boff[LB];
#pragma unroll
    for (int i = 0; i < LB; ++i)
        boff[i] = (uint32_t)((16 * i + bkr) * ldb + n0 + bpc * 8) * 2u;
    u16* wb = lds + wave * WBUF;                   // A rows [BM][CK], swizzled
    u16* wbb = wb + ABUF;                          // B rows [CK][BN], as they lie
    auto wr_a = [&](int i) {
        return (RPL * i + lrow) * CK + ((lpc ^ swz<KC>(RPL * i + lrow)) * 8);
    };
    // A loads whose 8 rows all lie past M are not issued; their LDS rows are zeroed once
    const int a_rows = M - m0;
    auto dead = [&](int i) { return RPL * i >= a_rows; };
#pragma unroll
    for (int i = 0; i < LA; ++i)
        if (dead(i))
            *reinterpret_cast<u32x4*>(wb + wr_a(i)) = u32x4{0u, 0u, 0u, 0u};

    const int nch = (K + CK - 1) / CK;
    const int c_lo = wave * nch / NW, len = (wave + 1) * nch / NW - c_lo;
    // the two workgroups of a column pair start their walks at the same chunk (so the
    // second read of each shared B line finds it in L2), pairs at different chunks
    const int rot = len > 0 ? (int)((unsigned)(nblk >> 1) % (unsigned)len) : 0;

    u32x4 abuf[D][LA], bbuf[D][LB];
    auto load_chunk = [&](int t, auto slot) {     // t-th chunk of this wave's walk
        constexpr int S = decltype(slot)::value;
        const bool live = t < len;
        const int p = t + rot < len ? t + rot : t + rot - len;
        const int k0 = live ? (c_lo + p) * CK : 0;
        const bool ok = live && k0 + lpc * 8 < K;
#pragma unroll
        for (int i = 0; i < LA; ++i)
            if (!dead(i))
                abuf[S][i] = load16(ra, ok ? aoff[i] : kOutOfRange, (uint32_t)k0 * 2u);
#pragma unroll
        for (int i = 0; i < LB; ++i) {
            const bool bok = live && bcol && k0 + 16 * i + bkr < K;
            bbuf[S][i] = load16(rb, bok ? boff[i] : kOutOfRange, (uint32_t)k0 * (uint32_t)ldb * 2u);
        }
    };

    const int g = lane >> 4, sl = lane & 15;
    const int btr = (8 * (g >> 1) + (sl >> 2)) * BN + 16 * (g & 1) + 4 * (sl & 3);
    auto read_tr = [&](const u16* p0) {            // k rows kl and kl + 4
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 4 * BN));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
    };

    const int xr = swz<KC>(lane & 31);
    f32x16 acc[MT];
#pragma unroll
    for (int h = 0; h < MT; ++h)
        acc[h] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

    static_for<0, D>([&](auto d) { load_chunk(decltype(d)::value, d); });
    for (int c = 0; c < len; c += D) {
        static_for<0, D>([&](auto dc) {
            constexpr int d = decltype(dc)::value;
#pragma unroll
            for (int i = 0; i < LA; ++i)
                if (!dead(i))
                    *reinterpret_cast<u32x4*>(wb + wr_a(i)) = abuf[d][i];
#pragma unroll
            for (int i = 0; i < LB; ++i)
                *reinterpret_cast<u32x4*>(wbb + (16 * i + bkr) * BN + bpc * 8) = bbuf[d][i];
            u32x4 fa[CK / 16][MT], fb[CK / 16];
#pragma unroll
            for (int j = 0; j < CK / 16; ++j) {
                const int koff = (((2 * j) | half) ^ xr) * 8;
#pragma unroll
                for (int h = 0; h < MT; ++h)
                    fa[j][h] = *reinterpret_cast<const u32x4*>(
                        wb + (32 * h + (lane & 31)) * CK + koff);
                fb[j] = read_tr(wbb + 16 * j * BN + btr);
            }
            load_chunk(c + d + D, dc);
#pragma unroll
            for (int j = 0; j < CK / 16; ++j)
#pragma unroll
                for (int h = 0; h < MT; ++h)
                    acc[h] = mfma_32x32x16<DT>(fb[j], fa[j][h], acc[h]);
        });
    }
    skinny_epilogue<DT, MT, NW>(lds, acc, C, M, N, ldc, m0, n0, tid, lane, wave);
}

// ------------------------------------------------------------------------------------
// The generic kernel: any alignment, any M, N, K.  64 x 64 tile, K step 16, 4 waves each
// owning one 32 x 32 MFMA block; element-by-element masked loads into one LDS stage.
// ------------------------------------------------------------------------------------
template <int DT, int ALAYOUT, int LAYOUT>
__global__ void __launch_bounds__(256)
gemm_generic(const u16* __restrict__ A, const u16* __restrict__ B, u16* __restrict__ C, int M,
             int N, int K, int lda, int ldb, int ldc, int grid_m, int grid_n, int group_m) {
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
            // consecutive threads walk the contiguous index of each operand
            if constexpr (ALAYOUT == LAYOUT_MK) {
                const int r = e >> 4, kk = e & 15;
                const int gm = m0 + r, gk = k0 + kk;
                As[r * 16 + kk] = (gm < M && gk < K) ? A[(size_t)gm * lda + gk] : (u16)0;
            } else {
                const int r = e & 63, kk = e >> 6;
                const int gm = m0 + r, gk = k0 + kk;
                As[r * 16 + kk] = (gm < M && gk < K) ? A[(size_t)gk * lda + gm] : (u16)0;
            }
            if constexpr (LAYOUT == LAYOUT_NK) {
                const int r = e >> 4, kk = e & 15;
                const int gn = n0 + r, gk = k0 + kk;
                Bs[r * 16 + kk] = (gn < N && gk < K) ? B[(size_t)gn * ldb + gk] : (u16)0;
            } else {
                const int r = e & 63, kk = e >> 6;
                const int gn = n0 + r, gk = k0 + kk;
                Bs[r * 16 + kk] = (gn < N && gk < K) ? B[(size_t)gk * ldb + gn] : (u16)0;
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
                C[(size_t)m * ldc + n] = cvt1<DT>(acc[v]);
        }
    }
}

}  // namespace tgemm
