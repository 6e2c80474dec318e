// Attention forward on the matrix cores of gfx950: the tile pipeline of the product kernels
// (direct-to-LDS loads into a ring of swizzled LDS stages, MFMA operands read from LDS)
// applied twice per key tile, with the softmax kept online in registers.
//
// "TileLang: a tile language one level below Triton", section "FlashAttention: online
// softmax as tile code": each block takes block_M queries and walks the keys tile by tile;
// it keeps a running row maximum and row sum, rescales what it has accumulated to each new
// maximum, uses base-2 exponentials with log2(e) folded into the 1/sqrt(dim) scale, casts
// the probabilities to float16 for the product with V, divides by the row sum once at the
// end, and handles the causal mask at two levels (key tiles wholly above the diagonal are
// not visited; inside the diagonal tile the masked scores become -infinity).
#pragma once

#include "kernels.hpp"

namespace tgemm {

// Q, K, V, O: fp16 [batch, seq, heads, D] (D contiguous).  One workgroup per 128 queries
// of one (batch, head); 4 waves, wave w owning queries [32w, 32w+32) of the block.
//   Scores:  S = Q K^T for 64 keys at a time with v_mfma_f32_32x32x16_f16, the key rows
//            as the first source and the query rows as the second, so that lane l holds
//            query row l % 32 and keys 8g + 4(l/32) + (0..3) of each 32-key block: a
//            row's 64 scores sit in two lanes (l, l+32).
//   Softmax: row maximum over the lane's 32 scores and its partner's (one lane swap),
//            p = 2^(s*scale - max) in fp32, rescale of the running sum and of O by
//            2^(old max - new max).  Each lane keeps its half of the row sum; the halves
//            are added once at the end.
//   P V:     the probabilities, cast to fp16, are the second source as they lie: for the
//            16 keys of an MFMA step the lane supplies its own 8 (keys 0-3 and 8-11 of
//            the step for l < 32, keys 4-7 and 12-15 for l >= 32), and the first source
//            reads V^T in that same key order with two transposing LDS reads
//            (ds_read_b64_tr_b16), keys base and base + 8.
//   Loads:   K and V tiles (64 x D each) arrive by direct-to-LDS 16-byte loads into a
//            2-stage ring (32 KiB per workgroup, so four workgroups share a compute unit
//            and each SIMD holds four waves); tile t+1's loads go out once every wave has
//            met at the start of step t, into the stage tile t-1 left.  The step is
//            compiled once per stage, so every LDS address is a fixed lane offset plus an
//            immediate, and a tile's loads read through a descriptor based at its first
//            key row: the lane offsets stay fixed and the advance is scalar.  K rows are
//            stored with 16-byte chunk c at c ^ ((row / 2) mod KC) (the row-wise reads of
//            32 rows hit distinct banks); V rows with chunk c at
//            c ^ 2(row mod 4) (the 4 x 16 blocks of the transposing reads hit distinct
//            banks).  Rows past seq read as zeros (buffer range check).
//   The whole (b, h) slice spans at most 2^31 bytes (checked by the host).
// Lane l and lane l ^ 32 combined, in every lane: v_permlane32_swap exchanges the upper
// half of its first operand with the lower half of its second, so with both operands v
// the two results hold v of lanes 0-31 and v of lanes 32-63, each in all 64 lanes.
__device__ __forceinline__ float half_swap_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One transposing LDS read (ds_read_b64_tr_b16) at a byte address plus a constant offset
// (the instruction's offset field; the compiler's own form of this read does not fold
// constants into it).  Its result may be used only after lds_reads_done: the compiler does
// not count this read among the LDS operations it waits for.
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr16_b64(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "16-bit offset");
    u32x2 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}
// Wait for every LDS read issued so far; the values pass through the wait, so no use of
// them is scheduled before it.
__device__ __forceinline__ void lds_reads_done(u32x2 (&v)[2][2][2]) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(v[0][0][0]), "+v"(v[0][0][1]), "+v"(v[0][1][0]), "+v"(v[0][1][1]),
                   "+v"(v[1][0][0]), "+v"(v[1][0][1]), "+v"(v[1][1][0]), "+v"(v[1][1][1]));
}

template <int D, bool CAUSAL>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256),
                               amdgpu_waves_per_eu(4, 4)))
attn_fwd(const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V,
         u16* __restrict__ O, int S, int H, float scale_log2, int nqb) {
    constexpr int BM = 128, BN = 64, ST = 2;
    constexpr int KC = D / 8;                  // 16-byte chunks per row
    constexpr int ROWS = 64 / KC;              // rows per 1 KiB load
    constexpr int TILE = BN * D;               // elements of one K or V tile
    constexpr int LW = BN / ROWS / 4;          // loads per wave per K (or V) tile
    constexpr int NS = D / 16;                 // k-steps of Q K^T
    constexpr int NDB = D / 32;                // 32-wide column blocks of O
    // (the V swizzle and the load split are laid out for 128-byte rows)
    static_assert(D == 64, "head dimension 64");
    static_assert(LW >= 1 && (BN / ROWS) % 4 == 0, "load split");
    __shared__ __attribute__((aligned(1024))) u16 lds[ST * 2 * TILE];   // [stage][K|V]

    const int tid = (int)threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // One-dimensional grid, the (batch, head) index varying fastest and the query block
    // slowest, so that workgroups start in order of decreasing work (causal: the last
    // query blocks, which visit the most key tiles, first) and the short ones fill the
    // tail of the launch.
    const int nbh = (int)gridDim.x / nqb;
    const int qi = (int)blockIdx.x / nbh, bh = (int)blockIdx.x - qi * nbh;
    const int qb = CAUSAL ? nqb - 1 - qi : qi;
    const int b = bh / H, h = bh - (bh / H) * H;
    const int q0 = qb * BM + 32 * wave;
    const int r = lane & 31, hh = lane >> 5;
    const uint32_t rs = (uint32_t)H * D;               // elements between sequence positions
    const size_t base = ((size_t)b * S * H + h) * D;   // (b, 0, h, 0)
    const uint32_t span = S > 0 ? ((uint32_t)(S - 1) * rs + D) * 2u : 0u;
    const rsrc_t rq = make_rsrc(Q + base, span);

    // key tiles this block visits: those holding a key at or before its last query
    const int ntile_all = (S + BN - 1) / BN;
    const int nkt = CAUSAL ? min(ntile_all, ((qb + 1) * BM + BN - 1) / BN) : ntile_all;

    // Q fragments (second source of the score MFMAs): query row q0 + r, 8 dims per lane
    u32x4 qf[NS];
    {
        const int q = q0 + r;
#pragma unroll
        for (int s = 0; s < NS; ++s)
            qf[s] = load16(rq, q < S ? ((uint32_t)q * rs + 16 * s + 8 * hh) * 2u : kOutOfRange,
                           0);
#pragma unroll
        for (int s = 0; s < NS; ++s)
            asm volatile("" ::"v"(qf[s]));     // landed before the loop, not waited in it
    }

    // direct-to-LDS loads: wave w fills rows [BN/4 * w, BN/4 * (w+1)) of a tile, ROWS at a
    // time; lane l lands in row l / KC at physical chunk l % KC
    const int prow = lane / KC, pch = lane % KC;
    int kchunk[LW], vchunk[LW], trow[LW];
#pragma unroll
    for (int i = 0; i < LW; ++i) {
        trow[i] = (BN / 4) * wave + ROWS * i + prow;
        kchunk[i] = pch ^ swz<KC>(trow[i]);
        vchunk[i] = pch ^ (2 * (trow[i] & 3));
    }
    const uint32_t lds0 = lds_addr(lds);
    // a tile's loads read through descriptors based at its first key row and ending where
    // the (b, h) slice ends, so the lane offsets are fixed and rows past seq (whose offsets
    // reach past the descriptor's end, the row stride being at least D) read as zeros
    uint32_t kgo[LW], vgo[LW];
#pragma unroll
    for (int i = 0; i < LW; ++i) {
        kgo[i] = ((uint32_t)trow[i] * rs + kchunk[i] * 8) * 2u;
        vgo[i] = ((uint32_t)trow[i] * rs + vchunk[i] * 8) * 2u;
    }
    auto issue = [&](auto stc, int kt) {
        constexpr int st = decltype(stc)::value;
        const uint32_t skip = (uint32_t)kt * BN * rs * 2u;      // kt * BN < S: below span
        const rsrc4_t rkt = make_rsrc4(K + base + (size_t)kt * BN * rs, span - skip);
        const rsrc4_t rvt = make_rsrc4(V + base + (size_t)kt * BN * rs, span - skip);
#pragma unroll
        for (int i = 0; i < LW; ++i) {
            const uint32_t ldsb = lds0 + (uint32_t)((st * 2 * TILE + (BN / 4 * wave + ROWS * i) * D) * 2);
            dma16_at(rkt, ldsb, kgo[i], 0);
            dma16_at(rvt, ldsb + TILE * 2, vgo[i], 0);
        }
    };

    // V^T reads: lane sl of 16-lane group g points at key row base + 4(g/2) + sl/4 and the
    // 4 columns 16(g%2) + 4(sl%4) of a 32-column block.  The lane's part of the address
    // (row, swizzled column) is fixed; the tile rows of a step (32 kb + 16 step, + 8 for the
    // second read, a multiple of 4: same swizzle) come in as constant offsets.
    const int g = lane >> 4, sl = lane & 15;
    const int vrow = 4 * (g >> 1) + (sl >> 2);
    const int vcol = 16 * (g & 1) + 4 * (sl & 3);
    int vofs[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int col = 32 * db + vcol;
        vofs[db] = vrow * D + ((col >> 3) ^ (2 * (vrow & 3))) * 8 + (col & 7);
    }
    // byte address of the lane's first V^T read in the V part of stage 0, per column block
    uint32_t vaddr0[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
        vaddr0[db] = lds_addr(lds) + (uint32_t)(TILE + vofs[db]) * 2u;
    // K reads: lane's key row r of a 32-key block, chunk (2 s + l/32) swizzled by the row
    // (the swizzle of rows r and 32 + r agree)
    int kofs[NS];
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2)
        kofs[s2] = r * D + (((2 * s2 + hh) ^ swz<KC>(r)) * 8);
    // fp16 pair, nearest-even (one packed conversion)
    auto pack_f16 = [](float a, float b) {
        typedef float f2 __attribute__((ext_vector_type(2)));
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, h2));
    };

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
        oacc[db] = f32x16{};
    constexpr float kSlack = 8.0f;             // log2 of the largest weight allowed
    float m_run = -__builtin_huge_valf();      // reference maximum (scaled scores, base 2)
    float l_run = 0.0f;                        // this lane's half of the running row sum
    const int q = q0 + r;

    if (nkt > 0)
        issue(std::integral_constant<int, 0>{}, 0);
    // one copy of the step per ring stage, the stage a compile-time constant in each
    for (int kt0 = 0; kt0 < nkt; kt0 += ST) {
      static_for<0, ST>([&](auto stc) {
        constexpr int st = decltype(stc)::value;
        const int kt = kt0 + st;
        if (kt >= nkt)
            return;
        // tile kt has landed and every wave is done with tile kt-1, whose stage tile kt+1
        // then fills
        wait_vm_then_sync<0>();
        if (kt + 1 < nkt)
            issue(std::integral_constant<int, (st + 1) % ST>{}, kt + 1);
        const u16* kt_lds = lds + st * 2 * TILE;

        // S = Q K^T, two 32-key blocks
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sacc[kb] = f32x16{};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const u32x4 kf =
                    *reinterpret_cast<const u32x4*>(kt_lds + kofs[s] + 32 * kb * D);
                sacc[kb] = mfma_32x32x16<DT_F16>(kf, qf[s], sacc[kb]);
            }
        }
        // mask (tiles on the diagonal or past the end only), row maximum of the raw scores
        if (kt * BN + BN > S || (CAUSAL && kt * BN + BN - 1 > q0)) {
            const int lim = CAUSAL ? min(S, q + 1) : S;   // keys below lim count
            const int k0 = kt * BN + 4 * hh;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    sacc[kb][v] = k0 + 32 * kb + 8 * (v >> 2) + (v & 3) < lim
                                      ? sacc[kb][v]
                                      : -__builtin_huge_valf();
        }
        // row maximum of the raw scores: three-input maxima (the scores come straight
        // from the matrix core, so no NaN needs quieting first)
        float mx = -__builtin_huge_valf();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; v += 2)
                asm("v_max3_f32 %0, %1, %2, %3" : "=v"(mx) : "v"(mx), "v"(sacc[kb][v]),
                    "v"(sacc[kb][v + 1]));
        mx = half_swap_max(mx);
        // The exponentials are taken against a reference m_run that moves only when the
        // row maximum (scaled) has risen more than kSlack above it, so most tiles skip the
        // rescale of O: a weight is then at most 2^kSlack, which fp16 and the fp32 sums
        // hold exactly as well (the softmax does not depend on the reference).
        const float m_cand = fmaxf(m_run, mx * scale_log2);
        const bool move = m_cand > m_run + kSlack;         // also the first finite maximum
        // (the rescale is skipped when no lane of the wave moves: it would multiply by 1,
        // or, for a row with no key yet, multiply zeros by 0)
        if (__builtin_amdgcn_ballot_w64(move)) {
            const float m_new = move ? m_cand : m_run;
            // a row with no key yet keeps an offset of 0 (its scores are all -infinity)
            const float m_use = m_new == -__builtin_huge_valf() ? 0.0f : m_new;
            const float rescale = __builtin_amdgcn_exp2f(m_run - m_use);   // 1 if not moved
            m_run = m_new;
            l_run *= rescale;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    oacc[db][v] *= rescale;
        }
        const float m_use = m_run == -__builtin_huge_valf() ? 0.0f : m_run;
        float psum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                // p = 2^(s * scale - m_run), one fused multiply-add before the exponential
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][v], scale_log2, -m_use));
                sacc[kb][v] = p;
                psum += p;
            }
        }
        l_run += psum;

        // O += P V: four 16-key steps, the probabilities in fp16.  The V^T operands of a
        // 32-key block are read first (8 transposing reads), then the weights packed, then
        // the reads waited for and the four products issued.
        static_for<0, 2>([&](auto kbc) {
            constexpr int kb = decltype(kbc)::value;
            u32x2 vf[2][NDB][2];
            static_for<0, 2>([&](auto qqc) {
                constexpr int qq = decltype(qqc)::value;
                constexpr int off = (st * 2 * TILE + 32 * kb * D + 16 * qq * D) * 2;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    vf[qq][db][0] = ds_read_tr16_b64<off>(vaddr0[db]);
                    vf[qq][db][1] = ds_read_tr16_b64<off + 8 * D * 2>(vaddr0[db]);
                }
            });
            u32x4 pf[2];
#pragma unroll
            for (int qq = 0; qq < 2; ++qq)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    pf[qq][e] = pack_f16(sacc[kb][8 * qq + 2 * e], sacc[kb][8 * qq + 2 * e + 1]);
            lds_reads_done(vf);
#pragma unroll
            for (int qq = 0; qq < 2; ++qq)
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    oacc[db] = mfma_32x32x16<DT_F16>(
                        u32x4{vf[qq][db][0][0], vf[qq][db][0][1], vf[qq][db][1][0],
                              vf[qq][db][1][1]},
                        pf[qq], oacc[db]);
        });
      });
    }
    wait_vm<0>();                               // no load left in flight

    // divide by the row sum once, cast, store: lane holds row q, columns 8g' + 4hh + 0..3
    const float l_tot = half_swap_sum(l_run);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (q < S) {
        u16* orow = O + base + (size_t)q * rs;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                u32x2 v;
                v[0] = pack_f16(oacc[db][4 * gg + 0] * inv, oacc[db][4 * gg + 1] * inv);
                v[1] = pack_f16(oacc[db][4 * gg + 2] * inv, oacc[db][4 * gg + 3] * inv);
                *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * gg + 4 * hh) = v;
            }
        }
    }
}

}  // namespace tgemm
