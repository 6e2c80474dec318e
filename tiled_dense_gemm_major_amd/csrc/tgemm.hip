// libtgemm: the C ABI, argument checks, the compiled-configuration registry, the
// per-shape configuration table and the launches.  Declarations and conventions are in
// include/tgemm.h.
#include "tgemm.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "registry.hpp"

// The fixed scratch of gemm_ex_noalloc (split-K's fp32 partial tiles), for callers that
// cannot allocate.  File-scope device memory: each GPU the library runs on holds its own
// copy until the process ends.  Host code never passes this name to a kernel (on the
// host it is only a stand-in); it uses the device address hipGetSymbolAddress returns.
constexpr int64_t kScratchBytes = int64_t(16) << 20;
static __device__ __align__(256) float scratch[kScratchBytes / 4];

namespace {

constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;

using tgemm_reg::kMaxSplits;
using tgemm_reg::Variant;

// The kernels that split K over workgroups, with fp32 partials in a workspace.
bool is_split(int kernel) {
    return kernel == TGEMM_KERNEL_SPLITK || kernel == TGEMM_KERNEL_QUAD_SPLITK;
}

// Position of a kernel family in the listing order of one (A storage, B storage, dtype)
// group: generic, masked, tiled, direct-to-LDS ring, ping-pong, quad, skinny, split-K,
// quad split-K, quad stream-K, direct.
int family_rank(int kernel) {
    switch (kernel) {
    case TGEMM_KERNEL_GENERIC: return 0;
    case TGEMM_KERNEL_MASKED: return 1;
    case TGEMM_KERNEL_TILED: return 2;
    case TGEMM_KERNEL_DMA: return 3;
    case TGEMM_KERNEL_PINGPONG: return 4;
    case TGEMM_KERNEL_QUAD: return 5;
    case TGEMM_KERNEL_SKINNY: return 6;
    case TGEMM_KERNEL_SPLITK: return 7;
    case TGEMM_KERNEL_QUAD_SPLITK: return 8;
    case TGEMM_KERNEL_QUAD_STREAMK: return 9;
    default: return 10;
    }
}

// Every compiled configuration, from the translation units' lists, in one fixed order:
// grouped by A storage, B storage and dtype, then by family; a family's entries keep the
// order its unit lists them in.
const std::vector<const Variant*>& registry() {
    static const std::vector<const Variant*> all = [] {
        std::vector<const Variant*> v;
        for (const tgemm_reg::VariantList& l :
             {tgemm_reg::variants_tiled(), tgemm_reg::variants_masked_nk(),
             tgemm_reg::variants_masked(), tgemm_reg::variants_small(),
              tgemm_reg::variants_pingpong_nk(), tgemm_reg::variants_pingpong_other(),
              tgemm_reg::variants_quad(), tgemm_reg::variants_quad_kn(),
              tgemm_reg::variants_quad_km(), tgemm_reg::variants_direct(),
              tgemm_reg::variants_quad_split()})
            for (int i = 0; i < l.n; ++i)
                v.push_back(&l.v[i]);
        const auto key = [](const Variant* x) {
            return ((x->a_layout * 2 + x->layout) * 2 + x->dtype) * 16 +
                   family_rank(x->cfg.kernel);
        };
        std::stable_sort(v.begin(), v.end(),
                         [&](const Variant* a, const Variant* b) { return key(a) < key(b); });
        return v;
    }();
    return all;
}

bool same_shape(const tgemm_config& a, const tgemm_config& b) {
    // a split-K configuration's split count is a per-call choice
    const bool split_ok = is_split(a.kernel) ? b.split_k >= 2 && b.split_k <= kMaxSplits
                                             : a.split_k == b.split_k;
    return a.kernel == b.kernel && a.block_m == b.block_m && a.block_n == b.block_n &&
           a.block_k == b.block_k && a.waves_m == b.waves_m && a.waves_n == b.waves_n &&
           a.stages == b.stages && split_ok && a.mfma == b.mfma;
}

const Variant* find_variant(int dtype, int a_layout, int layout, const tgemm_config& cfg) {
    for (const Variant* v : registry()) {
        if (v->dtype == dtype && v->a_layout == a_layout && v->layout == layout &&
            same_shape(v->cfg, cfg))
            return v;
    }
    return nullptr;
}

// The table: fast configurations by how many workgroups they give, so that the chip
// (256 compute units) is filled with the largest tile that still fills it; small M with
// long K goes to the split-K skinny kernel.
// The frozen per-device table (tile_table.inc, written by the sweep's --emit-table from
// timings of every fast configuration on a grid of shapes): for A [M,K], the entry at
// the grid point nearest in log2 of M, N and K, if the table has one.
struct TableEntry {
    int8_t layout, mi, ni, ki;
    tgemm_config cfg;
};
#include "tile_table.inc"

template <int N>
int nearest_point(const int64_t (&grid)[N], int64_t x) {
    const double lx = log2((double)(x > 1 ? x : 1));
    int best = 0;
    double bd = 1e300;
    for (int i = 0; i < N; ++i) {
        const double d = fabs(log2((double)grid[i]) - lx);
        if (d < bd) {
            bd = d;
            best = i;
        }
    }
    return best;
}

const tgemm_config* table_lookup(int layout, int64_t m, int64_t n, int64_t k) {
    const int mi = nearest_point(kTableM, m), ni = nearest_point(kTableN, n),
              ki = nearest_point(kTableK, k);
    constexpr int NM = sizeof(kTableM) / sizeof(kTableM[0]);
    constexpr int NN = sizeof(kTableN) / sizeof(kTableN[0]);
    constexpr int NK = sizeof(kTableK) / sizeof(kTableK[0]);
    constexpr int NE = sizeof(kTable) / sizeof(kTable[0]);
    auto match = [&](const TableEntry& e) {
        return e.layout == layout && e.mi == mi && e.ni == ni && e.ki == ki;
    };
    // the generator writes every point in (layout, m, n, k) order: index it directly
    const int idx = ((layout * NM + mi) * NN + ni) * NK + ki;
    if (idx >= 0 && idx < NE && match(kTable[idx]))
        return &kTable[idx].cfg;
    for (const TableEntry& e : kTable)
        if (match(e))
            return &e.cfg;
    return nullptr;
}

bool on_grid(const int64_t* grid, int count, int64_t x) {
    for (int i = 0; i < count; ++i)
        if (grid[i] == x)
            return true;
    return false;
}

// The quad kernel's tile height for an m x n product, by wave quantization: a tile row
// count that needs fewer waves of the 256 compute units wins.  A 192-row tile does
// three quarters of a 256-row tile's work at ~10 % less work per cycle (measured: 0.81
// of the 256-row time where both need one wave), so it costs 0.825 of a 256-row wave.
// Returns 0 when the two are within 5 % (the caller keeps its choice).
int quad_rows_by_waves(int64_t m, int64_t n) {
    const int64_t tn = (n + 255) / 256;
    const double w256 = (double)((((m + 255) / 256) * tn + 255) / 256);
    const double w192 = 0.825 * (double)((((m + 191) / 192) * tn + 255) / 256);
    if (w192 < 0.95 * w256)
        return 192;
    if (w256 < 0.95 * w192)
        return 256;
    return 0;
}

// Operands without the fast kernels' alignment: the masked tiled kernel, with the tile
// that minimises (waves of 256 workgroups) x (one tile's time).  The tile times relative
// to 256x256 (1, 0.646, 0.373, 0.180 for 256x256, 128x256 or 256x128, 128x128, 64x64)
// are the per-wave times of bf16 4096x4096x4094, which fills the chip with every tile;
// the model picked the fastest tile on all 7 shapes timed against it (1024^2 to 4096^2,
// square, wide and tall).  The tiles above 128x128 only where A [M,K] and B [N,K] are
// both read as realigned 16-byte blocks; an operand read as 2-byte elements holds a
// register per element, and larger tiles would spill.
tgemm_config choose_masked(int a_layout, int layout, int64_t m, int64_t n) {
    struct Option {
        int bm, bn, group;
        double tile_time;
    };
    static const Option kOptions[] = {{256, 256, 4, 1.0},
                                      {128, 256, 8, 0.646},
                                      {256, 128, 8, 0.646},
                                      {128, 128, 8, 0.373},
                                      {64, 64, 8, 0.180}};
    const bool large = a_layout == TGEMM_A_MK && layout == TGEMM_B_NK;
    const Option* best = nullptr;
    double best_cost = 0;
    for (const Option& o : kOptions) {
        if (!large && (o.bm > 128 || o.bn > 128))
            continue;
        const int64_t tiles = ((m + o.bm - 1) / o.bm) * ((n + o.bn - 1) / o.bn);
        const double cost = (double)((tiles + 255) / 256) * o.tile_time;
        if (!best || cost < best_cost) {
            best = &o;
            best_cost = cost;
        }
    }
    return tgemm_config{TGEMM_KERNEL_MASKED, best->bm, best->bn, 64, 2, 2, 2, best->group, 1, 32};
}

// The skinny kernel's 64-column forms: 32 rows with 64-wide chunks two ahead, 64 rows
// with 64-wide chunks one ahead, eight waves each.
constexpr tgemm_config kSkinnyN64Rows32{TGEMM_KERNEL_SKINNY, 32, 64, 64, 1, 8, 2, 1, 8, 32};
constexpr tgemm_config kSkinnyN64Rows64{TGEMM_KERNEL_SKINNY, 64, 64, 64, 1, 8, 1, 1, 8, 32};

constexpr tgemm_config kTiled128{TGEMM_KERNEL_TILED, 128, 128, 64, 2, 2, 2, 8, 1, 32};
constexpr tgemm_config kDma64x128{TGEMM_KERNEL_DMA, 64, 128, 64, 1, 4, 4, 2, 1, 32};
constexpr tgemm_config kQuadRows192{TGEMM_KERNEL_QUAD, 192, 256, 64, 2, 2, 5, 4, 1, 32};

// Products with B [N,K] past the grid's widest N whose nearest grid point takes the
// skinny kernel (up to about 180 rows): they stream B, and that choice re-reads all of A
// once per 32 columns and, at thousands of workgroups, leaves a ragged last wave.  Measured
// hot, bf16, K = 4096, M 1-128, N 12288-50264 (us, the grid's choice -> this one):
// - below N = 40960, at most 64 rows: the 64-column skinny form, half the A re-reads
//   (8x12288 22.5 -> 19.0, 32x14336 27.5 -> 21.5, 64x14336 33.0 -> 23.2, 64x28672
//   61.1 -> 42.9);
// - below N = 40960, more than 64 rows: the first of these whose tiles make one wave
//   (at most 256): the direct-to-LDS kernel's 64x128 tiles (128x12288 42.4 -> 33.8,
//   96x14336 37.6 -> 33.7, 80x16384 40.0 -> 35.3), the tiled kernel's 128x128 tiles
//   (128x28672 82.0 -> 44.0, 160x16384 71.5 -> 43.2, 72x20480 -> 39.4), else the quad
//   kernel's 192x256 tiles (144x24576 -> 55.0 against 75.1 for 128x128 tiles);
// - from N = 40960 (one wave of 192x256 tiles), more than 8 rows: the quad kernel
//   (16x50264 90.0 -> 81.4, 32x50264 92.9 -> 82.0, 64x50264 103.5 -> 83.9, 128x50264
//   169.9 -> 84.9); up to 8 rows the two are level (78.5-84.5 against 80.5-82.8) and
//   the skinny form stays.
tgemm_config choose_wide_n(int64_t m, int64_t n, const tgemm_config& grid_choice) {
    if (n >= 40960)
        return m <= 8 ? grid_choice : kQuadRows192;
    if (m <= 64)
        return m <= 32 ? kSkinnyN64Rows32 : kSkinnyN64Rows64;
    const auto tiles = [&](int64_t bm, int64_t bn) {
        return ((m + bm - 1) / bm) * ((n + bn - 1) / bn);
    };
    if (tiles(64, 128) <= 256)
        return kDma64x128;
    return tiles(128, 128) <= 256 ? kTiled128 : kQuadRows192;
}

// The kernel for operands past what the masked kernel's buffer offsets reach.
constexpr tgemm_config kGenericConfig{TGEMM_KERNEL_GENERIC, 64, 64, 16, 2, 2, 1, 8, 1, 32};

tgemm_config choose(int dtype, int a_layout, int layout, int64_t m, int64_t n, int64_t k,
                    bool aligned) {
    (void)dtype;
    if (!aligned)
        return choose_masked(a_layout, layout, m, n);
    if (a_layout == TGEMM_A_MK) {
        if (const tgemm_config* c = table_lookup(layout, m, n, k)) {
            tgemm_config cfg = *c;
            // Between grid points the nearest point's tile height can cost a wave: the
            // quad kernel's 256- or 192-row tiles are re-decided for the actual size
            // (on 19 shapes off the grid the rule picked the faster height every time,
            // 5-26 % faster than the nearest point's where they differed).
            constexpr int NM = sizeof(kTableM) / sizeof(kTableM[0]);
            constexpr int NN = sizeof(kTableN) / sizeof(kTableN[0]);
            // With B [K,N] the MFMA form is re-decided as well.  The 16x16x32 form spends
            // less energy per product but spills with 256-row tiles, so 256-row tiles
            // take the 32x32x16 form everywhere; off the grid, 192-row tiles take the
            // 16x16x32 form when the grid has more than one wave of tiles (a
            // power-limited run) and the 32x32x16 form otherwise.  On 30 random shapes
            // with B [K,N] (a set not used to find the rule) the nearest point's form
            // lost 2.5 % on average and up to 31 % to the fastest quad configuration;
            // with the rule, 0.3 % and 2.4 %.
            if (cfg.kernel == TGEMM_KERNEL_QUAD) {
                const bool off_grid = !(on_grid(kTableM, NM, m) && on_grid(kTableN, NN, n));
                if (off_grid) {
                    const int rows = quad_rows_by_waves(m, n);
                    if (rows != 0)
                        cfg.block_m = rows;
                }
                if (layout == TGEMM_B_KN) {
                    const int64_t tiles = ((m + cfg.block_m - 1) / cfg.block_m) *
                                          ((n + cfg.block_n - 1) / cfg.block_n);
                    if (cfg.block_m == 256)
                        cfg.mfma = 32;
                    else if (off_grid)
                        cfg.mfma = tiles > 256 ? 16 : 32;
                }
            }
            // (65-192 rows whose grid point takes 64x64 to 128x128 tiles are re-decided
            // the same way: 128x20480x2048 40.4 -> 23.9 us, 192x28672x4096 80.1 -> 56.8)
            const bool small_tiles =
                cfg.kernel == TGEMM_KERNEL_TILED || cfg.kernel == TGEMM_KERNEL_DMA;
            if ((cfg.kernel == TGEMM_KERNEL_SKINNY || (small_tiles && m > 64 && m <= 192)) &&
                layout == TGEMM_B_NK && k >= 1024 && n > kTableN[NN - 1])
                cfg = choose_wide_n(m, n, cfg);
            // With B [K,N] the same past-the-grid choice goes to the quad kernel's
            // 192-row form from N = 26624 above 8 rows, from N = 40960 at any height,
            // and above 128 rows (hot, bf16, K = 4096: 8x50264 129.3 -> 93.4 us,
            // 32x28672 57.6 -> 53.9, 64x28672 66.2 -> 54.2, 128x50264 205.9 -> 98.2,
            // 160x14336 71.5 -> 55.0, 160x50264 326.0 -> 102.9); below, the skinny
            // kernel stays (8x28672 49.7 against 54.0, 128x14336 46.8 against 54.6,
            // 48x24576 48.1 against 54.6).  The quad kernel's time follows its K walk and
            // the skinny kernel's B's bytes, so above 64 rows a K of at most 2048 also
            // goes to the quad kernel (100x20480x1024 27.2 -> 21.2 us, 96x24576x2048
            // 38.2 -> 32.6, 128x20480x2048 42.3 -> 32.3; at K = 4096 72x16384 37.0
            // against 54.0 and 80x12288 39.0 against 54.3 keep the skinny kernel)
            if (cfg.kernel == TGEMM_KERNEL_SKINNY && layout == TGEMM_B_KN && k >= 1024 &&
                n > kTableN[NN - 1] &&
                (m > 128 || n >= 40960 || (n >= 26624 && m > 8) || (m > 64 && k <= 2048)))
                cfg = kQuadRows192;
            return cfg;
        }
    }
    if (a_layout == TGEMM_A_MK && layout == TGEMM_B_KN && m <= 128 && k >= 1024) {
        const int mt = m <= 32 ? 1 : (m <= 64 ? 2 : 4);
        return tgemm_config{TGEMM_KERNEL_SKINNY, mt * 32, 32, 64, 1, 8, mt == 1 ? 4 : (mt == 2 ? 3 : 1),
                            1, 8, 32};
    }
    if (a_layout == TGEMM_A_MK && layout == TGEMM_B_NK && m <= 128 && k >= 1024) {
        const int mt = m <= 32 ? 1 : (m <= 64 ? 2 : 4);
        // 32- and 64-row blocks take 128-wide k chunks (256-byte row segments), one chunk
        // ahead (64-row blocks with four waves)
        if (mt == 1)
            return tgemm_config{TGEMM_KERNEL_SKINNY, 32, 32, 128, 1, 8, 1, 1, 8, 32};
        if (mt == 2)
            return tgemm_config{TGEMM_KERNEL_SKINNY, 64, 32, 128, 1, 4, 1, 1, 4, 32};
        return tgemm_config{TGEMM_KERNEL_SKINNY, 128, 32, 64, 1, 8, 1, 1, 8, 32};
    }
    const int64_t t256 = ((m + 255) / 256) * ((n + 255) / 256);
    const int64_t t128 = ((m + 127) / 128) * ((n + 127) / 128);
    if (t256 >= 192 && a_layout == TGEMM_A_MK && layout == TGEMM_B_NK)
        return tgemm_config{TGEMM_KERNEL_QUAD, 256, 256, 64, 2, 2, 5, 4, 1, 16};
    // A [K,M]: the quad kernel (32x32x16, transposing A reads) from 48 tiles of 256x256
    // up; measured against the ping-pong and tiled kernels it ran 24 % faster at 8192^3
    // and 17 % at 2048x2048x4096, and tied with the 128x128 tiled kernel at 32 tiles
    if (t256 >= 48 && a_layout == TGEMM_A_KM)
        return tgemm_config{TGEMM_KERNEL_QUAD, 256, 256, 64, 2, 2, 5, 4, 1, 32};
    if (t256 >= 192)
        return tgemm_config{TGEMM_KERNEL_PINGPONG, 256, 256, 64, 2, 4, 2, 4, 1, 32};
    if (t128 >= 128)
        return tgemm_config{TGEMM_KERNEL_TILED, 128, 128, 64, 2, 2, 2, 8, 1, 32};
    return tgemm_config{TGEMM_KERNEL_TILED, 64, 64, 64, 2, 2, 2, 8, 1, 32};
}

// The choice when the caller lends a workspace ("Tiling a matmul", section "Where it
// breaks": a product with few output tiles leaves compute units idle unless its K range
// is split).
//   - With B [N,K], M <= 64 or fewer than 16 tiles of 256x256: the split-K kernel's
//     64x128 tiles, up to 128 of them, else its 64x256 tiles, up to 128 of them (a 64-row
//     tile reads B once per 64 rows, so larger M goes to the quad kernel's 256-row tiles).
//     Streaming B from memory (operands past the last-level cache) at 64x28672x4096 the
//     wider tiles took 56.6 us against 88.4 without a workspace.
//   - Otherwise, up to 128 tiles of 256x256: the quad kernel in split-K mode, unless the
//     workspace-free choice already fills the chip and the splits would be shallow: with
//     more than 64 tiles each split must be at least 3072 deep; where that choice (a
//     tiled, ping-pong or quad kernel) has 256 workgroups or more, 2048; with B [N,K]
//     and 128 or more, 1024.
//   - The split count is the largest power of two within 256 / tiles (about one wave of
//     workgroups), 16, and K / 192 (three K steps per split): more splits add partial
//     traffic and fixed costs faster than parallelism.
//   - The skinny and direct kernels keep products with K <= 4096 and N <= 2048, where
//     their single pass is as fast, and the skinny kernel's 32-row blocks those whose
//     workgroups make one wave.
// Fitted on 102 random shapes (few to 144 tiles, K 2048-16384; every configuration and
// split counts 2-64 timed): the pick was within 5 % of the fastest on 88 and 1.5 %
// slower on average (at most 17 %).  The rules before, which left small-M products with
// B [K,N] and many mid-size ones unsplit, were 146 % slower on average on the 20 few-tile
// shapes where their pick was timed.  On 36 shapes drawn after the rule was fixed the
// pick was within 5 % of the fastest on 26, 3.8 % slower on average (at most 25 %).
int64_t pow2_at_most(int64_t x) {
    int64_t p = 1;
    while (p * 2 <= x)
        p *= 2;
    return p;
}

tgemm_config choose_ws(int dtype, int a_layout, int layout, int64_t m, int64_t n, int64_t k,
                       bool aligned) {
    const tgemm_config plain = choose(dtype, a_layout, layout, m, n, k, aligned);
    if (!aligned || a_layout != TGEMM_A_MK || k < 1024)
        return plain;
    if ((plain.kernel == TGEMM_KERNEL_SKINNY || plain.kernel == TGEMM_KERNEL_DIRECT) &&
        k <= 4096 && n <= 2048)
        return plain;
    // The skinny kernel's 64-column form (products past the grid's widest N) keeps its
    // plain launch: split-K over workgroups was slower on 6 of 9 shapes measured
    // (64x24576x8192 106.1 against 90.3 us, 8x32000x8192 109.9 against 95.1, 4x10240x4096
    // 20.3 against 17.0) and at most 4.5 us faster on the others (32x16384x8192 45.4
    // against 49.9, 48x20480x4096 34.1 against 37.7)
    if (plain.kernel == TGEMM_KERNEL_SKINNY && plain.block_n == 64)
        return plain;
    // A 32-row skinny product whose workgroups make one wave (192-256 of them) streams B
    // at the chip's rate on its own; split-K would add only its partials' traffic
    // (1-32 x 8192 x 8192: 23.4-24.8 against 25.4-26.7 us hot, 27.8-29.6 against
    // 36.4-37.8 us with operands past the last-level cache)
    if (plain.kernel == TGEMM_KERNEL_SKINNY && plain.block_m == 32) {
        const int64_t wgs = ((n + 31) / 32) * ((m + 31) / 32);
        if (wgs >= 192 && wgs <= 256)
            return plain;
    }
    const auto tiles = [&](int64_t bm, int64_t bn) {
        return ((m + bm - 1) / bm) * ((n + bn - 1) / bn);
    };
    const int64_t t256 = tiles(256, 256);
    const int64_t deep = pow2_at_most(k / 192);       // splits of at least 3 K steps
    if (layout == TGEMM_B_NK && (m <= 64 || t256 < 16)) {
        // 64-column-deep tiles 128 wide, or 256 wide where the narrow ones would exceed
        // 128; past that a wave of tiles needs no split
        const int32_t bn = tiles(64, 128) <= 128 ? 128 : 256;
        const int64_t t = tiles(64, bn);
        if (t > 128)
            return plain;
        int64_t splits = pow2_at_most(256 / t);
        splits = splits > 16 ? 16 : splits;
        splits = splits > deep ? deep : splits;
        splits = splits < 2 ? 2 : splits;
        return tgemm_config{TGEMM_KERNEL_SPLITK, 64, bn, 64, 1, 4, 4, 1, (int32_t)splits, 32};
    }
    if (t256 == 0 || t256 > 128)
        return plain;
    int64_t splits = pow2_at_most(256 / t256);
    splits = splits > 16 ? 16 : splits;
    splits = splits > deep ? deep : splits;
    if (splits < 2)
        return plain;
    const int64_t depth = k / splits;
    const bool full_tiles = plain.kernel == TGEMM_KERNEL_TILED ||
                            plain.kernel == TGEMM_KERNEL_PINGPONG ||
                            plain.kernel == TGEMM_KERNEL_QUAD;
    const int64_t plain_wgs = full_tiles ? tiles(plain.block_m, plain.block_n) : 0;
    if ((t256 > 64 && depth < 3072) || (plain_wgs >= 256 && depth < 2048) ||
        (layout == TGEMM_B_NK && plain_wgs >= 128 && depth < 1024))
        return plain;
    return tgemm_config{TGEMM_KERNEL_QUAD_SPLITK, 256, 256, 64, 2, 2, 5, 4, (int32_t)splits,
                        layout == TGEMM_B_NK ? 16 : 32};
}

// Workspace bytes of a configuration for an m x n product: the fp32 partial tiles of a
// split-K or stream-K configuration, nothing for the others.
int64_t workspace_bytes(const tgemm_config& cfg, int64_t m, int64_t n) {
    if (cfg.kernel == TGEMM_KERNEL_QUAD_STREAMK)
        return TGEMM_STREAMK_WORKSPACE_BYTES;
    return is_split(cfg.kernel) ? (int64_t)cfg.split_k * m * n * 4 : 0;
}

// One product as the caller described it.
struct Problem {
    int dtype;
    int64_t m, n, k;
    const void* A;
    int64_t lda;
    int a_layout;
    const void* B;
    int64_t ldb;
    int b_layout;
    void* C;
    int64_t ldc;
};

// Elements spanned by `rows` rows of `cols` elements, `ld` apart.
int64_t span(int64_t rows, int64_t cols, int64_t ld) {
    return rows > 0 && cols > 0 ? (rows - 1) * ld + cols : 0;
}
int64_t span_a(const Problem& p) {
    return p.a_layout == TGEMM_A_MK ? span(p.m, p.k, p.lda) : span(p.k, p.m, p.lda);
}
int64_t span_b(const Problem& p) {
    return p.b_layout == TGEMM_B_NK ? span(p.n, p.k, p.ldb) : span(p.k, p.n, p.ldb);
}
int64_t span_c(const Problem& p) { return span(p.m, p.n, p.ldc); }

int check_sizes(int dtype, int64_t m, int64_t n, int64_t k, int a_layout, int b_layout) {
    if (dtype != TGEMM_F16 && dtype != TGEMM_BF16)
        return TGEMM_ERR_INVALID_VALUE;
    if (a_layout != TGEMM_A_MK && a_layout != TGEMM_A_KM)
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

int check_problem(const Problem& p) {
    int rc = check_sizes(p.dtype, p.m, p.n, p.k, p.a_layout, p.b_layout);
    if (rc != TGEMM_OK)
        return rc;
    // a leading dimension covers at least the contiguous extent of a row (and is >= 1)
    const int64_t a_min = p.a_layout == TGEMM_A_MK ? p.k : p.m;
    const int64_t b_min = p.b_layout == TGEMM_B_NK ? p.k : p.n;
    if (p.lda < 1 || p.lda < a_min || p.ldb < 1 || p.ldb < b_min || p.ldc < 1 || p.ldc < p.n)
        return TGEMM_ERR_INVALID_VALUE;
    if (p.lda > kMaxElems || p.ldb > kMaxElems || p.ldc > kMaxElems)
        return TGEMM_ERR_UNSUPPORTED;
    // spans, computed only once every factor is known to fit (no int64 overflow)
    if (span_a(p) > kMaxElems || span_b(p) > kMaxElems || span_c(p) > kMaxElems)
        return TGEMM_ERR_UNSUPPORTED;
    return TGEMM_OK;
}

bool overlaps(const void* p, int64_t pbytes, const void* q, int64_t qbytes) {
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return pbytes > 0 && qbytes > 0 && a < b + (uintptr_t)qbytes && b < a + (uintptr_t)pbytes;
}

// The fast kernels read A and B through buffer resources whose range check rejects any
// offset with bit 31 set, which holds only for operands spanning at most 2^31 bytes; they
// move 16-byte pieces, so every contiguous extent and leading dimension is a multiple of
// 8 elements and every base address 16-byte aligned.  The masked kernel reads through
// the same resources, its buffers widened to the 16-byte blocks around each operand
// (up to 30 bytes more): it needs the span limit only, 32 bytes lower.
constexpr int64_t kMaxFastOperandBytes = int64_t(1) << 31;

bool buffer_reachable(const Problem& p) {
    return 2 * span_a(p) + 32 <= kMaxFastOperandBytes &&
           2 * span_b(p) + 32 <= kMaxFastOperandBytes;
}

bool fast_aligned(const Problem& p) {
    const auto al16 = [](const void* q) { return ((uintptr_t)q % 16) == 0; };
    return p.k % 8 == 0 && p.n % 8 == 0 && (p.a_layout == TGEMM_A_MK || p.m % 8 == 0) &&
           p.lda % 8 == 0 && p.ldb % 8 == 0 && p.ldc % 8 == 0 && al16(p.A) && al16(p.B) &&
           al16(p.C) && 2 * span_a(p) <= kMaxFastOperandBytes &&
           2 * span_b(p) <= kMaxFastOperandBytes;
}

// A [M,K] and B [N,K] alone meet those rules (C or N may not): the skinny kernels read
// only A and B through buffers and store C element by element where it is not aligned,
// so they serve such products as well (an odd vocabulary size, say).
bool operands_fast(const Problem& p) {
    const auto al16 = [](const void* q) { return ((uintptr_t)q % 16) == 0; };
    return p.a_layout == TGEMM_A_MK && p.b_layout == TGEMM_B_NK && p.k % 8 == 0 &&
           p.lda % 8 == 0 && p.ldb % 8 == 0 && al16(p.A) && al16(p.B) &&
           2 * span_a(p) <= kMaxFastOperandBytes && 2 * span_b(p) <= kMaxFastOperandBytes;
}

// Alignment classes of a call or a query: kAlignNone (the masked kernel's rules), kAlignAll
// (every fast-kernel rule), kAlignOperands (A and B meet them, C or N does not).
constexpr int kAlignNone = 0, kAlignAll = 1, kAlignOperands = 2;

// The choice for an alignment class: kAlignOperands takes the choice for aligned operands
// when that is a skinny kernel (A [M,K], B [N,K]), else the masked one.
tgemm_config choose_for(int dtype, int a_layout, int layout, int64_t m, int64_t n, int64_t k,
                        int align, bool with_ws) {
    if (align == kAlignAll)
        return with_ws ? choose_ws(dtype, a_layout, layout, m, n, k, true)
                       : choose(dtype, a_layout, layout, m, n, k, true);
    if (align == kAlignOperands && a_layout == TGEMM_A_MK && layout == TGEMM_B_NK) {
        const tgemm_config c = choose(dtype, a_layout, layout, m, n, k, true);
        if (c.kernel == TGEMM_KERNEL_SKINNY)
            return c;
        // past the grid's widest N, where aligned operands would take the quad kernel,
        // up to 64 rows keep the skinny kernel's 64-column form (8-64 x 50257 x 4096:
        // 84-115 us against 134-143 for the best masked tiling)
        constexpr int NN = sizeof(kTableN) / sizeof(kTableN[0]);
        if (m <= 64 && k >= 1024 && n > kTableN[NN - 1])
            return m <= 32 ? kSkinnyN64Rows32 : kSkinnyN64Rows64;
    }
    return with_ws ? choose_ws(dtype, a_layout, layout, m, n, k, false)
                   : choose(dtype, a_layout, layout, m, n, k, false);
}

// The device address of `scratch` on the current device, looked up once per device (with
// that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_at[kMaxDevices];

int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return TGEMM_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_at[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return TGEMM_ERR_DEVICE;
        g_scratch_at[dev] = p;
    }
    *out = g_scratch_at[dev];
    return TGEMM_OK;
}

// One product.  ws / ws_bytes: the caller's workspace (NULL: none).  use_scratch: the
// library's fixed scratch serves as the workspace instead (gemm_ex_noalloc).
int run(const Problem& p, const tgemm_config* cfg, void* ws, int64_t ws_bytes, void* stream,
        bool use_scratch = false) {
    int rc = check_problem(p);
    if (rc != TGEMM_OK)
        return rc;
    if (p.m == 0 || p.n == 0)
        return TGEMM_OK;
    if (!p.C || (p.k > 0 && (!p.A || !p.B)))
        return TGEMM_ERR_NULL_POINTER;
    if (((uintptr_t)p.C & 1) || ((uintptr_t)p.A & 1) || ((uintptr_t)p.B & 1))
        return TGEMM_ERR_ALIGNMENT;
    if (overlaps(p.C, 2 * span_c(p), p.A, 2 * span_a(p)) ||
        overlaps(p.C, 2 * span_c(p), p.B, 2 * span_b(p)))
        return TGEMM_ERR_ALIASING;
    const bool aligned = fast_aligned(p);
    const int align = aligned ? kAlignAll : (operands_fast(p) ? kAlignOperands : kAlignNone);
    tgemm_config use = cfg ? *cfg
                           : choose_for(p.dtype, p.a_layout, p.b_layout, p.m, p.n, p.k, align,
                                        ws || use_scratch);
    // the fixed scratch holds the skinny products' partials; a larger split goes plain
    if (!cfg && use_scratch && workspace_bytes(use, p.m, p.n) > kScratchBytes)
        use = choose_for(p.dtype, p.a_layout, p.b_layout, p.m, p.n, p.k, align, false);
    const bool reachable = buffer_reachable(p);
    if (!cfg && use.kernel == TGEMM_KERNEL_MASKED && !reachable)
        use = kGenericConfig;
    const Variant* v = find_variant(p.dtype, p.a_layout, p.b_layout, use);
    if (!v)
        return TGEMM_ERR_UNSUPPORTED;
    // the skinny kernels need A and B aligned only (B [N,K]); the other fast kernels need
    // every rule
    const bool operands_ok = use.kernel == TGEMM_KERNEL_SKINNY && align == kAlignOperands;
    if (use.kernel == TGEMM_KERNEL_MASKED
            ? !reachable
            : use.kernel != TGEMM_KERNEL_GENERIC && !aligned && !operands_ok)
        return TGEMM_ERR_ALIGNMENT;
    const int64_t need = workspace_bytes(use, p.m, p.n);
    if (use_scratch && need > 0) {
        if (need > kScratchBytes)
            return TGEMM_ERR_SCRATCH;
        rc = scratch_address(&ws);
        if (rc != TGEMM_OK)
            return rc;
        ws_bytes = kScratchBytes;
    }
    if (need > 0) {
        if (!ws || ws_bytes < need)
            return TGEMM_ERR_WORKSPACE;
        if ((uintptr_t)ws % 16 != 0)
            return TGEMM_ERR_ALIGNMENT;
        if (overlaps(ws, need, p.A, 2 * span_a(p)) || overlaps(ws, need, p.B, 2 * span_b(p)) ||
            overlaps(ws, need, p.C, 2 * span_c(p)))
            return TGEMM_ERR_ALIASING;
    }
    const int group_m = use.group_m > 0 ? use.group_m : v->cfg.group_m;
    (void)hipGetLastError();   // start from a clean error state for this launch
    const hipError_t e =
        v->split_launch
            ? v->split_launch(p.A, p.B, p.C, (int)p.m, (int)p.n, (int)p.k, (int)p.lda,
                              (int)p.ldb, (int)p.ldc, group_m, use.split_k, ws,
                              static_cast<hipStream_t>(stream))
            : v->launch(p.A, p.B, p.C, (int)p.m, (int)p.n, (int)p.k, (int)p.lda, (int)p.ldb,
                        (int)p.ldc, group_m, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TGEMM_OK : TGEMM_ERR_LAUNCH;
}

// A packed product: A [M,K], B [N,K] or [K,N], C [M,N], no padding between rows (an
// empty row length still gives a leading dimension of 1).
Problem packed(int dtype, int64_t m, int64_t n, int64_t k, const void* A, const void* B,
               void* C, int b_layout) {
    const auto ld = [](int64_t x) { return x > 1 ? x : int64_t(1); };
    return Problem{dtype,     m, n, k, A, ld(k), TGEMM_A_MK, B, ld(b_layout == TGEMM_B_KN ? n : k),
                   b_layout, C, ld(n)};
}

int query(int dtype, int64_t m, int64_t n, int64_t k, int a_layout, int b_layout, int aligned,
          tgemm_config* out, bool with_ws = false) {
    int rc = check_sizes(dtype, m, n, k, a_layout, b_layout);
    if (rc != TGEMM_OK)
        return rc;
    if (!out)
        return TGEMM_ERR_NULL_POINTER;
    const int align = aligned == kAlignOperands ? kAlignOperands
                                                : (aligned != 0 ? kAlignAll : kAlignNone);
    *out = choose_for(dtype, a_layout, b_layout, m, n, k, align, with_ws);
    const Variant* v = find_variant(dtype, a_layout, b_layout, *out);
    if (v)
        out->group_m = v->cfg.group_m;
    return TGEMM_OK;
}

int list(int dtype, int a_layout, int b_layout, tgemm_config* out, int capacity) {
    if (dtype != TGEMM_F16 && dtype != TGEMM_BF16)
        return TGEMM_ERR_INVALID_VALUE;
    if (a_layout != TGEMM_A_MK && a_layout != TGEMM_A_KM)
        return TGEMM_ERR_INVALID_VALUE;
    if (b_layout != TGEMM_B_NK && b_layout != TGEMM_B_KN)
        return TGEMM_ERR_INVALID_VALUE;
    if (capacity < 0 || (capacity > 0 && !out))
        return TGEMM_ERR_INVALID_VALUE;
    int count = 0;
    for (const Variant* v : registry()) {
        if (v->dtype != dtype || v->a_layout != a_layout || v->layout != b_layout)
            continue;
        if (count < capacity)
            out[count] = v->cfg;
        ++count;
    }
    return count;
}

// The engine-cycle counter is not one counter per chip, nor even per XCD: stamps of the
// same XCD taken on different compute units disagree.  So stamps are kept per compute
// unit: 4096 one-wave workgroups (about 16 per compute unit), each of whose first lanes
// writes its compute unit's engine-clock counter and the chip's constant-rate wall clock,
// as one 16-byte store, to slot (XCD id, hardware id bits 8..15: CU, SH and SE) of
// out[16 * 256][2].
constexpr int kStampSlots = 16 * 256;
static_assert(kStampSlots == TGEMM_CLOCK_STAMP_SLOTS, "stamp slots as documented");
constexpr int kStampBlocks = 4096;

__global__ void __launch_bounds__(64) clock_stamp_kernel(unsigned long long* out) {
    if (threadIdx.x == 0) {
        unsigned xcc, hw;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
        const unsigned slot = (xcc & 15) * 256 + ((hw >> 8) & 255);
        ulonglong2 v;
        v.x = (unsigned long long)clock64();
        v.y = (unsigned long long)wall_clock64();
        reinterpret_cast<ulonglong2*>(out)[slot] = v;
    }
}

}  // namespace

extern "C" {

int tgemm_clock_stamp(void* out, void* stream) {
    if (!out)
        return TGEMM_ERR_NULL_POINTER;
    if ((uintptr_t)out % 16 != 0)
        return TGEMM_ERR_ALIGNMENT;
    (void)hipGetLastError();
    hipLaunchKernelGGL(clock_stamp_kernel, dim3(kStampBlocks), dim3(64), 0,
                       static_cast<hipStream_t>(stream),
                       static_cast<unsigned long long*>(out));
    return hipGetLastError() == hipSuccess ? TGEMM_OK : TGEMM_ERR_LAUNCH;
}

int tgemm_wall_clock_hz(int64_t* hz) {
    if (!hz)
        return TGEMM_ERR_NULL_POINTER;
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
        khz <= 0)
        return TGEMM_ERR_DEVICE;
    *hz = (int64_t)khz * 1000;
    return TGEMM_OK;
}

int gemm_f16(int64_t m, int64_t n, int64_t k, const void* A, const void* B, void* C,
             int b_layout, void* stream) {
    return run(packed(TGEMM_F16, m, n, k, A, B, C, b_layout), nullptr, nullptr, 0, stream);
}

int gemm_bf16(int64_t m, int64_t n, int64_t k, const void* A, const void* B, void* C,
              int b_layout, void* stream) {
    return run(packed(TGEMM_BF16, m, n, k, A, B, C, b_layout), nullptr, nullptr, 0, stream);
}

int gemm_ex(int dtype, int64_t m, int64_t n, int64_t k, const void* A, const void* B, void* C,
            int b_layout, const tgemm_config* cfg, void* stream) {
    return run(packed(dtype, m, n, k, A, B, C, b_layout), cfg, nullptr, 0, stream);
}

int gemm_ex_ws(int dtype, int64_t m, int64_t n, int64_t k, const void* A, const void* B,
               void* C, int b_layout, const tgemm_config* cfg, void* workspace,
               int64_t workspace_bytes, void* stream) {
    if (workspace_bytes < 0)
        return TGEMM_ERR_INVALID_VALUE;
    return run(packed(dtype, m, n, k, A, B, C, b_layout), cfg, workspace, workspace_bytes,
               stream);
}

int gemm_ex_noalloc(int dtype, int64_t m, int64_t n, int64_t k, const void* A, const void* B,
                    void* C, int b_layout, const tgemm_config* cfg, void* stream) {
    return run(packed(dtype, m, n, k, A, B, C, b_layout), cfg, nullptr, 0, stream, true);
}

int gemm_strided(int dtype, int64_t m, int64_t n, int64_t k, const void* A, int64_t lda,
                 int a_layout, const void* B, int64_t ldb, int b_layout, void* C, int64_t ldc,
                 const tgemm_config* cfg, void* stream) {
    return run(Problem{dtype, m, n, k, A, lda, a_layout, B, ldb, b_layout, C, ldc}, cfg,
               nullptr, 0, stream);
}

int tgemm_query_config(int dtype, int64_t m, int64_t n, int64_t k, int b_layout,
                       tgemm_config* out) {
    // the packed problem at 16-byte-aligned addresses: the sizes decide alignment
    const int rc = check_sizes(dtype, m, n, k, TGEMM_A_MK, b_layout);
    if (rc != TGEMM_OK)
        return rc;
    const Problem p = packed(dtype, m, n, k, reinterpret_cast<const void*>(uintptr_t(256)),
                             reinterpret_cast<const void*>(uintptr_t(256)),
                             reinterpret_cast<void*>(uintptr_t(256)), b_layout);
    const int q = query(
        dtype, m, n, k, TGEMM_A_MK, b_layout,
        fast_aligned(p) ? kAlignAll : (operands_fast(p) ? kAlignOperands : kAlignNone), out);
    // as a call does: the masked kernel gives way to the generic one past its span limit
    if (q == TGEMM_OK && out->kernel == TGEMM_KERNEL_MASKED && !buffer_reachable(p))
        *out = kGenericConfig;
    return q;
}

int tgemm_query_config_ex(int dtype, int64_t m, int64_t n, int64_t k, int a_layout,
                          int b_layout, int aligned, tgemm_config* out) {
    return query(dtype, m, n, k, a_layout, b_layout, aligned, out);
}

int tgemm_query_config_ws(int dtype, int64_t m, int64_t n, int64_t k, int b_layout,
                          int aligned, tgemm_config* out, int64_t* workspace_bytes_out) {
    if (!workspace_bytes_out)
        return TGEMM_ERR_NULL_POINTER;
    const int rc = query(dtype, m, n, k, TGEMM_A_MK, b_layout, aligned, out, true);
    if (rc != TGEMM_OK)
        return rc;
    *workspace_bytes_out = workspace_bytes(*out, m, n);
    return TGEMM_OK;
}

int tgemm_workspace_size(int64_t m, int64_t n, const tgemm_config* cfg, int64_t* bytes) {
    if (!cfg || !bytes)
        return TGEMM_ERR_NULL_POINTER;
    if (m < 0 || n < 0)
        return TGEMM_ERR_INVALID_VALUE;
    if (is_split(cfg->kernel) && (cfg->split_k < 2 || cfg->split_k > kMaxSplits))
        return TGEMM_ERR_UNSUPPORTED;
    if (m > kMaxElems || n > kMaxElems || (n > 0 && m > kMaxElems / n))
        return TGEMM_ERR_UNSUPPORTED;
    *bytes = workspace_bytes(*cfg, m, n);
    return TGEMM_OK;
}

int tgemm_list_configs(int dtype, int b_layout, tgemm_config* out, int capacity) {
    return list(dtype, TGEMM_A_MK, b_layout, out, capacity);
}

int tgemm_list_configs_ex(int dtype, int a_layout, int b_layout, tgemm_config* out,
                          int capacity) {
    return list(dtype, a_layout, b_layout, out, capacity);
}

const char* tgemm_status_string(int status) {
    switch (status) {
    case TGEMM_OK: return "TGEMM_OK";
    case TGEMM_ERR_INVALID_VALUE:
        return "TGEMM_ERR_INVALID_VALUE: bad size, leading dimension, dtype or layout";
    case TGEMM_ERR_NULL_POINTER: return "TGEMM_ERR_NULL_POINTER: NULL operand";
    case TGEMM_ERR_ALIGNMENT: return "TGEMM_ERR_ALIGNMENT: operand alignment not supported";
    case TGEMM_ERR_ALIASING: return "TGEMM_ERR_ALIASING: C overlaps A or B";
    case TGEMM_ERR_UNSUPPORTED: return "TGEMM_ERR_UNSUPPORTED: size or configuration not supported";
    case TGEMM_ERR_LAUNCH: return "TGEMM_ERR_LAUNCH: kernel launch failed";
    case TGEMM_ERR_DEVICE: return "TGEMM_ERR_DEVICE: device query failed";
    case TGEMM_ERR_WORKSPACE:
        return "TGEMM_ERR_WORKSPACE: the configuration needs a larger workspace";
    case TGEMM_ERR_SCRATCH:
        return "TGEMM_ERR_SCRATCH: the configuration needs more than the library's fixed "
               "16 MiB scratch (gemm_ex_noalloc)";
    default: return "unknown tgemm status";
    }
}

int tgemm_version(void) { return 300; }

}  // extern "C"
