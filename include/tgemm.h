/*
 * libtgemm -- block-tiled dense matrix multiply for AMD Instinct MI355X (gfx950).
 *
 *   C[m,n] = sum_{k<K} a(m,k) * b(n,k)
 *     a(m,k) = A[m*lda + k]  (A stored [M,K], K contiguous; the packed entry points)
 *     a(m,k) = A[k*lda + m]  (A stored [K,M], M contiguous; gemm_strided, TGEMM_A_KM)
 *     b_layout TGEMM_B_NK: B stored [N,K] row-major (K contiguous), b(n,k) = B[n*ldb+k],
 *                          so C = A x B^T ("0. A Minimal Hopper Matmul", Tilus tutorial,
 *                          section "Block Tiling": A (M,K), B (N,K), C (M,N), both K-major)
 *     b_layout TGEMM_B_KN: B stored [K,N] row-major (N contiguous), b(n,k) = B[k*ldb+n],
 *                          so C = A x B ("Tiling a matmul", section "Code"; "TileLang: a
 *                          tile language one level below Triton", section "The first
 *                          kernel: GEMM", where B is a (K,N) tensor)
 *   and C[m,n] is stored at C[m*ldc + n].  gemm_f16, gemm_bf16 and gemm_ex take packed
 *   operands (lda = K, ldb = K or N, ldc = N); gemm_strided takes leading dimensions
 *   and either storage of A (operands may be K- or MN-contiguous: Tilus tutorial,
 *   section "Block Tiling").
 *
 * Inputs are IEEE binary16 (f16) or bfloat16 (bf16); products are summed in fp32 and the
 * fp32 sum is rounded once, to nearest-even, to the same 16-bit type for C (the fp32
 * accumulator and the single cast in the epilogue of the Tilus tutorial, sections "The
 * Full Kernel" and "Epilogue").  The summation order is the kernel's own: results agree
 * with an exact sum to within fp32 rounding, not bit for bit.
 *
 * Conventions shared by every entry point:
 *   - Ownership: the caller allocates A, B and C (and the workspace of gemm_ex_ws) in
 *     device memory and keeps ownership.  The library allocates no device memory and
 *     keeps no pointer after the call returns.  C is fully overwritten (no alpha/beta).
 *   - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns at once.  Faults during execution surface at the caller's
 *     next synchronisation with that stream, as for any HIP launch.
 *   - Errors: a negative status; all argument checks run before anything is enqueued, and
 *     a failed check enqueues nothing.  Nothing aborts or exits.
 *   - Degenerate shapes: M == 0 or N == 0 is a no-op returning TGEMM_OK; K == 0 writes
 *     +0.0 (the empty sum) to all of C.
 *   - Alignment: any 2-byte-aligned pointers, sizes and leading dimensions are accepted.
 *     The fast kernels need A, B, C 16-byte aligned, K, N, lda, ldb and ldc multiples of
 *     8, M a multiple of 8 when A is [K,M], and A and B each spanning at most 2^31 bytes;
 *     the skinny kernels (A [M,K], B [N,K]) need those rules of A and B only, and store C
 *     element by element where C or N breaks them.  Other calls run the same tiles with
 *     masked loads and element-wise stores (TGEMM_KERNEL_MASKED), or, when A or B spans
 *     more than 2^31 - 32 bytes, a slower generic kernel; the arithmetic is the same.
 *   - Limits: M, N, K < 2^31, M*K, N*K, M*N < 2^31, and the element span of each operand
 *     ((rows - 1) * ld + row length) < 2^31 (TGEMM_ERR_UNSUPPORTED).
 *   - Aliasing: the span of C may not overlap the span of A or B (TGEMM_ERR_ALIASING).
 *     A and B may overlap.
 *   - Thread safety: the configuration table is read-only; calls from several host
 *     threads are safe.  Calls on one stream execute in order.
 */
#ifndef TGEMM_H
#define TGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { TGEMM_F16 = 0, TGEMM_BF16 = 1 } tgemm_dtype;

typedef enum {
    TGEMM_B_NK = 0, /* B is [N,K], K contiguous: C = A x B^T */
    TGEMM_B_KN = 1  /* B is [K,N], N contiguous: C = A x B   */
} tgemm_b_layout;

typedef enum {
    TGEMM_A_MK = 0, /* A is [M,K], K contiguous (the packed entry points) */
    TGEMM_A_KM = 1  /* A is [K,M], M contiguous                           */
} tgemm_a_layout;

typedef enum {
    TGEMM_OK = 0,
    TGEMM_ERR_INVALID_VALUE = -1, /* negative size, unknown dtype or layout, or a
                                     leading dimension below its row length (or < 1)    */
    TGEMM_ERR_NULL_POINTER = -2,  /* A, B or C NULL for a non-empty product            */
    TGEMM_ERR_ALIGNMENT = -3,     /* a pointer not 2-byte aligned, or an explicit fast
                                     configuration given operands it cannot take        */
    TGEMM_ERR_ALIASING = -4,      /* C's span overlaps A's or B's                       */
    TGEMM_ERR_UNSUPPORTED = -5,   /* sizes past the limits, or a configuration that is
                                     not compiled into the library                      */
    TGEMM_ERR_LAUNCH = -6,        /* the HIP launch was refused (no gfx950 device...)   */
    TGEMM_ERR_DEVICE = -7,        /* the current device could not be queried            */
    TGEMM_ERR_WORKSPACE = -8,     /* the configuration needs a workspace and none, or
                                     too small a one, was given                         */
    TGEMM_ERR_SCRATCH = -9        /* gemm_ex_noalloc: the configuration needs more than
                                     the library's fixed scratch (TGEMM_SCRATCH_BYTES)  */
} tgemm_status;

/* Workspace of a TGEMM_KERNEL_QUAD_STREAMK configuration: two 256x256 fp32 partial
 * tiles for each of its 256 workgroups, 128 MiB, whatever the shape. */
#define TGEMM_STREAMK_WORKSPACE_BYTES (128ll << 20)

/* Size of the fixed per-GPU scratch that gemm_ex_noalloc uses: 16 MiB. */
#define TGEMM_SCRATCH_BYTES (16ll << 20)

/* Kernel families in the library. */
typedef enum {
    TGEMM_KERNEL_GENERIC = 0, /* any alignment and size: element loads, one LDS stage    */
    TGEMM_KERNEL_TILED = 1,   /* 128-bit loads, register prefetch, two swizzled LDS
                                 stages, MFMA 32x32x16, grouped XCD-aware tile order     */
    TGEMM_KERNEL_SKINNY = 2,  /* small M: the K range of a tile split over the waves of a
                                 workgroup and summed in LDS (either B storage)           */
    TGEMM_KERNEL_DMA = 3,     /* A [M,K], B [N,K] only: global loads written straight into
                                 a deep ring of swizzled LDS stages (no register staging) */
    TGEMM_KERNEL_PINGPONG = 4,/* 8 waves, two per SIMD, alternating between operand fetch
                                 and back-to-back MFMAs half a period apart; direct-to-LDS
                                 loads; [K,N] B and [K,M] A through transposing reads    */
    TGEMM_KERNEL_QUAD = 5,    /* one wave per SIMD, each owning a 128x128 quadrant of a
                                 256x256 tile (or 96x128 of 192x256); direct-to-LDS loads
                                 into three A and two B slots, one barrier per K step;
                                 [K,N] B and [K,M] A through transposing reads          */
    TGEMM_KERNEL_SPLITK = 6,  /* A [M,K], B [N,K] only, with a workspace: the K range of
                                 each C tile split over split_k workgroups (direct-to-LDS
                                 ring), fp32 partial tiles in the workspace, summed in
                                 split order and cast by a second kernel               */
    TGEMM_KERNEL_DIRECT = 7,  /* A [M,K], B [N,K] only, small products: 32x32 C tiles, the
                                 K range split over the split_k = 4 waves of a workgroup,
                                 MFMA operands loaded from global memory straight into
                                 registers, partial tiles added in LDS                  */
    TGEMM_KERNEL_QUAD_SPLITK = 8,/* A [M,K], with a workspace: the quad kernel's 256x256
                                 tiles, the K range of each split over split_k
                                 workgroups, fp32 partial tiles in the workspace, summed
                                 in split order and cast by a second kernel            */
    TGEMM_KERNEL_QUAD_STREAMK = 9,/* A [M,K], with a workspace: the tile rows that fill
                                 whole waves of 256x256 tiles as a plain quad product,
                                 the rest by stream-K (256 workgroups, equal contiguous
                                 shares of the remaining tiles' K steps, at most two
                                 tile segments each, fp32 partial tiles in the
                                 workspace) and a reduction in workgroup order        */
    TGEMM_KERNEL_MASKED = 10  /* the TILED kernel for operands of any 2-byte alignment
                                 and any sizes (A and B each at most 2^31 - 32 bytes):
                                 K-contiguous tile rows read as the aligned 16-byte
                                 blocks around each piece and realigned in registers,
                                 [K,M] A and [K,N] B as 2-byte elements, every element
                                 masked by its own position; C stored element by
                                 element                                                */
} tgemm_kernel;

/* One tile configuration.  block_m x block_n is the C tile of one workgroup, block_k
 * the K step (SKINNY: the k chunk a wave loads at once, 64 or 128), waves_m x waves_n the wavefront grid inside the workgroup (64 lanes each),
 * stages the LDS buffers (QUAD: operand slots of block_m x block_k elements, three for
 * A tiles and two for B tiles), group_m the tile rows of one launch-order group,
 * split_k the number of waves (SKINNY) or workgroups (SPLITK and QUAD_SPLITK, 2..64,
 * chosen per call)
 * that share one C tile's K range (else 1), and mfma the matrix instruction's block
 * size: 32 (32x32x16) or 16 (16x16x32). */
typedef struct {
    int32_t kernel;
    int32_t block_m, block_n, block_k;
    int32_t waves_m, waves_n;
    int32_t stages;
    int32_t group_m;
    int32_t split_k;
    int32_t mfma;
} tgemm_config;

/*
 * C = A x B^T (TGEMM_B_NK) or A x B (TGEMM_B_KN) for fp16 inputs and output.
 *   m, n, k   : sizes (>= 0)
 *   A         : device pointer, m*k halves, row-major [m,k]
 *   B         : device pointer, n*k halves, [n,k] or [k,n] per b_layout
 *   C         : device pointer, m*n halves, row-major [m,n]; written, never read
 *   b_layout  : tgemm_b_layout
 *   stream    : hipStream_t to enqueue on (NULL = null stream)
 * Returns a tgemm_status.  The configuration comes from the library's table.
 */
int gemm_f16(int64_t m, int64_t n, int64_t k, const void* A, const void* B, void* C,
             int b_layout, void* stream);

/* The same for bfloat16 inputs and output. */
int gemm_bf16(int64_t m, int64_t n, int64_t k, const void* A, const void* B, void* C,
              int b_layout, void* stream);

/*
 * The same product with an explicit dtype (tgemm_dtype) and, optionally, an explicit
 * configuration (cfg == NULL: the table's choice).  A configuration must be one that
 * tgemm_list_configs reports (else TGEMM_ERR_UNSUPPORTED); a fast-kernel configuration
 * given operands that break its alignment rules fails with TGEMM_ERR_ALIGNMENT (a
 * TGEMM_KERNEL_SKINNY configuration with B [N,K] checks A and B only).  This is
 * the entry point of the tile-configuration sweep.
 */
int gemm_ex(int dtype, int64_t m, int64_t n, int64_t k, const void* A, const void* B,
            void* C, int b_layout, const tgemm_config* cfg, void* stream);

/*
 * gemm_ex with a workspace lent by the caller, for configurations that need one
 * (TGEMM_KERNEL_SPLITK and TGEMM_KERNEL_QUAD_SPLITK: split_k * m * n * 4 bytes of fp32
 * partial tiles; TGEMM_KERNEL_QUAD_STREAMK: TGEMM_STREAMK_WORKSPACE_BYTES).  Split-K over
 * workgroups follows "Tiling a matmul", section "Where it breaks": a product with few
 * output tiles (small or skinny) leaves compute units idle unless K is split.
 *   workspace       : device pointer, 16-byte aligned, not overlapping A, B or C; its
 *                     contents on entry do not matter and are overwritten; the caller
 *                     keeps ownership and must not reuse it until the stream has run
 *                     this call (two calls in flight on one workspace race)
 *   workspace_bytes : its size in bytes (>= 0)
 *   cfg             : NULL = the table's choice given a workspace (see
 *                     tgemm_query_config_ws), else as for gemm_ex; a split-K configuration
 *                     (SPLITK, QUAD_SPLITK) names its split count in split_k
 * Errors as gemm_ex, plus TGEMM_ERR_WORKSPACE (workspace NULL or smaller than the
 * configuration needs), TGEMM_ERR_ALIGNMENT (workspace not 16-byte aligned) and
 * TGEMM_ERR_ALIASING (workspace overlapping an operand).  A configuration that needs no
 * workspace ignores it.
 */
int gemm_ex_ws(int dtype, int64_t m, int64_t n, int64_t k, const void* A, const void* B,
               void* C, int b_layout, const tgemm_config* cfg, void* workspace,
               int64_t workspace_bytes, void* stream);

/*
 * gemm_ex_ws without a caller workspace and without any allocation, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The split-K partial tiles go to a fixed scratch
 * array inside the library: TGEMM_SCRATCH_BYTES of device memory per GPU, set aside when
 * the library's code is loaded on that GPU and held until the process ends.  Nothing is
 * allocated by the call (no hipMalloc, no hipFree); the first call on a device looks up
 * that device's scratch address and keeps it.
 *   arguments as for gemm_ex; cfg == NULL takes the table's choice given a workspace (as
 *   gemm_ex_ws does) when its partial tiles fit TGEMM_SCRATCH_BYTES, else the
 *   choice without a workspace
 * Errors as gemm_ex_ws, plus TGEMM_ERR_SCRATCH when an explicit configuration needs more
 * than TGEMM_SCRATCH_BYTES (split_k * m * n * 4 bytes for the split-K kernels) and
 * TGEMM_ERR_DEVICE
 * when the scratch address cannot be found.  Results are bit for bit those of gemm_ex_ws
 * with the same configuration.  Every call on one GPU uses that GPU's one scratch array:
 * nothing in it needs to start at zero (each call overwrites what it reads), but two
 * calls whose kernels overlap in time on one GPU (different streams, other host threads)
 * race on it; calls in order on one stream do not.
 */
int gemm_ex_noalloc(int dtype, int64_t m, int64_t n, int64_t k, const void* A, const void* B,
                    void* C, int b_layout, const tgemm_config* cfg, void* stream);

/*
 * The general product: either storage of A, either storage of B, leading dimensions.
 *   A        : device pointer; a_layout TGEMM_A_MK: a(m,k) = A[m*lda + k] (lda >= k);
 *              TGEMM_A_KM: a(m,k) = A[k*lda + m] (lda >= m)
 *   B        : device pointer; TGEMM_B_NK: b(n,k) = B[n*ldb + k] (ldb >= k);
 *              TGEMM_B_KN: b(n,k) = B[k*ldb + n] (ldb >= n)
 *   C        : device pointer; C[m*ldc + n] (ldc >= n); elements between rows are left
 *              untouched
 *   lda, ldb, ldc are in elements and at least 1.  cfg as for gemm_ex (NULL = table);
 *   the configurations are those tgemm_list_configs_ex reports for the two layouts.
 * Returns a tgemm_status.
 */
int gemm_strided(int dtype, int64_t m, int64_t n, int64_t k, const void* A, int64_t lda,
                 int a_layout, const void* B, int64_t ldb, int b_layout, void* C,
                 int64_t ldc, const tgemm_config* cfg, void* stream);

/* The configuration gemm_f16 / gemm_bf16 / gemm_ex(cfg = NULL) pick for this packed
 * problem (A [M,K], B per b_layout, C [M,N], no padding) with operands at 16-byte-aligned
 * addresses, written to *out; whether the fast kernels can take it follows from the sizes
 * (K and N multiples of 8, A and B each at most 2^31 bytes; with B [N,K] and only N off a
 * multiple of 8, a skinny configuration where the aligned choice is one; else the masked
 * kernel, or the generic one past 2^31 - 32 bytes).  Host-only: it touches no
 * device.  Returns TGEMM_OK, TGEMM_ERR_NULL_POINTER (out NULL) or the size, dtype and
 * layout errors of gemm_ex. */
int tgemm_query_config(int dtype, int64_t m, int64_t n, int64_t k, int b_layout,
                       tgemm_config* out);

/* The configurations compiled into the library for (dtype, b_layout).  Writes up to
 * `capacity` entries to `out` (which may be NULL when capacity is 0) and returns the
 * total count, or a negative status.  Host-only. */
int tgemm_list_configs(int dtype, int b_layout, tgemm_config* out, int capacity);

/* The choice for either storage of A (tgemm_a_layout) and a caller-stated alignment:
 * `aligned` 1 (or any value but 0 and 2) says the operands meet every fast-kernel rule
 * (16-byte-aligned addresses, sizes and leading dimensions multiples of 8, spans within
 * 2^31 bytes); 0 that they do not (the choice is then a TGEMM_KERNEL_MASKED
 * configuration; a call whose A or B spans more than 2^31 - 32 bytes runs the generic
 * kernel instead, which this query cannot see); 2 that A [M,K] and B [N,K] meet the rules
 * but C or N does not (an odd N, say): then a call takes the aligned choice where that is
 * a TGEMM_KERNEL_SKINNY configuration (the skinny kernels store C element by element
 * where it is not aligned), else the masked one.  The list for either storage of A;
 * tgemm_list_configs answers for TGEMM_A_MK. */
int tgemm_query_config_ex(int dtype, int64_t m, int64_t n, int64_t k, int a_layout,
                          int b_layout, int aligned, tgemm_config* out);
int tgemm_list_configs_ex(int dtype, int a_layout, int b_layout, tgemm_config* out,
                          int capacity);

/* The configuration the table picks when the caller can lend a workspace (A [M,K]), and
 * the workspace bytes it needs (0 when it needs none).  Only for K >= 1024 and aligned
 * operands: with B [N,K] and M <= 64 (or fewer than 16 tiles of 256x256), split-K over
 * workgroups with 64x128 tiles when there are at most 128 of them, else 64x256 tiles
 * when there are at most 128 of those; otherwise the quad
 * kernel's split-K when there are at most 128 tiles of 256x256; in both cases the split
 * count is the power of two at most 256 / tiles (at most 16, and K / split at least 192).
 * Shallow splits where the choice without a workspace already fills the chip keep that
 * choice, as do short-K skinny products (K <= 4096, N <= 2048) and products of at most 32
 * rows whose skinny workgroups make one wave (192-256 of them).  Host-only. */
int tgemm_query_config_ws(int dtype, int64_t m, int64_t n, int64_t k, int b_layout,
                          int aligned, tgemm_config* out, int64_t* workspace_bytes);

/* Workspace bytes a configuration needs for an m x n product (0 for all but SPLITK,
 * QUAD_SPLITK and QUAD_STREAMK).
 * Host-only. */
int tgemm_workspace_size(int64_t m, int64_t n, const tgemm_config* cfg, int64_t* bytes);

/*
 * Attention forward, fp16 ("TileLang: a tile language one level below Triton", section
 * "FlashAttention: online softmax as tile code"):
 *   O[b,i,h,:] = sum_j softmax_j( Q[b,i,h,:] . K[b,j,h,:] / sqrt(dim) ) V[b,j,h,:]
 * over the keys j < seq, or j <= i when causal is 1, per batch b and head h.
 *   batch, seq, heads, dim : sizes (>= 0); dim must be 64; batch and heads at most 65535
 *   Q, K, V                : device pointers, fp16, each [batch, seq, heads, dim]
 *                            (dim contiguous), 16-byte aligned
 *   O                      : device pointer, same shape and alignment; written, never
 *                            read; may not overlap Q, K or V
 *   causal                 : 0 (every key) or 1 (keys up to the query's own position)
 *   stream                 : hipStream_t (NULL = null stream)
 * The scores and the softmax run in fp32 (base-2 exponentials, log2(e) folded into the
 * scale), the probabilities are cast to fp16 for the product with V (fp32 sums), and
 * each output is divided by its row sum and rounded once to fp16.  Returns a
 * tgemm_status: TGEMM_ERR_INVALID_VALUE (negative size, causal not 0 or 1),
 * TGEMM_ERR_UNSUPPORTED (dim != 64, or a tensor over 2^31 bytes), TGEMM_ERR_NULL_POINTER,
 * TGEMM_ERR_ALIGNMENT, TGEMM_ERR_ALIASING, TGEMM_ERR_LAUNCH.  An empty tensor (batch,
 * seq or heads 0) is a no-op.  Same ownership, stream and thread-safety rules as the
 * products; nothing is allocated.
 */
int attn_fwd_f16(int64_t batch, int64_t seq, int64_t heads, int64_t dim, const void* Q,
                 const void* K, const void* V, void* O, int causal, void* stream);

/*
 * Diagnostics for measurements: clock stamps on every compute unit.  Engine cycles are
 * counted per compute unit (counters of different units are not aligned with each
 * other), at the clock of the die the unit sits on; the wall clock runs at a constant
 * rate.  A small kernel on `stream` (4096 one-wave workgroups, about 16 per compute unit)
 * writes, for the compute unit with slot s = 256 * XCD id + (hardware id bits 8..15),
 * its engine-clock counter to out[2s] and the wall clock to out[2s + 1].
 *   out    : device pointer to 4096 x 2 uint64 (64 KiB), 16-byte aligned; a slot whose
 *            compute unit ran none of the workgroups keeps its previous contents, so
 *            clear it first (slots no compute unit maps to are never written)
 *   stream : hipStream_t (NULL = null stream)
 * Two stamps around a stretch of work on one stream give each compute unit's average
 * engine clock: (after[2s] - before[2s]) / (after[2s+1] - before[2s+1]) *
 * tgemm_wall_clock_hz, for the slots written by both.
 * Returns TGEMM_OK, TGEMM_ERR_NULL_POINTER, TGEMM_ERR_ALIGNMENT or TGEMM_ERR_LAUNCH.
 * Nothing is allocated.
 */
#define TGEMM_CLOCK_STAMP_SLOTS 4096
int tgemm_clock_stamp(void* out, void* stream);

/* The rate of the wall clock that tgemm_clock_stamp reads, in Hz, for the current
 * device (written to *hz).  Returns TGEMM_OK, TGEMM_ERR_NULL_POINTER or TGEMM_ERR_DEVICE. */
int tgemm_wall_clock_hz(int64_t* hz);

/* A static, human-readable name for a status code. */
const char* tgemm_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int tgemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TGEMM_H */
