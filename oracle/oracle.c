/*
 * CPU oracle for the block-tiled dense matrix multiply (and, at the end of this file, the
 * attention forward pass built on the same tiles).  TEST INFRASTRUCTURE ONLY:
 * the test suite, the smoke check and the CPU-baseline leg of the benchmark are the
 * only callers.  It shares no code, header, table or helper with the GPU library.
 *
 * What it computes (the plain definition, no tiling, fusion or reordering):
 *
 *   C[m,n] = round_out( sum_{k=0}^{K-1} a(m,k) * b(n,k) )
 *
 *   a(m,k) = A[m*K + k]                      A stored [M,K], K contiguous
 *   b(n,k) = B[n*K + k]   (layout NK = 0)    B stored [N,K], K contiguous: C = A x B^T
 *   b(n,k) = B[k*N + n]   (layout KN = 1)    B stored [K,N], N contiguous: C = A x B
 *
 * Sources:
 *   - "0. A Minimal Hopper Matmul" (Tilus tutorial), section "Block Tiling": the product
 *     C = A x B^T with A (M,K), B (N,K), C (M,N); section "The Full Kernel" / "Epilogue":
 *     an fp32 accumulator cast once to the 16-bit output type.
 *   - "Tiling a matmul" (H. Sonawane), section "Code": the naive product sums a(i,k)*b(k,j)
 *     over k with B indexed [k][j], i.e. the [K,N] storage.
 *   - "TileLang: a tile language one level below Triton", section "The first kernel: GEMM":
 *     B given as a (K, N) tensor.
 *
 * Precision (chosen for the oracle, stricter than the kernels): every 16-bit input is
 * decoded exactly to fp64, each product is exact in fp64 (at most 22 significant bits),
 * the sum runs strictly in increasing k from +0.0 with one rounded add per term, and the
 * fp64 sum is rounded ONCE to the output format with round-to-nearest-even (no detour
 * through fp32, which would round twice).  Built with -ffp-contract=off and without
 * -ffast-math so the compiler keeps that order.  Threads split the output elements only;
 * every element keeps its own k order, so results do not depend on the thread count.
 *
 * K == 0 gives +0.0 (the empty sum).  M == 0 or N == 0 computes nothing.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F16 = 0, ORC_BF16 = 1 };
enum { ORC_B_NK = 0, ORC_B_KN = 1 };
enum { ORC_OK = 0, ORC_EINVAL = -1, ORC_ENOMEM = -2 };

/* ------------------------------------------------------------------------------------ */
/* 16-bit formats -> fp64, exactly, from the bit fields.                                 */
/* ------------------------------------------------------------------------------------ */

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double decode_f16(uint16_t h) {
    int sign = h >> 15;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);                 /* zero or subnormal: frac * 2^-24 */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(frac | 0x400), expo - 25); /* 1.frac * 2^(expo-15) */
    return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32 (1 sign, 8 exponent bits with bias
 * 127, 7 fraction bits). */
static double decode_bf16(uint16_t b) {
    int sign = b >> 15;
    int expo = (b >> 7) & 0xff;
    int frac = b & 0x7f;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -133);                /* zero or subnormal: frac * 2^-133 */
    else if (expo == 255)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(frac | 0x80), expo - 134); /* 1.frac * 2^(expo-127) */
    return sign ? -v : v;
}

/* ------------------------------------------------------------------------------------ */
/* fp64 -> 16-bit format, round to nearest, ties to even, from the fp64 bit pattern.      */
/*   frac_bits : stored fraction bits (10 for fp16, 7 for bf16)                          */
/*   bias      : exponent bias (15, 127)                                                 */
/*   exp_field_max : all-ones exponent field (31, 255)                                   */
/* ------------------------------------------------------------------------------------ */
static uint16_t encode_rne(double x, int frac_bits, int bias, int exp_field_max) {
    uint64_t u;
    memcpy(&u, &x, sizeof u);
    const uint16_t sign = (uint16_t)((u >> 63) << 15);
    const uint64_t mag = u & 0x7fffffffffffffffULL;
    const uint16_t inf_bits = (uint16_t)(exp_field_max << frac_bits);
    if (mag > 0x7ff0000000000000ULL) /* NaN stays NaN (quiet, payload not kept) */
        return sign | inf_bits | (uint16_t)(1u << (frac_bits - 1));
    if (mag == 0x7ff0000000000000ULL)
        return sign | inf_bits;
    const int e64 = (int)(mag >> 52);
    if (e64 == 0) /* zero, or an fp64 subnormal: far below half the smallest output step */
        return sign;
    const uint64_t sig = (mag & 0x000fffffffffffffULL) | (1ULL << 52); /* 53-bit significand */
    const int e = e64 - 1023;           /* x = sig * 2^(e-52) */
    const int emin = 1 - bias;          /* smallest normal exponent of the output format */
    /* Output step (unit in the last place) at this magnitude: 2^q. */
    const int q = (e < emin) ? (emin - frac_bits) : (e - frac_bits);
    const int shift = q - (e - 52);     /* bits of sig below the output step; >= 52-frac_bits */
    if (shift >= 54)                    /* |x| < 2^(q-1): below half a step, rounds to zero */
        return sign;
    uint64_t r = sig >> shift;
    const uint64_t rem = sig & ((1ULL << shift) - 1);
    const uint64_t half = 1ULL << (shift - 1);
    if (rem > half || (rem == half && (r & 1)))
        r += 1;
    /* r = |rounded x| / 2^q */
    const uint64_t hidden = 1ULL << frac_bits;
    if (e < emin) {
        /* Subnormal range.  r <= hidden; r == hidden is exactly the smallest normal, whose
         * encoding (exponent field 1, fraction 0) is the same integer. */
        return sign | (uint16_t)r;
    }
    int e_out = e;
    if (r == (hidden << 1)) { /* rounding carried into the next binade */
        r = hidden;
        e_out += 1;
    }
    if (e_out + bias >= exp_field_max) /* overflow: IEEE rounding sends it to infinity */
        return sign | inf_bits;
    return sign | (uint16_t)((e_out + bias) << frac_bits) | (uint16_t)(r - hidden);
}

static uint16_t encode_f16(double x) { return encode_rne(x, 10, 15, 31); }
static uint16_t encode_bf16(double x) { return encode_rne(x, 7, 127, 255); }

static double decode(int dtype, uint16_t v) {
    return dtype == ORC_F16 ? decode_f16(v) : decode_bf16(v);
}
static uint16_t encode(int dtype, double x) {
    return dtype == ORC_F16 ? encode_f16(x) : encode_bf16(x);
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Bulk codec entry points (exposed so the tests can check them exhaustively). */
int oracle_decode(int dtype, const uint16_t* in, double* out, int64_t count) {
    if (dtype != ORC_F16 && dtype != ORC_BF16)
        return ORC_EINVAL;
    for (int64_t i = 0; i < count; ++i)
        out[i] = decode(dtype, in[i]);
    return ORC_OK;
}

int oracle_encode(int dtype, const double* in, uint16_t* out, int64_t count) {
    if (dtype != ORC_F16 && dtype != ORC_BF16)
        return ORC_EINVAL;
    for (int64_t i = 0; i < count; ++i)
        out[i] = encode(dtype, in[i]);
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------ */
/* The sum itself, on fp64 operands.  A is [M,K]; Bnk holds b(n,k) at n*K + k.           */
/* Rows [m_lo, m_hi) of the fp64 sums are written to S (row-major [m_hi-m_lo, N]).        */
/* ------------------------------------------------------------------------------------ */
static void sum_rows(int64_t m_lo, int64_t m_hi, int64_t N, int64_t K, const double* A,
                     const double* Bnk, double* S) {
    const int64_t rows = m_hi - m_lo;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t n = 0; n < N; ++n) {
            const double* a = A + (m_lo + i) * K;
            const double* b = Bnk + n * K;
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += a[k] * b[k];
            S[i * N + n] = s;
        }
    }
}

/* b(n,k) for both storage orders, gathered into a [N,K] fp64 array (exact). */
static void gather_b(int dtype, int64_t N, int64_t K, const uint16_t* B, int b_layout,
                     double* Bnk) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            Bnk[n * K + k] = decode(dtype, b_layout == ORC_B_NK ? B[n * K + k] : B[k * N + n]);
}

static int check_common(int dtype, int64_t M, int64_t N, int64_t K, const void* A,
                        const void* B, int b_layout) {
    if (dtype != ORC_F16 && dtype != ORC_BF16)
        return ORC_EINVAL;
    if (b_layout != ORC_B_NK && b_layout != ORC_B_KN)
        return ORC_EINVAL;
    if (M < 0 || N < 0 || K < 0)
        return ORC_EINVAL;
    if (K > 0 && ((M > 0 && !A) || (N > 0 && !B)))
        return ORC_EINVAL;
    return ORC_OK;
}

/*
 * Rows [m_lo, m_hi) of C for 16-bit inputs.
 *   C_out : rounded results, [m_hi-m_lo, N] (may be NULL)
 *   S_out : the fp64 sums before rounding, [m_hi-m_lo, N] (may be NULL)
 */
int oracle_gemm_rows(int dtype, int64_t M, int64_t N, int64_t K, const uint16_t* A,
                     const uint16_t* B, int b_layout, int64_t m_lo, int64_t m_hi,
                     uint16_t* C_out, double* S_out, int nthreads) {
    int rc = check_common(dtype, M, N, K, A, B, b_layout);
    if (rc)
        return rc;
    if (m_lo < 0 || m_hi > M || m_lo > m_hi)
        return ORC_EINVAL;
    const int64_t rows = m_hi - m_lo;
    if (rows == 0 || N == 0)
        return ORC_OK;
    set_threads(nthreads);
    double* Ad = (double*)malloc(sizeof(double) * (size_t)(rows * K + 1));
    double* Bd = (double*)malloc(sizeof(double) * (size_t)(N * K + 1));
    double* S = S_out ? S_out : (double*)malloc(sizeof(double) * (size_t)(rows * N));
    if (!Ad || !Bd || !S) {
        free(Ad);
        free(Bd);
        if (!S_out)
            free(S);
        return ORC_ENOMEM;
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows * K; ++i)
        Ad[i] = decode(dtype, A[m_lo * K + i]);
    gather_b(dtype, N, K, B, b_layout, Bd);
    /* The decoded rows start at m_lo, so index them from 0. */
    sum_rows(0, rows, N, K, Ad, Bd, S);
    if (C_out) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < rows * N; ++i)
            C_out[i] = encode(dtype, S[i]);
    }
    free(Ad);
    free(Bd);
    if (!S_out)
        free(S);
    return ORC_OK;
}

/* The whole product: C_out is [M,N]. */
int oracle_gemm(int dtype, int64_t M, int64_t N, int64_t K, const uint16_t* A,
                const uint16_t* B, int b_layout, uint16_t* C_out, double* S_out,
                int nthreads) {
    return oracle_gemm_rows(dtype, M, N, K, A, B, b_layout, 0, M, C_out, S_out, nthreads);
}

/*
 * Selected entries (rows[i], cols[i]) of C, each computed on its own from the raw 16-bit
 * inputs, without decoding whole matrices: this is what lets a full-size product be
 * checked at sampled positions.
 */
int oracle_gemm_entries(int dtype, int64_t M, int64_t N, int64_t K, const uint16_t* A,
                        const uint16_t* B, int b_layout, int64_t count, const int64_t* rows,
                        const int64_t* cols, uint16_t* C_out, double* S_out, int nthreads) {
    int rc = check_common(dtype, M, N, K, A, B, b_layout);
    if (rc)
        return rc;
    for (int64_t i = 0; i < count; ++i)
        if (rows[i] < 0 || rows[i] >= M || cols[i] < 0 || cols[i] >= N)
            return ORC_EINVAL;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i) {
        const int64_t m = rows[i], n = cols[i];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const uint16_t bv = b_layout == ORC_B_NK ? B[n * K + k] : B[k * N + n];
            s += decode(dtype, A[m * K + k]) * decode(dtype, bv);
        }
        if (S_out)
            S_out[i] = s;
        if (C_out)
            C_out[i] = encode(dtype, s);
    }
    return ORC_OK;
}

/*
 * The same sum on fp64 operands, without any rounding to 16 bits: used to repeat the
 * small tiled-versus-naive experiment of "Tiling a matmul" (section "Code"), whose inputs
 * are doubles.  S is [M,N].
 */
int oracle_gemm_f64(int64_t M, int64_t N, int64_t K, const double* A, const double* B,
                    int b_layout, double* S, int nthreads) {
    if (b_layout != ORC_B_NK && b_layout != ORC_B_KN)
        return ORC_EINVAL;
    if (M < 0 || N < 0 || K < 0)
        return ORC_EINVAL;
    if (M == 0 || N == 0)
        return ORC_OK;
    set_threads(nthreads);
    double* Bnk = (double*)malloc(sizeof(double) * (size_t)(N * K + 1));
    if (!Bnk)
        return ORC_ENOMEM;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            Bnk[n * K + k] = b_layout == ORC_B_NK ? B[n * K + k] : B[k * N + n];
    sum_rows(0, M, N, K, A, Bnk, S);
    free(Bnk);
    return ORC_OK;
}

/*
 * The square tiled product of "Tiling a matmul" (sections "The idea in one minute" and
 * "Code"), on n x n fp64 matrices with B stored [K,N], written as a staged computation:
 * for each t x t block of C, the K range is walked t at a time; each step copies a t x t
 * block of A and one of B into small staging buffers (the "loads": 2 t^2 elements per
 * step, counted in *loads, so n^2/t^2 blocks x n/t steps give 2 n^3 / t in all) and adds,
 * for every element of the block, the partial dot product of that step to the element's
 * running sum.  n must be a multiple of t.  With t = 1 the running sums receive one
 * product at a time in increasing k: the naive order.
 */
int oracle_tiled_f64(int64_t n, int64_t t, const double* A, const double* B, double* C,
                     int64_t* loads) {
    if (n < 0 || t <= 0 || n % t != 0)
        return ORC_EINVAL;
    double* sa = (double*)malloc(sizeof(double) * (size_t)(t * t));   /* A block [t][t] */
    double* sb = (double*)malloc(sizeof(double) * (size_t)(t * t));   /* B block [t][t] */
    double* run = (double*)malloc(sizeof(double) * (size_t)(t * t));  /* running sums   */
    if (!sa || !sb || !run) {
        free(sa);
        free(sb);
        free(run);
        return ORC_ENOMEM;
    }
    int64_t staged = 0;
    const int64_t nb = n / t;
    for (int64_t blk = 0; blk < nb * nb; ++blk) {
        const int64_t row0 = (blk / nb) * t, col0 = (blk % nb) * t;
        for (int64_t e = 0; e < t * t; ++e)
            run[e] = 0.0;
        for (int64_t k0 = 0; k0 < n; k0 += t) {
            for (int64_t r = 0; r < t; ++r) {
                memcpy(sa + r * t, A + (row0 + r) * n + k0, sizeof(double) * (size_t)t);
                memcpy(sb + r * t, B + (k0 + r) * n + col0, sizeof(double) * (size_t)t);
            }
            staged += 2 * t * t;
            for (int64_t e = 0; e < t * t; ++e) {
                const int64_t r = e / t, c = e % t;
                double dot = 0.0;
                for (int64_t q = 0; q < t; ++q)
                    dot += sa[r * t + q] * sb[q * t + c];
                run[e] += dot;
            }
        }
        for (int64_t e = 0; e < t * t; ++e)
            C[(row0 + e / t) * n + col0 + e % t] = run[e];
    }
    free(sa);
    free(sb);
    free(run);
    if (loads)
        *loads = staged;
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------ */
/* Attention forward, the plain definition (no tiling and no online rescaling):          */
/*                                                                                        */
/*   s_j    = ( sum_{d<D} q(i,d) * k(j,d) ) / sqrt(D)      keys j < S (and j <= i if causal) */
/*   O(i,d) = round_f16( sum_j e^{s_j - m} v(j,d) / sum_j e^{s_j - m} ),   m = max_j s_j  */
/*                                                                                        */
/* per batch b and head h, with Q, K, V, O stored [B, S, H, D] (D contiguous), fp16.     */
/* Source: "TileLang: a tile language one level below Triton", section "FlashAttention:  */
/* online softmax as tile code": the forward pass over (batch, seq, heads, dim) tensors  */
/* in float16, scores Q K^T scaled by 1/sqrt(dim), the causal mask (a query sees the keys */
/* at or before its own position), the softmax over the keys and the product with V.     */
/* The page's kernel reaches the same result up to rounding by an online softmax with    */
/* base-2 exponentials (log2(e) folded into the scale); the oracle uses e^x and one pass */
/* over all scores.  Every sum runs in increasing index order in fp64; the result is     */
/* rounded once to fp16 (nearest-even).  O64 (optional) receives the unrounded values.   */
/* A query with no key (S == 0) does not exist; D == 0 gives +0.0.                       */
/* ------------------------------------------------------------------------------------ */
int oracle_attention(int64_t B, int64_t S, int64_t H, int64_t D, const uint16_t* Q,
                     const uint16_t* K, const uint16_t* V, int causal, uint16_t* O,
                     double* O64, int nthreads) {
    if (B < 0 || S < 0 || H < 0 || D < 0 || (causal != 0 && causal != 1))
        return ORC_EINVAL;
    const int64_t n = B * S * H * D;
    if (n == 0)
        return ORC_OK;
    set_threads(nthreads);
    double* q = (double*)malloc(sizeof(double) * (size_t)n);
    double* k = (double*)malloc(sizeof(double) * (size_t)n);
    double* v = (double*)malloc(sizeof(double) * (size_t)n);
    if (!q || !k || !v) {
        free(q);
        free(k);
        free(v);
        return ORC_ENOMEM;
    }
    for (int64_t i = 0; i < n; ++i) {
        q[i] = decode_f16(Q[i]);
        k[i] = decode_f16(K[i]);
        v[i] = decode_f16(V[i]);
    }
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    int rc = ORC_OK;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)S);
        if (!s) {
#pragma omp atomic write
            rc = ORC_ENOMEM;
        }
#pragma omp for collapse(3) schedule(static)
        for (int64_t b = 0; b < B; ++b) {
            for (int64_t h = 0; h < H; ++h) {
                for (int64_t i = 0; i < S; ++i) {
                    if (!s)
                        continue;
                    const double* qi = q + ((b * S + i) * H + h) * D;
                    const int64_t nkeys = causal ? i + 1 : S;
                    double m = -INFINITY;
                    for (int64_t j = 0; j < nkeys; ++j) {
                        const double* kj = k + ((b * S + j) * H + h) * D;
                        double dot = 0.0;
                        for (int64_t d = 0; d < D; ++d)
                            dot += qi[d] * kj[d];
                        s[j] = dot * inv_sqrt_d;
                        if (s[j] > m)
                            m = s[j];
                    }
                    double denom = 0.0;
                    for (int64_t j = 0; j < nkeys; ++j) {
                        s[j] = exp(s[j] - m);
                        denom += s[j];
                    }
                    for (int64_t d = 0; d < D; ++d) {
                        double num = 0.0;
                        for (int64_t j = 0; j < nkeys; ++j)
                            num += s[j] * v[((b * S + j) * H + h) * D + d];
                        const double o = num / denom;
                        const int64_t at = ((b * S + i) * H + h) * D + d;
                        O[at] = encode_f16(o);
                        if (O64)
                            O64[at] = o;
                    }
                }
            }
        }
        free(s);
    }
    free(q);
    free(k);
    free(v);
    return rc;
}
