/*
 * oracle.c -- plain, slow, host-only reference for the low-M split-K bf16 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no source, header, table or
 * helper with the HIP library.
 *
 * What it computes (the plain definition the method reaches up to rounding
 * order): C[m][n] = sum_{k=0}^{K-1} a(m,k) * w(n,k), with A[M,K] and W[N,K]
 * both row-major bf16, i.e. C = A * W^T.  Source: TensorRT-LLM PR "Fix two
 * synchronization gaps in the MiniMax M3 low-M split-K GEMM", Description,
 * item 2 (each split-K rank holds an fp32 partial over its part of K and rank
 * 0 sums them) and Hardware verification (bf16 inputs, output checked against
 * the fp32 product of the same operands).  The split over K is not modelled:
 * sum_r sum_{k in slice r} equals sum_k exactly in real arithmetic, and this
 * oracle sums in fp64, where every bf16*bf16 product is exact (8+8 significant
 * bits < 53) and the only rounding is fp64 addition in ascending k.
 *
 * bf16 is decoded from its IEEE-754 binary32 meaning (bf16 is the upper half of
 * a binary32 word: 1 sign bit, 8 exponent bits with bias 127, 7 fraction bits).
 * Rounding back to bf16 is round-to-nearest, ties-to-even, straight from fp64,
 * so there is no double rounding through fp32.
 *
 * Compile with -O2 -ffp-contract=off and without fast-math, so every fp64
 * operation is one IEEE operation in program order.
 */
#include <stdint.h>
#include <stdlib.h>
#include <math.h>

/* bf16 bit pattern -> exact value.  IEEE-754 binary32 field layout,
 * restricted to the upper 16 bits. */
double oracle_bf16_to_f64(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 7) & 0xFF;
    int frac = bits & 0x7F;
    double mag;
    if (expo == 0xFF) {
        mag = frac ? NAN : INFINITY;
    } else if (expo == 0) {
        /* subnormal: 0.frac * 2^(1-127) */
        mag = ldexp((double)frac, -126 - 7);
    } else {
        /* normal: 1.frac * 2^(expo-127) */
        mag = ldexp((double)(128 + frac), expo - 127 - 7);
    }
    return sign ? -mag : mag;
}

/* Round-to-nearest-even to an integer, done by hand on a non-negative double
 * that is below 2^52 (so it has a fractional part to inspect). */
static double rne_int(double v)
{
    double fl = floor(v);
    double rem = v - fl; /* exact: v and fl share the exponent range */
    if (rem > 0.5) return fl + 1.0;
    if (rem < 0.5) return fl;
    /* exact tie: pick the even neighbour */
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* fp64 value -> nearest bf16 bit pattern, ties to even.  NaN becomes the
 * quiet NaN 0x7FC0 (sign kept); overflow past the largest finite bf16 goes to
 * infinity as IEEE round-to-nearest prescribes. */
uint16_t oracle_round_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double ax = fabs(x);
    if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);
    if (isinf(x)) return (uint16_t)(sign | 0x7F80u);
    if (ax == 0.0) return sign;

    const double min_normal = ldexp(1.0, -126);
    if (ax < min_normal) {
        /* subnormal range: the quantum is 2^-133; a count of 128 quanta is
         * exactly the smallest normal, whose encoding is also 128. */
        double q = rne_int(ldexp(ax, 133));
        return (uint16_t)(sign | (uint16_t)q);
    }
    int e;                       /* ax = f * 2^e, 0.5 <= f < 1 */
    double f = frexp(ax, &e);
    double q = rne_int(ldexp(f, 8)); /* 8 significant bits: q in [128, 256] */
    if (q == 256.0) { q = 128.0; e += 1; }
    int biased = (e - 1) + 127;  /* ax ~= (q/128) * 2^(e-1) */
    if (biased >= 255) return (uint16_t)(sign | 0x7F80u);
    return (uint16_t)(sign | (uint16_t)(biased << 7) | (uint16_t)((int)q - 128));
}

/* Element-wise helpers over arrays, so the Python side makes one call. */
void oracle_bf16_to_f64_array(const uint16_t* bits, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f64(bits[i]);
}

void oracle_round_bf16_array(const double* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_round_bf16(x[i]);
}

/* Columns n in [n_begin, n_end) of C = A * W^T and of S = |A| * |W|^T, fp64,
 * ascending k.  A: [M][K] bf16 bits, W: [N][K] bf16 bits, both row-major.
 * C and S are [M][n_end - n_begin] row-major; S may be NULL.  The column range
 * lets a caller evaluate sampled outputs of a very large problem. */
void oracle_gemm_f64_cols(const uint16_t* A, const uint16_t* W,
                          int64_t M, int64_t N, int64_t K,
                          int64_t n_begin, int64_t n_end,
                          double* C, double* S)
{
    int64_t width = n_end - n_begin;
    if (n_begin < 0 || n_end > N || width < 0 || M < 0 || K < 0) return;
    /* Decode the operands to exact fp64 values first (element by element). */
    double* a = (double*)malloc(sizeof(double) * (size_t)(M * K + 1));
    double* w = (double*)malloc(sizeof(double) * (size_t)(K + 1));
    if (!a || !w) { free(a); free(w); return; }
    for (int64_t i = 0; i < M * K; ++i) a[i] = oracle_bf16_to_f64(A[i]);
    for (int64_t n = n_begin; n < n_end; ++n) {
        for (int64_t k = 0; k < K; ++k) w[k] = oracle_bf16_to_f64(W[n * K + k]);
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            double mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                acc += a[m * K + k] * w[k];
                mag += fabs(a[m * K + k]) * fabs(w[k]);
            }
            C[m * width + (n - n_begin)] = acc;
            if (S) S[m * width + (n - n_begin)] = mag;
        }
    }
    free(a);
    free(w);
}
