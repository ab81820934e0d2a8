/*
 * Plain CPU oracle for the half-precision TN GEMM  D = alpha * A * B^T, and
 * for the attention forward O = softmax(alpha * Q K^T) V built on it.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header or table with the HIP
 * library.
 *
 * What it computes (sources):
 *   - "cute(9) multistage_gemm", section 11.1 (test configuration): A is
 *     M x K row-major, B is N x K row-major, D is M x N row-major and
 *     D = A @ B^T.
 *   - "CUDA operator notes 2", section "GEMM": all matrices are fp16 and the
 *     scale factor alpha is an fp32 value; D = alpha * (A B) before the cast
 *     to half.  (The beta * C term of that page is not part of this path.)
 *   - The accumulation precision follows the WMMA kernel of the same page
 *     (fp32 accumulators); the oracle goes further and accumulates in fp64 or
 *     exactly, then rounds once.
 *
 * Two independent evaluations of the same definition are provided:
 *   sgo_gemm_tn_f64    decode every fp16 to fp64 (exact), multiply (exact in
 *                      fp64: 11+11 significant bits), add in index order
 *                      k = 0..K-1 in fp64, scale by alpha in fp64, round once
 *                      to fp16 (round-to-nearest-even).
 *   sgo_gemm_tn_exact  every finite fp16 is an integer multiple of 2^-24 below
 *                      2^16 in magnitude, so every product is an integer
 *                      multiple of 2^-48 below 2^80; the sum is kept exactly
 *                      in a signed 128-bit integer and rounded once to fp16.
 *                      No floating point is used anywhere on this path.
 *
 * Readings where the pages are silent (listed in the design notes as well):
 *   - rounding to fp16 is IEEE-754 round-to-nearest-even, magnitudes at or
 *     above 65520 become infinity, subnormals are kept both ways;
 *   - an exactly zero sum is +0; a negative value that rounds to zero is -0;
 *   - K == 0 is the empty sum (+0).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* binary16 codec, written from the IEEE-754 definition: 1 sign bit, 5 exponent
 * bits with bias 15, 10 fraction bits; exponent field 0 = zero/subnormal with
 * value fraction * 2^-24, exponent field 31 = infinity / NaN.                 */

double sgo_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 31;
    int frac = h & 1023;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);
    return sign ? -v : v;
}

/* Pack a rounded magnitude n * 2^(e - 10), with e >= -14 and n < 2048 after
 * normalisation, into binary16 bits.  n < 1024 only occurs when e == -14
 * (subnormal or zero). */
static uint16_t pack_f16(int sign, uint64_t n, int e)
{
    if (n >= 2048) { n >>= 1; e += 1; }     /* rounding carried into a new binade */
    uint16_t s = (uint16_t)(sign ? 0x8000 : 0);
    if (n < 1024) return (uint16_t)(s | n); /* subnormal (e == -14) or zero */
    if (e + 15 >= 31) return (uint16_t)(s | 0x7c00);
    return (uint16_t)(s | ((uint16_t)(e + 15) << 10) | (uint16_t)(n - 1024));
}

/* Round a double to the nearest binary16, ties to even. */
uint16_t sgo_f64_to_f16(double x)
{
    if (isnan(x)) return (uint16_t)(signbit(x) ? 0xfe00 : 0x7e00);
    int sign = signbit(x) ? 1 : 0;
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign ? 0xfc00 : 0x7c00);
    if (a == 0.0) return (uint16_t)(sign ? 0x8000 : 0);
    int E;
    (void)frexp(a, &E);                      /* a = f * 2^E, f in [0.5, 1) */
    int e = E - 1;                           /* a in [2^e, 2^(e+1)) */
    if (e < -14) e = -14;                    /* subnormal quantum 2^-24 */
    if (e > 16) return (uint16_t)(sign ? 0xfc00 : 0x7c00);
    double n = ldexp(a, 10 - e);             /* exact: scaling by a power of two */
    double fl = floor(n);
    double rem = n - fl;                     /* exact */
    uint64_t q = (uint64_t)fl;
    if (rem > 0.5 || (rem == 0.5 && (q & 1))) q += 1;
    return pack_f16(sign, q, e);
}

void sgo_f16_to_f64_array(const uint16_t *h, double *out, long n)
{
    for (long i = 0; i < n; ++i) out[i] = sgo_f16_to_f64(h[i]);
}

void sgo_f64_to_f16_array(const double *x, uint16_t *out, long n)
{
    for (long i = 0; i < n; ++i) out[i] = sgo_f64_to_f16(x[i]);
}

/* ------------------------------------------------------------------------ */
/* fp64 evaluation: one output element is one fp64 sum in index order.       */

/* Decoded value of every bit pattern, filled once from sgo_f16_to_f64 so the
 * inner loop does not call ldexp.  Filled before any parallel region. */
static double g_dec[65536];
static int g_dec_ready = 0;

static void ensure_decode_table(void)
{
    if (g_dec_ready) return;
    for (int h = 0; h < 65536; ++h) g_dec[h] = sgo_f16_to_f64((uint16_t)h);
    g_dec_ready = 1;
}

static double dot_f64(const uint16_t *arow, const uint16_t *brow, int K)
{
    double sum = 0.0;
    for (int k = 0; k < K; ++k)
        sum += g_dec[arow[k]] * g_dec[brow[k]];   /* product exact in fp64 */
    return sum;
}

/* alpha * s in fp64 (exact: 24 x 53 bits fit unless s has more than 29
 * significant bits, and then one fp64 rounding far below fp16's), plus +0 so
 * that an exactly zero value is +0 for either sign of alpha: the value of an
 * exactly zero real sum has no sign, and round-to-nearest gives +0 for it. */
static double scaled_sum(double a64, double s)
{
    return a64 * s + 0.0;
}

/* D[i][j] = RNE16( alpha * sum_k A[i][k] * B[j][k] ), all row-major. */
void sgo_gemm_tn_f64(int M, int N, int K, float alpha,
                     const uint16_t *A, const uint16_t *B, uint16_t *D)
{
    ensure_decode_table();
    const double a64 = (double)alpha;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < M; ++i)
        for (int j = 0; j < N; ++j) {
            double s = dot_f64(A + (size_t)i * K, B + (size_t)j * K, K);
            D[(size_t)i * N + j] = sgo_f64_to_f16(scaled_sum(a64, s));
        }
}

/* D[i][j] = RNE16( alpha * sum_k A[i][k] * B[j][k] + beta * C[i][j] ): the
 * GEMM of "CUDA operator notes 2", section "GEMM" (C = alpha A B + beta C),
 * one rounding.  beta == 0 does not read C (C may be NULL). */
void sgo_gemm_tn_f64_beta(int M, int N, int K, float alpha, float beta,
                          const uint16_t *A, const uint16_t *B, const uint16_t *C,
                          uint16_t *D)
{
    ensure_decode_table();
    const double a64 = (double)alpha, b64 = (double)beta;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < M; ++i)
        for (int j = 0; j < N; ++j) {
            double s = a64 * dot_f64(A + (size_t)i * K, B + (size_t)j * K, K);
            if (beta != 0.0f) s += b64 * g_dec[C[(size_t)i * N + j]];   /* beta*c exact */
            D[(size_t)i * N + j] = sgo_f64_to_f16(s + 0.0);   /* exact zero -> +0 */
        }
}

/* The same definition evaluated only at the listed (row, col) pairs. */
void sgo_gemm_tn_f64_at(int K, float alpha, const uint16_t *A, const uint16_t *B,
                        long count, const int *rows, const int *cols, uint16_t *out)
{
    ensure_decode_table();
    const double a64 = (double)alpha;
    #pragma omp parallel for schedule(dynamic, 64)
    for (long t = 0; t < count; ++t) {
        double s = dot_f64(A + (size_t)rows[t] * K, B + (size_t)cols[t] * K, K);
        out[t] = sgo_f64_to_f16(scaled_sum(a64, s));
    }
}

/* Rows [r0, r1) of D only (used to time the oracle on a bounded sample). */
void sgo_gemm_tn_f64_rows(int N, int K, float alpha, const uint16_t *A,
                          const uint16_t *B, int r0, int r1, uint16_t *Drows)
{
    ensure_decode_table();
    const double a64 = (double)alpha;
    #pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int i = r0; i < r1; ++i)
        for (int j = 0; j < N; ++j) {
            double s = dot_f64(A + (size_t)i * K, B + (size_t)j * K, K);
            Drows[(size_t)(i - r0) * N + j] = sgo_f64_to_f16(scaled_sum(a64, s));
        }
}

/* Attention forward of "CUDA operator notes 2", section "Softmax Attention":
 * O = softmax(alpha * Q K^T) V with the softmax taken along each row, per head
 * h of H.  Q is H x M x d, K and V are H x N x d, O is H x M x d, all
 * row-major fp16.  For each output row: scores s_j = alpha * (q . k_j) in
 * fp64 (products exact, sum in index order, then the fp32 alpha widened
 * exactly), m = max_j s_j, w_j = exp(s_j - m), and
 * O[c] = (sum_j w_j v_jc) / (sum_j w_j), rounded once to fp16.  When wbound is
 * not NULL it receives, per output element, sum_j w_j |v_jc| / sum_j w_j: the
 * weight of |V| behind that output, which the GPU tolerance uses.  N >= 1. */
void sgo_attention_f64(int H, int M, int N, int d, float alpha, const uint16_t *Q,
                       const uint16_t *K, const uint16_t *V, uint16_t *O, double *wbound)
{
    ensure_decode_table();
    const double a64 = (double)alpha;
    #pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)N);
        double *num = (double *)malloc(sizeof(double) * (size_t)d);
        double *wabs = (double *)malloc(sizeof(double) * (size_t)d);
        #pragma omp for schedule(dynamic, 1) collapse(2)
        for (int h = 0; h < H; ++h)
            for (int i = 0; i < M; ++i) {
                const uint16_t *q = Q + ((size_t)h * M + i) * d;
                const uint16_t *kh = K + (size_t)h * N * d;
                const uint16_t *vh = V + (size_t)h * N * d;
                double m = -INFINITY;
                for (int j = 0; j < N; ++j) {
                    s[j] = a64 * dot_f64(q, kh + (size_t)j * d, d);
                    if (s[j] > m) m = s[j];
                }
                double den = 0.0;
                for (int c = 0; c < d; ++c) num[c] = wabs[c] = 0.0;
                for (int j = 0; j < N; ++j) {
                    const double w = exp(s[j] - m);
                    den += w;
                    for (int c = 0; c < d; ++c) {
                        const double v = g_dec[vh[(size_t)j * d + c]];
                        num[c] += w * v;
                        wabs[c] += w * fabs(v);
                    }
                }
                uint16_t *o = O + ((size_t)h * M + i) * d;
                for (int c = 0; c < d; ++c) {
                    o[c] = sgo_f64_to_f16(num[c] / den);
                    if (wbound) wbound[((size_t)h * M + i) * d + c] = wabs[c] / den;
                }
            }
        free(s);
        free(num);
        free(wabs);
    }
}

int sgo_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Exact evaluation: integers only.                                            */

typedef __int128 i128;
typedef unsigned __int128 u128;

/* A finite fp16 as a signed integer count of 2^-24.  Returns 0 and sets *bad
 * for infinity / NaN, which the exact path does not accept. */
static int64_t f16_to_units24(uint16_t h, int *bad)
{
    int expo = (h >> 10) & 31;
    int64_t frac = h & 1023;
    int64_t mag;
    if (expo == 31) { *bad = 1; return 0; }
    if (expo == 0) mag = frac;                          /* frac * 2^-24 */
    else mag = (1024 + frac) << (expo - 1);             /* (1024+frac) * 2^(expo-25) */
    return (h & 0x8000) ? -mag : mag;
}

static int bit_length_u128(u128 v)
{
    int n = 0;
    while (v) { v >>= 1; ++n; }
    return n;
}

/* Round sign * mag * 2^scale (mag an exact integer) to the nearest binary16,
 * ties to even.  An exactly zero input is +0. */
static uint16_t round_units_to_f16(int sign, u128 mag, int scale)
{
    if (mag == 0) return 0;
    int p = bit_length_u128(mag) - 1 + scale;           /* value in [2^p, 2^(p+1)) */
    int e = p < -14 ? -14 : p;
    if (e > 16) return (uint16_t)(sign ? 0xfc00 : 0x7c00);
    int qe = e - 10 - scale;                            /* quantum = 2^qe units */
    uint64_t n;
    if (qe <= 0) {
        n = (uint64_t)(mag << (-qe));                   /* exact, no rounding needed */
    } else {
        u128 q = mag >> qe;
        u128 rem = mag - (q << qe);
        u128 half = (u128)1 << (qe - 1);
        if (rem > half || (rem == half && (q & 1))) q += 1;
        n = (uint64_t)q;
    }
    return pack_f16(sign, n, e);
}

/* alpha as an exact dyadic rational: alpha = am * 2^ae with am a 24-bit
 * integer (or 0).  Returns -1 for non-finite alpha. */
static int split_f32(float alpha, int64_t *am, int *ae)
{
    if (!isfinite(alpha)) return -1;
    if (alpha == 0.0f) { *am = 0; *ae = 0; return 0; }
    int E;
    double f = frexp((double)alpha, &E);                /* exact for a float */
    *am = (int64_t)ldexp(f, 24);                        /* |am| < 2^24, exact */
    *ae = E - 24;
    return 0;
}

/* Exact D = RNE16(alpha * sum A[i][k] B[j][k]).  Returns 0 on success, -1 if
 * an input or alpha is not finite, -2 if K is too large for the 128-bit sum
 * once multiplied by alpha's 24-bit mantissa. */
int sgo_gemm_tn_exact(int M, int N, int K, float alpha,
                      const uint16_t *A, const uint16_t *B, uint16_t *D)
{
    int64_t am; int ae;
    if (split_f32(alpha, &am, &ae)) return -1;
    if (K >= (1 << 20)) return -2;      /* 2^80 * 2^20 * 2^24 < 2^126 */
    int bad = 0;
    for (size_t t = 0; t < (size_t)M * K; ++t) (void)f16_to_units24(A[t], &bad);
    for (size_t t = 0; t < (size_t)N * K; ++t) (void)f16_to_units24(B[t], &bad);
    if (bad) return -1;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < M; ++i) {
        int dummy = 0;
        for (int j = 0; j < N; ++j) {
            i128 sum = 0;
            for (int k = 0; k < K; ++k)
                sum += (i128)f16_to_units24(A[(size_t)i * K + k], &dummy) *
                       (i128)f16_to_units24(B[(size_t)j * K + k], &dummy);
            i128 scaled = sum * (i128)am;               /* units of 2^(-48 + ae) */
            int sign = scaled < 0;
            u128 mag = (u128)(sign ? -scaled : scaled);
            D[(size_t)i * N + j] = round_units_to_f16(sign, mag, ae - 48);
        }
    }
    return 0;
}

/* Exact D = RNE16(alpha * sum A[i][k] B[j][k] + beta * C[i][j]).  alpha*sum is
 * an integer times 2^(ae-48), beta*c an integer times 2^(be-24); both are
 * brought to the smaller exponent.  Returns -1 for non-finite input, -2 when
 * the alignment shift would not fit the 128-bit sum (refused, not rounded). */
int sgo_gemm_tn_exact_beta(int M, int N, int K, float alpha, float beta,
                           const uint16_t *A, const uint16_t *B, const uint16_t *C,
                           uint16_t *D)
{
    int64_t am, bm; int ae, be;
    if (split_f32(alpha, &am, &ae) || split_f32(beta, &bm, &be)) return -1;
    if (K >= (1 << 20)) return -2;
    int bad = 0;
    for (size_t t = 0; t < (size_t)M * K; ++t) (void)f16_to_units24(A[t], &bad);
    for (size_t t = 0; t < (size_t)N * K; ++t) (void)f16_to_units24(B[t], &bad);
    if (beta != 0.0f)
        for (size_t t = 0; t < (size_t)M * N; ++t) (void)f16_to_units24(C[t], &bad);
    if (bad) return -1;
    const int ea = ae - 48, eb = be - 24;
    const int e = ea < eb ? ea : eb;
    const int sa = ea - e, sb = eb - e;          /* left shifts onto the common exponent */
    /* |am*sum| < 2^24 * 2^80 * 2^20 = 2^124; |bm*c| < 2^24 * 2^40 = 2^64 */
    if ((am != 0 && sa > 2) || (bm != 0 && sb > 60)) return -2;
    int fail = 0;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < M; ++i) {
        int dummy = 0;
        for (int j = 0; j < N; ++j) {
            i128 sum = 0;
            for (int k = 0; k < K; ++k)
                sum += (i128)f16_to_units24(A[(size_t)i * K + k], &dummy) *
                       (i128)f16_to_units24(B[(size_t)j * K + k], &dummy);
            i128 total = (sum * (i128)am) * ((i128)1 << sa);
            if (beta != 0.0f)
                total += ((i128)bm * (i128)f16_to_units24(C[(size_t)i * N + j], &dummy)) *
                         ((i128)1 << sb);
            int sign = total < 0;
            u128 mag = (u128)(sign ? -total : total);
            D[(size_t)i * N + j] = round_units_to_f16(sign, mag, e);
        }
    }
    return fail;
}
