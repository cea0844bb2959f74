/*
 * oracle355.c -- plain CPU reference for the dense NT GEMM and its
 * block-scaled FP4 variant.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The GPU library
 * (libgemm355) never includes, links or calls it, and the two share no source
 * file, header, table or helper.
 *
 * What it computes -- the plain definition, with no blocking, fusion or
 * reordering of the arithmetic:
 *
 *     C[m][n] = bf16_round_nearest_even( sum_{k = 0 .. K-1} a(m,k) * b(n,k) )
 *
 * with the sum formed in IEEE binary64, k ascending, starting from +0.0.
 *
 *  - A is M x K, B is N x K, both row-major; C is M x N row-major; inputs and
 *    output are BF16 and the method accumulates in FP32
 *    ("Achieve cuBLAS Performance on NVIDIA GB300 for HGEMM", opening
 *    paragraph). The oracle accumulates in binary64 instead, which is the
 *    exact sum up to the rounding of the additions.
 *  - The output conversion rounds to nearest with ties to even
 *    ("Optimized B200 Matrix Multiplication", section 5 "The Epilogue: Escaping
 *    TMEM", whose conversion is the round-to-nearest one). The binary64 sum is
 *    rounded to BF16 directly, never through binary32.
 *  - Block-scaled FP4 ("NVFP4 GEMM on Blackwell", section "NVFP4 Datatype"):
 *    each element is an E2M1 code (1 sign, 2 exponent, 1 mantissa bit; values
 *    +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}) and every 16 consecutive elements of a row
 *    share one FP8 scale; a(m,k) = e2m1(code(m,k)) * scale(m, k/16).
 *    Readings where the page is silent: the scale is E4M3 with the "FN"
 *    encoding (bias 7, no infinities, S.1111.111 is NaN); codes are packed two
 *    per byte with the even k in the low nibble; scales are stored row-major,
 *    K/16 bytes per row; there is no per-tensor global scale.
 *
 * Every product here is exact in binary64 (a BF16 value has 8 significant
 * bits, a decoded FP4 element at most 6), so only the additions and the final
 * conversion round. Rows are shared out over OpenMP threads; each output
 * element is still summed by one thread in ascending k, so the result does
 * not depend on the thread count.
 */
#define _GNU_SOURCE /* M_PI */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARGS 1

/* ---- scalar codecs ----------------------------------------------------- */

/* A BF16 value is the upper 16 bits of an IEEE binary32 value. */
double oracle_bf16_to_double(uint16_t bits)
{
    uint32_t word = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &word, sizeof f);
    return (double)f;
}

/* Round a binary64 value to the nearest BF16 value, ties to even, in one step.
 * BF16 keeps 8 significant bits (1 implicit + 7 stored), exponent range as
 * binary32: normal numbers step by 2^(e-8) where x = f * 2^e, f in [0.5, 1);
 * below 2^-126 the step is the subnormal quantum 2^-133. */
uint16_t oracle_bf16_from_double(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    double mag = fabs(x);
    if (isinf(mag))
        return (uint16_t)(sign | 0x7F80u);
    if (mag == 0.0)
        return sign;

    int e;
    (void)frexp(mag, &e);
    int qexp = e - 8;
    if (qexp < -133)
        qexp = -133;
    double scaled = ldexp(mag, -qexp); /* power-of-two scaling: exact; < 256 */
    double lower = floor(scaled);
    double frac = scaled - lower;      /* exact: scaled has few integer bits */
    double q = lower;
    if (frac > 0.5)
        q = lower + 1.0;
    else if (frac == 0.5 && fmod(lower, 2.0) != 0.0)
        q = lower + 1.0;
    double rounded = ldexp(q, qexp);
    if (rounded >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80u); /* beyond the largest finite BF16 */

    /* rounded is a BF16 value, hence an exact binary32 value */
    float f = (float)rounded;
    uint32_t word;
    memcpy(&word, &f, sizeof word);
    return (uint16_t)(sign | (uint16_t)((word >> 16) & 0x7FFFu));
}

/* E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
 * Exponent 0 encodes 0 and 0.5 (m * 0.5); otherwise 2^(e-1) * (1 + m/2). */
double oracle_e2m1_to_double(unsigned code)
{
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* E4M3 ("FN"): sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.
 * Exponent 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; no infinities. */
double oracle_e4m3_to_double(unsigned byte)
{
    unsigned s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
    if (e == 15 && m == 7)
        return NAN;
    double mag = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

/* E8M0 (the shared scale of the microscaling formats, a reading outside the
 * pages -- see the MX product below): the byte is a biased exponent alone,
 * value 2^(byte - 127); 0xFF is NaN. */
double oracle_e8m0_to_double(unsigned byte)
{
    byte &= 255u;
    if (byte == 255u)
        return NAN;
    return ldexp(1.0, (int)byte - 127);
}

/* Array forms of the two BF16 codecs (same scalar routines, element by element). */
void oracle_bf16_to_double_n(const uint16_t *bits, double *out, long n)
{
    for (long i = 0; i < n; ++i)
        out[i] = oracle_bf16_to_double(bits[i]);
}

void oracle_bf16_from_double_n(const double *x, uint16_t *out, long n)
{
    for (long i = 0; i < n; ++i)
        out[i] = oracle_bf16_from_double(x[i]);
}

/* ---- element access ---------------------------------------------------- */

static double bf16_elem(const uint16_t *X, long K, long row, long k)
{
    return oracle_bf16_to_double(X[row * K + k]);
}

/* a(row, k) of a block-scaled FP4 operand: codes row-major, K/2 bytes per
 * row, even k in the low nibble; scales row-major, K/16 bytes per row. */
static double fp4_elem(const uint8_t *Q, const uint8_t *SF, long K, long row, long k)
{
    uint8_t byte = Q[row * (K / 2) + k / 2];
    unsigned code = (k & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 15u);
    return oracle_e2m1_to_double(code) * oracle_e4m3_to_double(SF[row * (K / 16) + k / 16]);
}

/* Microscaled FP4 element: the same E2M1 codes and nibble order, one E8M0
 * scale per 32 consecutive elements of a row (K/32 bytes per row). */
static double mx_elem(const uint8_t *Q, const uint8_t *S, long K, long row, long k)
{
    uint8_t byte = Q[row * (K / 2) + k / 2];
    unsigned code = (k & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 15u);
    return oracle_e2m1_to_double(code) * oracle_e8m0_to_double(S[row * (K / 32) + k / 32]);
}

static double dot_bf16(const uint16_t *A, const uint16_t *B, long K, long m, long n)
{
    double s = 0.0;
    for (long k = 0; k < K; ++k)
        s += bf16_elem(A, K, m, k) * bf16_elem(B, K, n, k);
    return s;
}

static double dot_fp4(const uint8_t *Aq, const uint8_t *SFA, const uint8_t *Bq,
                      const uint8_t *SFB, long K, long m, long n)
{
    double s = 0.0;
    for (long k = 0; k < K; ++k)
        s += fp4_elem(Aq, SFA, K, m, k) * fp4_elem(Bq, SFB, K, n, k);
    return s;
}

static double dot_mx(const uint8_t *Aq, const uint8_t *SA, const uint8_t *Bq, const uint8_t *SB, long K,
                     long m, long n)
{
    double s = 0.0;
    for (long k = 0; k < K; ++k)
        s += mx_elem(Aq, SA, K, m, k) * mx_elem(Bq, SB, K, n, k);
    return s;
}

/* ---- whole products ---------------------------------------------------- */

int oracle_gemm_bf16_nt(int M, int N, int K, const uint16_t *A, const uint16_t *B, uint16_t *C)
{
    if (M < 0 || N < 0 || K < 0)
        return ORACLE_BAD_ARGS;
#pragma omp parallel for schedule(dynamic, 1)
    for (long m = 0; m < M; ++m)
        for (long n = 0; n < N; ++n)
            C[m * (long)N + n] = oracle_bf16_from_double(dot_bf16(A, B, K, m, n));
    return ORACLE_OK;
}

int oracle_gemm_nvfp4_nt(int M, int N, int K, const uint8_t *Aq, const uint8_t *SFA,
                         const uint8_t *Bq, const uint8_t *SFB, uint16_t *C)
{
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0)
        return ORACLE_BAD_ARGS;
#pragma omp parallel for schedule(dynamic, 1)
    for (long m = 0; m < M; ++m)
        for (long n = 0; n < N; ++n)
            C[m * (long)N + n] = oracle_bf16_from_double(dot_fp4(Aq, SFA, Bq, SFB, K, m, n));
    return ORACLE_OK;
}

/* ---- chosen elements only (for products too large to form whole) --------
 * out_bf16[i] = C[ms[i]][ns[i]]; out_sum (may be NULL) gets the binary64 sum
 * before the final rounding. */

int oracle_gemm_bf16_nt_at(int M, int N, int K, const uint16_t *A, const uint16_t *B,
                           long count, const int32_t *ms, const int32_t *ns,
                           uint16_t *out_bf16, double *out_sum)
{
    if (M < 0 || N < 0 || K < 0 || count < 0)
        return ORACLE_BAD_ARGS;
    for (long i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N)
            return ORACLE_BAD_ARGS;
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < count; ++i) {
        double s = dot_bf16(A, B, K, ms[i], ns[i]);
        out_bf16[i] = oracle_bf16_from_double(s);
        if (out_sum)
            out_sum[i] = s;
    }
    return ORACLE_OK;
}

int oracle_gemm_nvfp4_nt_at(int M, int N, int K, const uint8_t *Aq, const uint8_t *SFA,
                            const uint8_t *Bq, const uint8_t *SFB, long count,
                            const int32_t *ms, const int32_t *ns, uint16_t *out_bf16,
                            double *out_sum)
{
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0 || count < 0)
        return ORACLE_BAD_ARGS;
    for (long i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N)
            return ORACLE_BAD_ARGS;
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < count; ++i) {
        double s = dot_fp4(Aq, SFA, Bq, SFB, K, ms[i], ns[i]);
        out_bf16[i] = oracle_bf16_from_double(s);
        if (out_sum)
            out_sum[i] = s;
    }
    return ORACLE_OK;
}

/* ---- fused epilogue -----------------------------------------------------
 * A bias and an activation applied to each sum before the output rounding
 * ("NVFP4 GEMM on Blackwell", "Kernel 1", "Epilogue Warps", which places
 * such per-element work in the epilogue).
 * The pages name no particular operation; the one computed here is the common
 * linear-layer epilogue, all in binary64:
 *
 *     z = sum_k a(m,k) b(n,k) + bias[n]        (bias NULL: no term)
 *     C[m][n] = bf16_round_nearest_even( act(z) )
 *
 * act 0: z; act 1 (ReLU): max(z, 0); act 2 (GELU, tanh form, the published
 * approximation of Hendrycks and Gimpel): z/2 (1 + tanh(sqrt(2/pi) (z +
 * 0.044715 z^3))). */

double oracle_activate(double z, int act)
{
    if (act == 1)
        return z > 0.0 ? z : 0.0;
    if (act == 2)
        return 0.5 * z * (1.0 + tanh(sqrt(2.0 / M_PI) * (z + 0.044715 * z * z * z)));
    return z;
}

static double bias_at(const uint16_t *bias, long n)
{
    return bias ? oracle_bf16_to_double(bias[n]) : 0.0;
}

int oracle_gemm_bf16_nt_bias_act(int M, int N, int K, const uint16_t *A, const uint16_t *B,
                                 const uint16_t *bias, int act, uint16_t *C)
{
    if (M < 0 || N < 0 || K < 0 || act < 0 || act > 2)
        return ORACLE_BAD_ARGS;
#pragma omp parallel for schedule(dynamic, 1)
    for (long m = 0; m < M; ++m)
        for (long n = 0; n < N; ++n)
            C[m * (long)N + n] =
                oracle_bf16_from_double(oracle_activate(dot_bf16(A, B, K, m, n) + bias_at(bias, n), act));
    return ORACLE_OK;
}

/* Chosen elements only; out_z (may be NULL) gets z before the activation. */
int oracle_gemm_bf16_nt_bias_act_at(int M, int N, int K, const uint16_t *A, const uint16_t *B,
                                    const uint16_t *bias, int act, long count, const int32_t *ms,
                                    const int32_t *ns, uint16_t *out_bf16, double *out_z)
{
    if (M < 0 || N < 0 || K < 0 || act < 0 || act > 2 || count < 0)
        return ORACLE_BAD_ARGS;
    for (long i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N)
            return ORACLE_BAD_ARGS;
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < count; ++i) {
        const double z = dot_bf16(A, B, K, ms[i], ns[i]) + bias_at(bias, ns[i]);
        out_bf16[i] = oracle_bf16_from_double(oracle_activate(z, act));
        if (out_z)
            out_z[i] = z;
    }
    return ORACLE_OK;
}

/* The block-scaled FP4 product with the same fused epilogue: z = sum of the
 * decoded products + bias[n], then the activation, in binary64. Chosen
 * elements only; out_z (may be NULL) gets z before the activation. */
int oracle_gemm_nvfp4_nt_bias_act_at(int M, int N, int K, const uint8_t *Aq, const uint8_t *SFA,
                                     const uint8_t *Bq, const uint8_t *SFB, const uint16_t *bias, int act,
                                     long count, const int32_t *ms, const int32_t *ns, uint16_t *out_bf16,
                                     double *out_z)
{
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0 || act < 0 || act > 2 || count < 0)
        return ORACLE_BAD_ARGS;
    for (long i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N)
            return ORACLE_BAD_ARGS;
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < count; ++i) {
        const double z = dot_fp4(Aq, SFA, Bq, SFB, K, ms[i], ns[i]) + bias_at(bias, ns[i]);
        out_bf16[i] = oracle_bf16_from_double(oracle_activate(z, act));
        if (out_z)
            out_z[i] = z;
    }
    return ORACLE_OK;
}

/* ---- microscaled FP4 (MXFP4) ---------------------------------------------
 * Not a format of the pages, which define the FP4 variant with an E4M3 scale
 * per 16 elements; this is the format the gfx950 matrix cores scale in
 * hardware (the microscaling convention: E2M1 elements, one power-of-two E8M0
 * scale per 32 elements). The product is the plain definition as for the
 * other formats:
 *     C[m][n] = bf16_round_nearest_even( sum_k a(m,k) b(n,k) ),
 *     a(m,k) = e2m1(code(m,k)) * 2^(SA[m][k/32] - 127),
 * K % 32 == 0, every product exact in binary64. */
int oracle_gemm_mxfp4_nt(int M, int N, int K, const uint8_t *Aq, const uint8_t *SA, const uint8_t *Bq,
                         const uint8_t *SB, uint16_t *C)
{
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0)
        return ORACLE_BAD_ARGS;
#pragma omp parallel for schedule(dynamic, 1)
    for (long m = 0; m < M; ++m)
        for (long n = 0; n < N; ++n)
            C[m * (long)N + n] = oracle_bf16_from_double(dot_mx(Aq, SA, Bq, SB, K, m, n));
    return ORACLE_OK;
}

int oracle_gemm_mxfp4_nt_at(int M, int N, int K, const uint8_t *Aq, const uint8_t *SA, const uint8_t *Bq,
                            const uint8_t *SB, long count, const int32_t *ms, const int32_t *ns,
                            uint16_t *out_bf16, double *out_sum)
{
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || count < 0)
        return ORACLE_BAD_ARGS;
    for (long i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N)
            return ORACLE_BAD_ARGS;
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < count; ++i) {
        double s = dot_mx(Aq, SA, Bq, SB, K, ms[i], ns[i]);
        out_bf16[i] = oracle_bf16_from_double(s);
        if (out_sum)
            out_sum[i] = s;
    }
    return ORACLE_OK;
}

/* The microscaled FP4 product with the fused epilogue (bias per column, then
 * the activation, in binary64), as for the other formats. Chosen elements
 * only; out_z (may be NULL) gets z before the activation. */
int oracle_gemm_mxfp4_nt_bias_act_at(int M, int N, int K, const uint8_t *Aq, const uint8_t *SA, const uint8_t *Bq,
                                     const uint8_t *SB, const uint16_t *bias, int act, long count,
                                     const int32_t *ms, const int32_t *ns, uint16_t *out_bf16, double *out_z)
{
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || act < 0 || act > 2 || count < 0)
        return ORACLE_BAD_ARGS;
    for (long i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N)
            return ORACLE_BAD_ARGS;
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < count; ++i) {
        const double z = dot_mx(Aq, SA, Bq, SB, K, ms[i], ns[i]) + bias_at(bias, ns[i]);
        out_bf16[i] = oracle_bf16_from_double(oracle_activate(z, act));
        if (out_z)
            out_z[i] = z;
    }
    return ORACLE_OK;
}

/* Decoded FP4 operand as binary64 (rows x K), for cross-checks. */
int oracle_decode_nvfp4(int rows, int K, const uint8_t *Q, const uint8_t *SF, double *out)
{
    if (rows < 0 || K < 0 || K % 16 != 0)
        return ORACLE_BAD_ARGS;
    for (long r = 0; r < rows; ++r)
        for (long k = 0; k < K; ++k)
            out[r * (long)K + k] = fp4_elem(Q, SF, K, r, k);
    return ORACLE_OK;
}

/* ---- threads ----------------------------------------------------------- */

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
