/*
 * sanitize_driver.c -- runs every entry point of oracle355.c on one case read
 * from a file and writes the results to another, so that the oracle can be
 * built as one executable with -fsanitize=address,undefined and exercised by
 * the CPU tests (an executable links the sanitizer runtime first, with no
 * preloading). TEST INFRASTRUCTURE ONLY, like the rest of oracle/.
 *
 * Case file: eight little-endian int32 (kind, M, N, K, act, count, 0, 0)
 * followed by the operands of the kind, each a dense row-major array:
 *   kind 1 (BF16):  A[M*K] u16, B[N*K] u16, bias[N] u16, ms[count] i32, ns[count] i32
 *   kind 2 (NVFP4): Aq[M*K/2], SFA[M*K/16], Bq[N*K/2], SFB[N*K/16] u8, bias, ms, ns
 *   kind 3 (MXFP4): Aq[M*K/2], SA[M*K/32], Bq[N*K/2], SB[N*K/32] u8, bias, ms, ns
 *   kind 4 (codecs): x[count] f64
 * Result file, in this order:
 *   kind 1: C[M*N] u16, at[count] u16, sum[count] f64, Cb[M*N] u16 (bias + act),
 *           atb[count] u16, z[count] f64
 *   kind 2: C, at, sum, atb, z (as kind 1 without Cb), dec(A)[M*K] f64
 *   kind 3: C, at, sum, atb, z
 *   kind 4: bf16->f64 of all 65536 patterns, e2m1 of 16 codes, e4m3 and e8m0 of
 *           256 bytes (f64), rne(x)[count] u16 singly and through the _n forms
 * Exit status 0 when every call returned 0; sanitizer reports abort the run.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gemm_bf16_nt(int M, int N, int K, const uint16_t *A, const uint16_t *B, uint16_t *C);
int oracle_gemm_nvfp4_nt(int M, int N, int K, const uint8_t *Aq, const uint8_t *SFA, const uint8_t *Bq,
                         const uint8_t *SFB, uint16_t *C);
int oracle_gemm_mxfp4_nt(int M, int N, int K, const uint8_t *Aq, const uint8_t *SA, const uint8_t *Bq,
                         const uint8_t *SB, uint16_t *C);
int oracle_gemm_bf16_nt_at(int M, int N, int K, const uint16_t *A, const uint16_t *B, long count,
                           const int32_t *ms, const int32_t *ns, uint16_t *out_bf16, double *out_sum);
int oracle_gemm_nvfp4_nt_at(int M, int N, int K, const uint8_t *Aq, const uint8_t *SFA, const uint8_t *Bq,
                            const uint8_t *SFB, long count, const int32_t *ms, const int32_t *ns,
                            uint16_t *out_bf16, double *out_sum);
int oracle_gemm_mxfp4_nt_at(int M, int N, int K, const uint8_t *Aq, const uint8_t *SA, const uint8_t *Bq,
                            const uint8_t *SB, long count, const int32_t *ms, const int32_t *ns,
                            uint16_t *out_bf16, double *out_sum);
int oracle_gemm_bf16_nt_bias_act(int M, int N, int K, const uint16_t *A, const uint16_t *B, const uint16_t *bias,
                                 int act, uint16_t *C);
int oracle_gemm_bf16_nt_bias_act_at(int M, int N, int K, const uint16_t *A, const uint16_t *B,
                                    const uint16_t *bias, int act, long count, const int32_t *ms,
                                    const int32_t *ns, uint16_t *out_bf16, double *out_z);
int oracle_gemm_nvfp4_nt_bias_act_at(int M, int N, int K, const uint8_t *Aq, const uint8_t *SFA,
                                     const uint8_t *Bq, const uint8_t *SFB, const uint16_t *bias, int act,
                                     long count, const int32_t *ms, const int32_t *ns, uint16_t *out_bf16,
                                     double *out_z);
int oracle_gemm_mxfp4_nt_bias_act_at(int M, int N, int K, const uint8_t *Aq, const uint8_t *SA, const uint8_t *Bq,
                                     const uint8_t *SB, const uint16_t *bias, int act, long count,
                                     const int32_t *ms, const int32_t *ns, uint16_t *out_bf16, double *out_z);
int oracle_decode_nvfp4(int rows, int K, const uint8_t *Q, const uint8_t *SF, double *out);
double oracle_bf16_to_double(uint16_t bits);
uint16_t oracle_bf16_from_double(double x);
double oracle_e2m1_to_double(unsigned code);
double oracle_e4m3_to_double(unsigned byte);
double oracle_e8m0_to_double(unsigned byte);
void oracle_bf16_to_double_n(const uint16_t *bits, double *out, long n);
void oracle_bf16_from_double_n(const double *x, uint16_t *out, long n);

static FILE *in_f, *out_f;

/* A heap array of exactly `bytes` bytes read from the case file (so that the
 * sanitizer sees every overrun), or NULL for an empty one. */
static void *take(size_t bytes)
{
    if (bytes == 0)
        return NULL;
    void *p = malloc(bytes);
    if (!p || fread(p, 1, bytes, in_f) != bytes) {
        fprintf(stderr, "short case file\n");
        exit(2);
    }
    return p;
}

static void *fresh(size_t bytes) { return bytes ? calloc(1, bytes) : NULL; }

static void put(const void *p, size_t bytes)
{
    if (bytes && fwrite(p, 1, bytes, out_f) != bytes) {
        fprintf(stderr, "short write\n");
        exit(2);
    }
}

int main(int argc, char **argv)
{
    if (argc != 3) {
        fprintf(stderr, "usage: %s case.bin result.bin\n", argv[0]);
        return 2;
    }
    in_f = fopen(argv[1], "rb");
    out_f = fopen(argv[2], "wb");
    if (!in_f || !out_f)
        return 2;
    int32_t h[8];
    if (fread(h, sizeof h, 1, in_f) != 1)
        return 2;
    const int kind = h[0], M = h[1], N = h[2], K = h[3], act = h[4];
    const long count = h[5];
    const size_t MN = (size_t)M * N;
    int bad = 0;

    if (kind == 4) {
        double *x = take(sizeof(double) * count);
        double d[65536];
        for (unsigned b = 0; b < 65536; ++b)
            d[b] = oracle_bf16_to_double((uint16_t)b);
        put(d, sizeof d);
        for (unsigned c = 0; c < 16; ++c)
            d[c] = oracle_e2m1_to_double(c);
        put(d, 16 * sizeof(double));
        for (unsigned b = 0; b < 256; ++b)
            d[b] = oracle_e4m3_to_double(b);
        put(d, 256 * sizeof(double));
        for (unsigned b = 0; b < 256; ++b)
            d[b] = oracle_e8m0_to_double(b);
        put(d, 256 * sizeof(double));
        uint16_t *r = fresh(2 * count), *rn = fresh(2 * count);
        for (long i = 0; i < count; ++i)
            r[i] = oracle_bf16_from_double(x[i]);
        oracle_bf16_from_double_n(x, rn, count);
        put(r, 2 * count);
        put(rn, 2 * count);
        double *back = fresh(sizeof(double) * count);
        oracle_bf16_to_double_n(rn, back, count);
        put(back, sizeof(double) * count);
        free(x);
        free(r);
        free(rn);
        free(back);
    } else if (kind >= 1 && kind <= 3) {
        const void *Aop, *Bop;
        const uint8_t *SA = NULL, *SB = NULL;
        const int sb = kind == 2 ? 16 : 32;
        if (kind == 1) {
            Aop = take((size_t)M * K * 2);
            Bop = take((size_t)N * K * 2);
        } else {
            Aop = take((size_t)M * K / 2);
            SA = take((size_t)M * K / sb);
            Bop = take((size_t)N * K / 2);
            SB = take((size_t)N * K / sb);
        }
        const uint16_t *bias = take((size_t)N * 2);
        const int32_t *ms = take(4 * count), *ns = take(4 * count);
        uint16_t *C = fresh(2 * MN), *at = fresh(2 * count), *atb = fresh(2 * count);
        double *sum = fresh(8 * count), *z = fresh(8 * count);
        if (kind == 1) {
            bad |= oracle_gemm_bf16_nt(M, N, K, Aop, Bop, C);
            bad |= oracle_gemm_bf16_nt_at(M, N, K, Aop, Bop, count, ms, ns, at, sum);
            bad |= oracle_gemm_bf16_nt_bias_act_at(M, N, K, Aop, Bop, bias, act, count, ms, ns, atb, z);
        } else if (kind == 2) {
            bad |= oracle_gemm_nvfp4_nt(M, N, K, Aop, SA, Bop, SB, C);
            bad |= oracle_gemm_nvfp4_nt_at(M, N, K, Aop, SA, Bop, SB, count, ms, ns, at, sum);
            bad |= oracle_gemm_nvfp4_nt_bias_act_at(M, N, K, Aop, SA, Bop, SB, bias, act, count, ms, ns, atb, z);
        } else {
            bad |= oracle_gemm_mxfp4_nt(M, N, K, Aop, SA, Bop, SB, C);
            bad |= oracle_gemm_mxfp4_nt_at(M, N, K, Aop, SA, Bop, SB, count, ms, ns, at, sum);
            bad |= oracle_gemm_mxfp4_nt_bias_act_at(M, N, K, Aop, SA, Bop, SB, bias, act, count, ms, ns, atb, z);
        }
        put(C, 2 * MN);
        put(at, 2 * count);
        put(sum, 8 * count);
        if (kind == 1) {
            uint16_t *Cb = fresh(2 * MN);
            bad |= oracle_gemm_bf16_nt_bias_act(M, N, K, Aop, Bop, bias, act, Cb);
            put(Cb, 2 * MN);
            free(Cb);
        }
        put(atb, 2 * count);
        put(z, 8 * count);
        if (kind == 2) {
            double *dec = fresh(8 * (size_t)M * K);
            bad |= oracle_decode_nvfp4(M, K, Aop, SA, dec);
            put(dec, 8 * (size_t)M * K);
            free(dec);
        }
        free((void *)Aop);
        free((void *)Bop);
        free((void *)SA);
        free((void *)SB);
        free((void *)bias);
        free((void *)ms);
        free((void *)ns);
        free(C);
        free(at);
        free(atb);
        free(sum);
        free(z);
    } else {
        return 2;
    }
    fclose(in_f);
    return fclose(out_f) != 0 || bad ? 1 : 0;
}
