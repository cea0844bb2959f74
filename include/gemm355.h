/*
 * gemm355.h -- C ABI of libgemm355: dense NT matrix products on AMD Instinct
 * MI355X (gfx950).
 *
 *   C = A * B^T    A is M x K, B is N x K, both row-major; C is M x N row-major.
 *
 * The operation is the one defined in "Achieve cuBLAS Performance on NVIDIA
 * GB300 for HGEMM" (opening paragraph): BF16 inputs and output, FP32
 * accumulation. The block-scaled variant takes its operand format from
 * "NVFP4 GEMM on Blackwell", section "NVFP4 Datatype": E2M1 codes with one FP8
 * scale per 16 consecutive elements. A microscaled variant (one power-of-two
 * E8M0 scale per 32 elements) runs on the matrix cores' own block scaling.
 * Each product also comes with a fused epilogue (bias per output column, then
 * identity, ReLU or tanh GELU).
 *
 * Conventions shared by every entry point
 *  - All array pointers are DEVICE pointers owned by the caller. The library
 *    allocates no memory, keeps no per-call state and never synchronises: it
 *    enqueues the work on `stream` and returns. The only scratch memory, the
 *    FP32 partials of a split K or the decoded operands of the decode-first
 *    NVFP4 path, is a workspace the caller passes to the *_ws entry points,
 *    or, for gemm_bf16_nt_noalloc only, a fixed static device array.
 *    `stream` is a hipStream_t passed as void*; NULL means the default (null)
 *    stream.
 *  - Arrays are dense, row-major, with no padding between rows (the leading
 *    dimension of A and B is K, that of C is N). C must not overlap any input.
 *  - Only the M x N elements of C are written.
 *  - Results for inputs holding NaN or infinity are unspecified.
 *  - Every argument check happens before the first HIP runtime call, so a
 *    rejected call touches neither the device nor the stream. A launch that
 *    fails returns GEMM355_ERR_LAUNCH (the status of the launch call itself);
 *    the library never reads or clears the thread's pending HIP error, so an
 *    error from the caller's own earlier HIP calls stays for the caller to
 *    collect. Faults that happen during the asynchronous execution surface at
 *    the caller's next synchronisation, as usual for HIP.
 *  - Calls are thread-safe: the library holds no mutable state apart from a
 *    per-device cache of the compute-unit count, filled once under a lock,
 *    the overrides set by gemm355_force_instance, gemm355_force_supergroup,
 *    gemm355_force_schedule and gemm355_force_fp4_path (process-wide
 *    diagnostics), and two static device arrays that only opt-in paths use:
 *    the scratch of gemm_bf16_nt_noalloc and the tile counters of the
 *    dynamic tile order (gemm355_force_schedule(1)); calls that use either
 *    and overlap on one GPU race. Calls may be captured into HIP graphs.
 */
#ifndef GEMM355_H
#define GEMM355_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
typedef enum gemm355_status {
    GEMM355_OK = 0,               /* work enqueued (or nothing to do)              */
    GEMM355_ERR_INVALID_ARG = 1,  /* negative size, NULL pointer, overlapping C    */
    GEMM355_ERR_UNSUPPORTED = 2,  /* valid but outside what the kernels handle:   */
                                  /* alignment, K or N granularity, extents       */
    GEMM355_ERR_NO_DEVICE = 3,    /* no usable HIP device / attribute query failed */
    GEMM355_ERR_LAUNCH = 4        /* the kernel launch itself reported an error    */
} gemm355_status;

/*
 * gemm_bf16_nt -- C[m][n] = bf16( sum_k A[m][k] * B[n][k] )
 *
 * ("Achieve cuBLAS Performance on NVIDIA GB300 for HGEMM", opening paragraph.)
 *   M, N, K  sizes, >= 0.
 *   A        M x K BF16 values (2 bytes each), row-major.
 *   B        N x K BF16 values, row-major.
 *   C        M x N BF16 output, row-major.
 * Products are exact, sums are FP32 (order unspecified), and the FP32 result
 * is rounded to BF16 to nearest, ties to even ("Optimized B200 Matrix
 * Multiplication", section 5 "The Epilogue").
 * Edge cases: M == 0 or N == 0 does nothing and returns GEMM355_OK (A, B and C
 * may then be NULL); K == 0 writes +0 to all of C (A and B may be NULL).
 * Requirements, else GEMM355_ERR_UNSUPPORTED: A, B, C 16-byte aligned;
 * K % 8 == 0 and N % 8 == 0 (whole 16-byte row segments); every operand,
 * padded up to a multiple of 256 rows, spans less than 2^31 bytes.
 * Three kernel instances compute it: 256 x 256 output tiles; or, when the
 * 256 x 256 tiling has fewer tiles than half the compute units, either
 * 64 x 64 tiles or 128 x 128 tiles -- whichever has the shorter estimated
 * time (the busiest compute unit's K steps at a measured cost per step, or
 * the operand traffic at a loaded HBM rate, plus fixed costs); whenever
 * K <= 192, not 256 x 256 tiles. This entry point never splits K (that needs
 * a workspace: gemm_bf16_nt_ws). gemm355_bf16_plan reports the choice.
 * All instances give results within the same bound; they may sum in different
 * orders. Each instance is deterministic: the same call gives the same bits.
 */
int gemm_bf16_nt(int M, int N, int K, const void *A, const void *B, void *C, void *stream);

/* Activations of gemm_bf16_nt_bias_act's fused epilogue. */
typedef enum gemm355_activation {
    GEMM355_ACT_NONE = 0,         /* y = z                                          */
    GEMM355_ACT_RELU = 1,         /* y = max(z, 0)                                  */
    GEMM355_ACT_GELU_TANH = 2     /* y = z/2 (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))) */
} gemm355_activation;

/*
 * gemm_bf16_nt_bias_act -- C = act(A * B^T + bias), BF16 in and out, with the
 * bias and the activation applied in the epilogue while the FP32 sums are
 * still in registers, so C is written once and never re-read ("NVFP4 GEMM on
 * Blackwell", "Kernel 1", "Epilogue Warps").
 *
 *   C[m][n] = bf16_rne(act(z)),  z = fp32(sum_k A[m][k] * B[n][k]) + bias[n]
 *
 * with the sum as in gemm_bf16_nt, the bias added in FP32, and the activation
 * (a gemm355_activation) evaluated in FP32; the GELU's exponential is the
 * hardware's (relative error about 1e-6), far below the BF16 rounding.
 *   bias     N BF16 values (one per column of C, e.g. per output feature of a
 *            linear layer), 16-byte aligned; NULL means zeros.
 *   activation  GEMM355_ACT_NONE, _RELU or _GELU_TANH.
 * Everything else (layouts, ownership, edge cases, requirements, instances,
 * workspace, determinism) is as for gemm_bf16_nt; K == 0 gives act(bias[n]).
 * Errors: an unknown activation or a bias overlapping C -> INVALID_ARG; a bias
 * not 16-byte aligned -> UNSUPPORTED. The bias must not be written while the
 * product runs.
 */
int gemm_bf16_nt_bias_act(int M, int N, int K, const void *A, const void *B, const void *bias,
                          int activation, void *C, void *stream);

/*
 * gemm_bf16_nt_workspace_size -- workspace bytes gemm_bf16_nt_ws and
 * gemm_bf16_nt_bias_act_ws need for M x N x K on the current device.
 *
 * A library interface, not a definition of the pages. Writes 0 when the plan
 * does not split K (then the workspace may be NULL), else the bytes of the
 * FP32 partial tiles: 64 KiB per 128 x 128 output tile and split, at most
 * 64 KiB per compute unit (16 MiB on a 256-unit device). Returns
 * GEMM355_ERR_INVALID_ARG for negative sizes or a NULL `bytes`,
 * GEMM355_ERR_NO_DEVICE when the device cannot be queried; no other HIP call
 * is made. The size depends on the shape, the device's compute-unit count and
 * the gemm355_force_instance setting.
 */
int gemm_bf16_nt_workspace_size(int M, int N, int K, size_t *bytes);

/*
 * gemm_bf16_nt_ws -- gemm_bf16_nt with a caller-owned workspace, which lets
 * the 128 x 128 instance split K over several workgroups.
 *
 * ("Achieve cuBLAS Performance on NVIDIA GB300 for HGEMM", opening paragraph,
 * for the operation; "NVFP4 GEMM on Blackwell", "Production Kernel", "Swap
 * AB", for why skinny problems need more workgroups than output tiles.)
 * The result is as for gemm_bf16_nt. When the 128 x 128 instance is chosen,
 * its K range may be split over up to 8 workgroups (at least 8 steps of 64
 * each, enough splits to give every compute unit a work item) that write FP32
 * partial tiles to `workspace`; a second kernel on the same stream adds each
 * element's partials in split order and rounds once to BF16, so the result is
 * deterministic.
 *   workspace        device memory, 16-byte aligned, owned by the caller; its
 *                    contents on entry do not matter and on return are
 *                    unspecified. It must stay untouched until the product
 *                    has run on `stream`, and two products running at the
 *                    same time must not share one.
 *   workspace_bytes  its size; at least gemm_bf16_nt_workspace_size(M, N, K),
 *                    else GEMM355_ERR_UNSUPPORTED (nothing is enqueued).
 *                    NULL with 0 bytes is accepted when the plan needs none.
 * Errors otherwise as for gemm_bf16_nt; a workspace overlapping A, B or C ->
 * GEMM355_ERR_INVALID_ARG, one not 16-byte aligned -> UNSUPPORTED, NULL with
 * workspace_bytes > 0 -> INVALID_ARG.
 */
int gemm_bf16_nt_ws(int M, int N, int K, const void *A, const void *B, void *C, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * gemm_bf16_nt_bias_act_ws -- gemm_bf16_nt_bias_act with a caller-owned
 * workspace, as gemm_bf16_nt_ws adds one to gemm_bf16_nt. With several K
 * splits the reduction kernel adds the bias and applies the activation to the
 * summed FP32 partials before rounding. A workspace overlapping the bias is
 * also INVALID_ARG.
 */
int gemm_bf16_nt_bias_act_ws(int M, int N, int K, const void *A, const void *B, const void *bias, int activation,
                             void *C, void *workspace, size_t workspace_bytes, void *stream);

/*
 * gemm_bf16_nt_noalloc -- gemm_bf16_nt_ws for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.
 *
 * Computes what gemm_bf16_nt_ws computes, with the same plan and bitwise the
 * same result, but the split-K partials live in a fixed 16 MiB scratch array
 * inside the library (one per device, held until the process ends) instead of
 * a caller's workspace. No memory is allocated or freed, by the library or by
 * any routine it calls. The first call on a device that splits K looks the
 * array's device address up (hipGetSymbolAddress) with that device current.
 * Every call on one device shares that device's array: calls whose execution
 * overlaps on one GPU (other streams, other threads) race on it when both
 * split K and give undefined results; calls ordered on one stream are safe.
 * The array keeps the last call's partials; nothing needs to start at zero.
 * Errors: as for gemm_bf16_nt_ws; a plan whose partials exceed 16 MiB (only
 * possible on a device with more than 256 compute units) ->
 * GEMM355_ERR_UNSUPPORTED, nothing enqueued; the address lookup failing ->
 * GEMM355_ERR_NO_DEVICE.
 */
int gemm_bf16_nt_noalloc(int M, int N, int K, const void *A, const void *B, void *C, void *stream);

/*
 * gemm355_force_instance -- override the choice of gemm_bf16_nt's instance.
 *
 * A diagnostic for tests and measurements (it is not defined by the pages):
 * instance 0 restores the choice by shape, 1 forces 256 x 256 tiles (except
 * for K <= 192, which always takes the 64 x 64 instance), 2 forces 64 x 64
 * tiles, 3 forces 128 x 128 tiles (through the *_ws entry points with split K:
 * as many splits as give every compute unit a work item, at most 8, each at
 * least 8 steps of 64; one split when K is too short for two or the tiles
 * alone fill the units), for every later BF16 product in the process. Returns
 * GEMM355_OK, or GEMM355_ERR_INVALID_ARG for any other value (the setting is
 * then unchanged). Calls racing with gemm_bf16_nt on other threads see either
 * the old or the new setting. No HIP call is made.
 */
int gemm355_force_instance(int instance);

/*
 * gemm355_force_supergroup -- override the band width of the supergroup
 * visiting order ("NVFP4 GEMM on Blackwell", section "Supergroup Size": the
 * pages ablate this width per shape) used by the persistent kernels of
 * gemm_bf16_nt and gemm_nvfp4_nt.
 *
 * A diagnostic for measurements: 0 restores the default (gemm355_supergroup's
 * width for 256 x 256 tiles, 8 for the 64 x 64 instance), 1..4096 forces that
 * width for every later launch in the process.
 * The result of a product does not depend on it (every tile is computed the
 * same way, only the order changes). Returns GEMM355_OK, or
 * GEMM355_ERR_INVALID_ARG for any other value (the setting is then
 * unchanged). No HIP call is made.
 */
int gemm355_force_supergroup(int supergroup);

/* Kernels of gemm355_supergroup's rule. */
typedef enum gemm355_kernel {
    GEMM355_KERNEL_BF16 = 0,        /* gemm_bf16_nt, 256 x 256 tiles      */
    GEMM355_KERNEL_NVFP4 = 1,       /* gemm_nvfp4_nt                       */
    GEMM355_KERNEL_MXFP4 = 2,       /* gemm_mxfp4_nt                       */
    GEMM355_KERNEL_BF16_SMALL = 3   /* gemm_bf16_nt, 64 x 64 tiles        */
} gemm355_kernel;

/*
 * gemm355_supergroup -- the default band width of the supergroup visiting
 * order ("NVFP4 GEMM on Blackwell", "Production Kernel", "Supergroup Size")
 * for a kernel (a gemm355_kernel), the number of output tiles across N and K.
 * A measured rule: 16 for short K loops with many tiles across N, where wide
 * bands write C in longer runs (BF16 and microscaled FP4: K <= 1024 and at
 * least 64 tiles; NVFP4: K <= 2048 and at least 32 tiles), else 8 (the
 * fewest A and B strips for the 32 tiles one XCD's L2 serves at once; always
 * for the 64 x 64 instance). Returns the width, or -GEMM355_ERR_INVALID_ARG
 * for an unknown kernel, tiles_n <= 0 or K < 0. Pure host arithmetic.
 */
int gemm355_supergroup(int kernel, int tiles_n, int K);

/*
 * gemm355_force_schedule -- tile order of gemm_nvfp4_nt's persistent kernel
 * ("NVFP4 GEMM on Blackwell", "Production Kernel", "Static vs Dynamic Tile
 * Scheduling"), a diagnostic for measurements: 0 (the default) the static
 * order; 1 a dynamic order -- one ticket counter per XCD, each workgroup
 * asking for its next tile as it starts the current one (one lane's atomic
 * add), taking tiles from the other XCDs once its own has none left. Applies
 * to gemm_nvfp4_nt with K % 64 == 0 (other calls keep the static order). The
 * result does not depend on the order. The counters are one fixed set per
 * device, cleared by the last workgroup of each launch: products running at
 * the same time on one GPU must not use the dynamic order. Returns GEMM355_OK
 * or GEMM355_ERR_INVALID_ARG for another mode (setting unchanged). No HIP
 * call is made.
 */
int gemm355_force_schedule(int mode);

/*
 * gemm355_bf16_plan -- the instance a BF16 product would run for M x N x K on
 * a device with `compute_units` compute units, under the current
 * gemm355_force_instance setting: gemm_bf16_nt / gemm_bf16_nt_bias_act when
 * with_workspace is 0, the *_ws entry points otherwise.
 *
 * A diagnostic for tests and measurements (it is not defined by the pages).
 * Writes the instance (1 = 256 x 256, 2 = 64 x 64, 3 = 128 x 128) to
 * *instance, the number of K splits (1 unless the instance is 3 and a
 * workspace is allowed) to *splits and the workspace bytes the plan needs to
 * *workspace_bytes. Returns GEMM355_OK, or GEMM355_ERR_INVALID_ARG for
 * M <= 0, N <= 0, K < 0, compute_units <= 0 or a NULL output pointer
 * (outputs then unchanged). Pure host arithmetic: no HIP call is made.
 */
int gemm355_bf16_plan(int M, int N, int K, int compute_units, int with_workspace, int *instance, int *splits,
                      size_t *workspace_bytes);

/*
 * gemm_nvfp4_nt -- block-scaled FP4 operands, BF16 output.
 *
 * ("NVFP4 GEMM on Blackwell", section "NVFP4 Datatype".)
 *   Aq   M x K/2 bytes: E2M1 codes, two per byte, element k = 2j in the low
 *        nibble of byte j and k = 2j+1 in the high nibble. An E2M1 code is
 *        sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; its 16
 *        values are +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}.
 *   SFA  M x K/16 bytes: one E4M3 ("FN": bias 7, no infinities) scale per 16
 *        consecutive elements of a row, row-major.
 *   Bq, SFB  the same for the N x K operand B.
 *   C    M x N BF16 output, row-major.
 * a(m,k) = e2m1(Aq code) * e4m3(SFA[m][k/16]), likewise b(n,k), and
 * C[m][n] = bf16( sum_k a(m,k) * b(n,k) ) with FP32 sums. There is no
 * per-tensor global scale. Every decoded element is exact in BF16 and in FP16
 * (at most 6 significant bits, magnitude within [2^-10, 2688]).
 * Edge cases as for gemm_bf16_nt.
 * Requirements, else GEMM355_ERR_UNSUPPORTED: Aq, Bq, C 16-byte aligned; SFA,
 * SFB 4-byte aligned; K % 32 == 0 (whole 16-byte groups of codes per row and
 * whole pairs of scale blocks); N % 8 == 0; extents as for gemm_bf16_nt.
 */
int gemm_nvfp4_nt(int M, int N, int K, const void *Aq, const void *SFA, const void *Bq,
                  const void *SFB, void *C, void *stream);

/*
 * gemm_nvfp4_nt_bias_act -- the block-scaled FP4 product with the fused
 * epilogue of gemm_bf16_nt_bias_act ("NVFP4 GEMM on Blackwell", "Kernel 1",
 * "Epilogue Warps"):
 *
 *   C[m][n] = bf16_rne(act(fp32(sum_k a(m,k) * b(n,k)) + bias[n]))
 *
 * with a, b, layouts and requirements as for gemm_nvfp4_nt and bias,
 * activation and their errors as for gemm_bf16_nt_bias_act (bias: N BF16
 * values, 16-byte aligned, or NULL; K == 0 gives act(bias[n])).
 */
int gemm_nvfp4_nt_bias_act(int M, int N, int K, const void *Aq, const void *SFA, const void *Bq,
                           const void *SFB, const void *bias, int activation, void *C, void *stream);

/*
 * gemm_nvfp4_nt_ws -- gemm_nvfp4_nt with a workspace the caller owns, for
 * products large enough that decoding each operand once beats decoding it
 * while staging. The staging-decode kernel decodes every operand strip again
 * for each 256 x 256 tile that uses it (N/256 times for A, M/256 times for
 * B), and writing the decoded values into LDS costs it matrix-busy cycles
 * that the BF16 kernels on decoded rows do not lose. When the saving
 * outweighs the decode -- the persistent grid
 * runs at least two rounds of 256 x 256 tiles and the rounds times 7000
 * exceed M + N, a balance measured on MI355X (on 256 units: M = N = 5120,
 * 6144 or 8192 decode first, M = N = 4096 and M x N = 2048 x 16384 do not,
 * for any K) -- this call decodes A into M x K BF16 rows at the workspace start and
 * B into N x K BF16 rows after it (at the next 256-byte boundary) -- the
 * decoding of gemm_nvfp4_nt, exact in BF16 -- then runs the BF16 product
 * (the kernels of gemm_bf16_nt) on them, all on `stream`. Otherwise it runs
 * gemm_nvfp4_nt and leaves the workspace untouched.
 * Results: within the parity bound of gemm_nvfp4_nt's (the FP32 sums run in
 * another order), bitwise equal where every partial sum is exact.
 * Arguments and requirements as for gemm_nvfp4_nt, plus: the workspace is
 * device memory of at least gemm_nvfp4_nt_workspace_size bytes, 16-byte
 * aligned, else GEMM355_ERR_UNSUPPORTED; NULL with workspace_bytes > 0, or a
 * workspace overlapping an operand or C, is GEMM355_ERR_INVALID_ARG; the
 * decoded operands (2 M K and 2 N K bytes, rows padded to 256) must stay
 * below 2^31 bytes each, else GEMM355_ERR_UNSUPPORTED. The library keeps no
 * reference to the workspace: it may be reused once the call's work on
 * `stream` is done; calls that run concurrently need their own.
 */
int gemm_nvfp4_nt_ws(int M, int N, int K, const void *Aq, const void *SFA, const void *Bq, const void *SFB,
                     void *C, void *workspace, size_t workspace_bytes, void *stream);

/*
 * gemm_nvfp4_nt_bias_act_ws -- gemm_nvfp4_nt_bias_act with a workspace the
 * caller owns: the product of gemm_nvfp4_nt_ws (the same shape rule, the same
 * workspace size and layout) with the fused epilogue of
 * gemm_nvfp4_nt_bias_act ("NVFP4 GEMM on Blackwell", "Kernel 1", "Epilogue
 * Warps": bias per output column added to the FP32 sum, then the activation,
 * before the BF16 rounding), applied by whichever kernel writes C.
 * Arguments, requirements and errors as for those two calls; a workspace
 * overlapping the bias is also GEMM355_ERR_INVALID_ARG.
 */
int gemm_nvfp4_nt_bias_act_ws(int M, int N, int K, const void *Aq, const void *SFA, const void *Bq,
                              const void *SFB, const void *bias, int activation, void *C, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * gemm_nvfp4_nt_workspace_size -- *bytes = the workspace gemm_nvfp4_nt_ws
 * uses for this shape on the current device: 2 M K rounded up to a multiple
 * of 256, plus 2 N K, when it decodes first; else 0 (also for M, N or K = 0).
 * Errors: GEMM355_ERR_INVALID_ARG (negative size, NULL bytes),
 * GEMM355_ERR_NO_DEVICE.
 */
int gemm_nvfp4_nt_workspace_size(int M, int N, int K, size_t *bytes);

/*
 * gemm355_nvfp4_plan -- host-only: whether gemm_nvfp4_nt_ws decodes first
 * for this shape on a device with `compute_units` compute units
 * (*decode_first = 1) and the workspace bytes it then needs (0 otherwise),
 * under the current gemm355_force_fp4_path setting. Errors:
 * GEMM355_ERR_INVALID_ARG for M or N <= 0, K < 0, compute_units <= 0 or a
 * NULL output.
 */
int gemm355_nvfp4_plan(int M, int N, int K, int compute_units, int *decode_first, size_t *workspace_bytes);

/*
 * gemm355_force_fp4_path -- gemm_nvfp4_nt_ws's choice, a process-wide
 * diagnostic for tests and measurements: 0 (default) by shape as above, 1
 * always the staging-decode kernel, 2 always decode first (when K > 0).
 * Errors: GEMM355_ERR_INVALID_ARG for other values.
 */
int gemm355_force_fp4_path(int path);

/*
 * gemm_mxfp4_nt -- C = A * B^T for microscaled FP4 operands (E2M1 codes with
 * one E8M0 power-of-two scale per 32 elements), on the gfx950 matrix cores'
 * own block scaling (v_mfma_scale_f32_16x16x128_f8f6f4, four times the BF16
 * rate). Not a format of the pages: their FP4 variant scales every 16
 * elements by an E4M3 value ("NVFP4 GEMM on Blackwell", "NVFP4 Datatype"),
 * whose mantissa the hardware scaling cannot apply; this is the block-scaled
 * matrix product with scales applied inside the instruction, in the format
 * the hardware takes.
 *
 *   a(m,k) = e2m1(code(m,k)) * 2^(SA[m][k/32] - 127),  likewise b(n,k)
 *   C[m][n] = bf16_rne(fp32(sum_k a(m,k) * b(n,k)))
 *
 *   Aq   M x K/2 bytes, row-major: two codes per byte, even k in the low nibble
 *   SA   M x K/32 E8M0 bytes, row-major (0xFF, NaN, is not supported)
 *   Bq, SB  the same with N rows;  C  M x N BF16, row-major.
 * Products of two scaled E2M1 values are exact; sums are FP32 (order
 * unspecified). Ownership, streams and edge cases as for gemm_nvfp4_nt.
 * Requirements, else GEMM355_ERR_UNSUPPORTED: K % 512 == 0 (scales travel
 * 16 bytes per row at a time), N % 8 == 0; Aq, Bq, SA, SB, C 16-byte aligned;
 * extents as for the other products. 256 x 256 output tiles.
 */
int gemm_mxfp4_nt(int M, int N, int K, const void *Aq, const void *SA, const void *Bq, const void *SB, void *C,
                  void *stream);

/*
 * gemm_mxfp4_nt_bias_act -- the microscaled FP4 product with the fused
 * epilogue of gemm_bf16_nt_bias_act ("NVFP4 GEMM on Blackwell", "Kernel 1",
 * "Epilogue Warps"):
 *
 *   C[m][n] = bf16_rne(act(fp32(sum_k a(m,k) * b(n,k)) + bias[n]))
 *
 * with a, b, layouts and requirements as for gemm_mxfp4_nt and bias,
 * activation and their errors as for gemm_bf16_nt_bias_act (bias: N BF16
 * values, 16-byte aligned, or NULL; K == 0 gives act(bias[n])).
 */
int gemm_mxfp4_nt_bias_act(int M, int N, int K, const void *Aq, const void *SA, const void *Bq, const void *SB,
                           const void *bias, int activation, void *C, void *stream);

/* Human-readable text for a status code (static storage; never NULL). */
const char *gemm355_status_string(int status);

/*
 * gemm355_tile_order -- host-only view of the output-tile visiting order.
 *
 * Writes, for positions p = 0 .. tiles_m*tiles_n - 1 of the visiting order,
 * the tile coordinates tm[p], tn[p]. The order is the "supergroup" order of
 * "NVFP4 GEMM on Blackwell", section "Kernel 5", "Redesign": bands of
 * `supergroup` adjacent N tiles; inside a band every M tile in turn, and for
 * each M tile the band's N tiles in turn; the last band may be narrower.
 * Returns GEMM355_ERR_INVALID_ARG for non-positive sizes or NULL outputs.
 * No HIP call is made.
 */
int gemm355_tile_order(int tiles_m, int tiles_n, int supergroup, int *tm, int *tn);

/*
 * gemm355_schedule -- host-only view of which workgroup computes which tile.
 *
 * For a persistent grid of `grid` workgroups, writes slot[w * rounds + r] =
 * the visiting-order position that workgroup w computes in its round r, or
 * -1 when it has none, for r < rounds = ceil(tiles / grid). Workgroups are
 * dispatched to the 8 XCDs round-robin (w % 8); positions are dealt out so
 * that the grid/8 workgroups of one XCD take consecutive positions in each
 * round. `slot` must hold grid * rounds ints. Returns the number of rounds,
 * or a negative status on bad arguments. No HIP call is made.
 */
int gemm355_schedule(int tiles, int grid, int *slot, int slot_len);

#ifdef __cplusplus
}
#endif

#endif /* GEMM355_H */
