// common.hpp -- pieces shared by the gfx950 kernels of libgemm355: vector
// types, the problem descriptor, buffer resources, barriers, scheduling hints
// and the epilogue that turns the FP32 accumulators of one 256 x 256 tile into
// BF16 rows of C.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "schedule.hpp"

namespace gemm355 {

// Compile-time loop: f(Int<0>{}), ..., f(Int<N - 1>{}).
template <int V> struct Int { static constexpr int value = V; };
template <class F, int... I>
__device__ inline void static_for_impl(F &&f, std::integer_sequence<int, I...>) { (f(Int<I>{}), ...); }
template <int N, class F>
__device__ inline void static_for(F &&f) { static_for_impl(f, std::make_integer_sequence<int, N>{}); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256;                      // output tile rows (M)
constexpr int BN = 256;                      // output tile columns (N)
constexpr int THREADS = 256;                 // 4 waves of 64 lanes, 2 x 2 over the tile
constexpr int OOB = (int)0x80000000;         // buffer offset beyond every range
constexpr unsigned RSRC_WORD3 = 0x00020000u; // raw buffer, 32-bit data format

struct Problem {
    const void *a;    // BF16 A, or E2M1 codes of A
    const void *b;    // BF16 B, or E2M1 codes of B
    const void *sfa;  // E4M3 scales of A (FP4 only)
    const void *sfb;  // E4M3 scales of B (FP4 only)
    void *c;
    const void *bias; // fused epilogue only: N BF16 values, or NULL (zeros)
    int M, N, K;
    int tiles_m, tiles_n, tiles;
    int supergroup;
    int grid;
};

// ---- fused epilogue --------------------------------------------------------
//
// This library's fused epilogue ("NVFP4 GEMM on Blackwell", "Kernel 1",
// "Epilogue Warps"): each FP32 sum gets its column's bias added and then the
// chosen activation, both in FP32 and while the sum is still in registers,
// and only then is it rounded to BF16 -- z = acc + bias[n], y = act(z).
enum Activation { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU_TANH = 2 };
// Kernel template argument EPI: EPI_PLAIN (no fused epilogue: C = the rounded
// sum), or the Activation of the fused epilogue (bias added in every case).
constexpr int EPI_PLAIN = -1;

// BF16 pair (low half = lower column) -> two floats, exactly.
__device__ inline float bf16_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float bf16_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// GELU, tanh form: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))), evaluated
// as z / (1 + exp(-2 u)) with u the tanh argument (the same function:
// 0.5 (1 + tanh u) = 1 / (1 + exp(-2 u))). exp overflows to +inf for very
// negative z, giving -0; it underflows to 0 for large z, giving z. The
// hardware exponential and reciprocal (about 1 ulp each) replace the
// correctly rounded division, a ten-instruction sequence per element.
template <int ACT>
__device__ inline float activate(float z)
{
    if constexpr (ACT == ACT_RELU) {
        return z > 0.0f ? z : 0.0f;
    } else if constexpr (ACT == ACT_GELU_TANH) {
        const float u = z * (0.7978845608f + 0.0356774081f * z * z);
        return z * __builtin_amdgcn_rcpf(1.0f + __expf(-2.0f * u));
    } else {
        return z;
    }
}

// z = x + bias (bias as two BF16 pairs: columns 0, 1 in w[0], 2, 3 in w[1]),
// then the activation, for four consecutive columns.
template <int ACT>
__device__ inline f32x4 epilogue4(f32x4 x, u32x2 w)
{
    return f32x4{activate<ACT>(x[0] + bf16_lo(w[0])), activate<ACT>(x[1] + bf16_hi(w[0])),
                 activate<ACT>(x[2] + bf16_lo(w[1])), activate<ACT>(x[3] + bf16_hi(w[1]))};
}


// A buffer resource whose range ends at the operand's last byte: loads past it
// return 0 and stores past it are dropped, which makes row tails (m >= M,
// n >= N) free and lets an offset of OOB switch one access off.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *p, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, RSRC_WORD3);
}

__device__ inline unsigned pack_bf16(float lo, float hi)
{
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2)); // round to nearest even
}

// Make this wave's LDS writes visible to the workgroup and wait for all waves.
// Only LDS is fenced: global loads still in flight stay in flight.
__device__ inline void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3..0 and 15..14, expcnt
// 6..4, lgkmcnt 11..8). vmcnt_le(n) waits until at most n vector-memory
// operations of this wave are outstanding and leaves the other counters alone.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(waitcnt_vm(n))
#define WAIT_ALL() __builtin_amdgcn_s_waitcnt(0)

// ---- instruction interleaving hints ---------------------------------------
//
// Each hint asks the scheduler for `n` instructions of one class at this point
// of the region's order (classes: matrix, LDS read, LDS write, global read,
// vector ALU); SCHED_FENCE stops the scheduler from moving anything across.
enum : int { SG_VALU = 0x002, SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100, SG_DS_WRITE = 0x200 };
#define SCHED(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)
#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)
// Like SCHED_FENCE, but plain vector ALU instructions may still cross.
#define SCHED_VALU_ONLY() __builtin_amdgcn_sched_barrier(SG_VALU)

// One sub-step: 16 matrix instructions with 8 fragment reads threaded in,
// one read after each of the first 8.
__device__ inline void schedule_reads_with_mma()
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        SCHED(SG_MFMA, 1);
        SCHED(SG_DS_READ, 1);
    }
    SCHED(SG_MFMA, 8);
}

// ---- epilogue ------------------------------------------------------------------
//
// The matrix instruction is fed B rows as its first operand and A rows as its
// second, so each 32 x 32 result block arrives transposed: lane (l32, half)
// of block (i, j) holds C[m][nb + 8 g + 4 half + e] in acc[i][j][4 g + e],
// m = row of the lane. Pairs of 4-column runs are exchanged between the two
// half-waves (v_permlane32_swap) so every lane stores one 16-byte row segment;
// a wave's store instruction covers 32 rows x 32 bytes.
//
// EPI: EPI_PLAIN, or the activation of the fused epilogue, applied with the
// bias of each column (rbias: N BF16 values; an empty range reads zeros).
// BI x BJ blocks of 32 x 32 (the wave's tile is 32 BI x 32 BJ).
template <int EPI, int BI, int BJ>
__device__ inline void store_tile(f32x16 (&acc)[BI][BJ], const __amdgpu_buffer_rsrc_t &rc,
                                  const __amdgpu_buffer_rsrc_t &rbias, int M, int N, int m0, int n0, int l32,
                                  int half)
{
    // fused: bias[n .. n + 3] of this lane's four-column runs, [j][g], columns
    // n0 + 32 j + 8 g + 4 half
    u32x2 bias_w[BJ][4];
    if constexpr (EPI != EPI_PLAIN) {
#pragma unroll
        for (int j = 0; j < BJ; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + 32 * j + 8 * g + 4 * half;
                bias_w[j][g] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rbias, n < N ? n * 2 : OOB, 0, 0));
            }
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
        const int m = m0 + i * 32 + l32;
#pragma unroll
        for (int j = 0; j < BJ; ++j) {
            const int nb = n0 + j * 32;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int g0 = 2 * q;
                f32x4 lo = {acc[i][j][4 * g0 + 0], acc[i][j][4 * g0 + 1], acc[i][j][4 * g0 + 2], acc[i][j][4 * g0 + 3]};
                f32x4 hi = {acc[i][j][4 * g0 + 4], acc[i][j][4 * g0 + 5], acc[i][j][4 * g0 + 6], acc[i][j][4 * g0 + 7]};
                if constexpr (EPI != EPI_PLAIN) {
                    lo = epilogue4<EPI>(lo, bias_w[j][g0]);
                    hi = epilogue4<EPI>(hi, bias_w[j][g0 + 1]);
                }
                unsigned x0 = pack_bf16(lo[0], lo[1]);
                unsigned x1 = pack_bf16(lo[2], lo[3]);
                unsigned y0 = pack_bf16(hi[0], hi[1]);
                unsigned y1 = pack_bf16(hi[2], hi[3]);
                // the lower half-wave keeps group g0 and receives the upper
                // half's part of it; the upper half-wave ends up with g0 + 1
                auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
                auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
                const u32x4 out = {s0[0], s1[0], s0[1], s1[1]};
                const int n = nb + (g0 + half) * 8;
                const int off = (m < M && n < N) ? (m * N + n) * 2 : OOB;
                __builtin_amdgcn_raw_buffer_store_b128(out, rc, off, 0, 0);
            }
        }
    }
}

// Epilogue for 16 x 16 result blocks. The matrix instruction is fed B rows
// as its first operand and A rows as its second, so lane (l16, grp) of block
// (i, j) holds C[m][n .. n + 3], m = m0 + 16 i + l16, n = n0 + 16 j + 4 grp.
// For x = block (i, 2 jp) and y = block (i, 2 jp + 1), v_permlane16_swap
// exchanges lane groups so that group 0 holds columns 0..7 of x, group 1
// columns 0..7 of y, group 2 columns 8..15 of x and group 3 columns 8..15 of
// y: one 16-byte store per lane, 64 contiguous bytes per C row and pair.
// BI x BJ blocks (BJ even; the wave's tile is 16 BI x 16 BJ).
template <int EPI, int BI, int BJ>
__device__ inline void store_tile16(f32x4 (&acc)[BI][BJ], const __amdgpu_buffer_rsrc_t &rc,
                                    const __amdgpu_buffer_rsrc_t &rbias, int M, int N, int m0, int n0, int lane)
{
    static_assert(BJ % 2 == 0, "blocks are stored in pairs of columns");
    const int l16 = lane & 15, grp = lane >> 4;
    // fused: bias[n .. n + 3] of this lane's columns in block column j
    u32x2 bias_w[BJ];
    if constexpr (EPI != EPI_PLAIN) {
#pragma unroll
        for (int j = 0; j < BJ; ++j) {
            const int n = n0 + 16 * j + 4 * grp;
            bias_w[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rbias, n < N ? n * 2 : OOB, 0, 0));
        }
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
        const int m = m0 + 16 * i + l16;
#pragma unroll
        for (int jp = 0; jp < BJ / 2; ++jp) {
            f32x4 x = acc[i][2 * jp], y = acc[i][2 * jp + 1];
            if constexpr (EPI != EPI_PLAIN) {
                x = epilogue4<EPI>(x, bias_w[2 * jp]);
                y = epilogue4<EPI>(y, bias_w[2 * jp + 1]);
            }
            const unsigned x0 = pack_bf16(x[0], x[1]), x1 = pack_bf16(x[2], x[3]);
            const unsigned y0 = pack_bf16(y[0], y[1]), y1 = pack_bf16(y[2], y[3]);
            const auto s0 = __builtin_amdgcn_permlane16_swap(x0, y0, false, false);
            const auto s1 = __builtin_amdgcn_permlane16_swap(x1, y1, false, false);
            const u32x4 out = {s0[0], s1[0], s0[1], s1[1]};
            const int n = n0 + 32 * jp + 16 * (grp & 1) + 8 * (grp >> 1);
            const int off = (m < M && n < N) ? (m * N + n) * 2 : OOB;
            __builtin_amdgcn_raw_buffer_store_b128(out, rc, off, 0, 0);
        }
    }
}

} // namespace gemm355
