// gemm_bf16_small.hpp -- BF16 NT GEMM for gfx950 on 64 x 64 output tiles, for
// problems whose 256 x 256 tiles cannot fill the 256 compute units (few output
// rows or columns, e.g. M = 128 against N = K = 8192).
//
// Such problems are bound by memory traffic, not by the matrix cores: with
// 64 x 64 tiles every compute unit streams (64 + 64) rows x K of operands for
// 64 x 64 x K multiply-adds, and the per-unit copy rate and HBM decide the
// time. The kernel therefore spends its LDS on depth instead of tile size.
//
//   * 4 waves in 2 x 2, each wave 32 x 32 = 2 x 2 blocks of
//     v_mfma_f32_16x16x32_bf16 (16 accumulation registers per lane).
//   * K advances 64 per step. Stage = A tile (64 rows) + B tile (64 rows) of
//     one step, 128-byte rows, 16 KiB; STAGES stages form a ring. Each wave
//     copies two 1 KiB blocks of each operand per step with the LDS-DMA form
//     of buffer_load_dwordx4 (same row swizzle as the large-tile kernel).
//     A wave's four blocks are contiguous in the stage (A rows 16 w .. 16 w +
//     15, then the same B rows), so one m0 value serves all four copies, which
//     differ only in their instruction offset: rewriting m0 while an earlier
//     LDS copy still waits to use it stalls the wave (~50 cycles per copy when
//     the copies are back to back).
//   * Step s: copy step s + STAGES - 1 into the stage of step s - 1 (which
//     every wave finished reading before the previous barrier), wait until
//     this wave's copies of step s + 1 have landed, one barrier (everybody's
//     copies of step s + 1 are visible), then read the fragments of step
//     s + 1 interleaved with the eight matrix instructions of step s on
//     fragments read during step s - 1. Copies of a step are issued
//     STAGES - 2 steps before their first use and overlap the barrier.
#pragma once

#include "common.hpp"

#include <utility>

namespace gemm355 {
namespace bf16_small {

constexpr int TM = 64;                       // output tile rows
constexpr int TN = 64;                       // output tile columns
constexpr int BK = 64;                       // K elements per step
constexpr int ROW_BYTES = BK * 2;            // 128-byte LDS rows
constexpr int TILE_BYTES = TM * ROW_BYTES;   // 8 KiB per operand per stage
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
constexpr int STAGES = 10;
constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
constexpr int COPIES = 4;                    // 1 KiB copies per wave per step (2 A + 2 B)

static_assert(LDS_BYTES <= 163840, "LDS ring exceeds the 160 KiB of a gfx950 workgroup");
static_assert(TM == 64 && TN == 64 && THREADS == 256, "the copy map assumes 64 x 64 tiles and 4 waves");
static_assert(COPIES * (STAGES - 1) <= 63, "vmcnt counts at most 63 outstanding operations");

__device__ inline int swizzle(int r, int c) { return c ^ ((r >> 1) & 7); }

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ inline i32x4 rsrc_words(const void *p, unsigned bytes)
{
    const unsigned long long a = reinterpret_cast<unsigned long long>(p);
    return i32x4{(int)(unsigned)a, (int)(unsigned)(a >> 32), (int)bytes, (int)RSRC_WORD3};
}

// The instruction offset of a copy moves both its global address and its LDS
// destination. Buffer resources start SHIFT bytes before their operand (and
// span SHIFT bytes more) so that the per-lane offset, global offset + SHIFT -
// instruction offset, is never negative; OOB_SHIFTED stays past the end of
// every resource after any instruction offset is added.
constexpr int SHIFT = 3072;
constexpr unsigned OOB_SHIFTED = 0xFFFF0000u;

// Set the LDS base of the following copies.
// The s_nop: on gfx9 an LDS-DMA instruction must not directly follow a scalar
// write of m0 (one wait state).
__device__ inline void set_m0(unsigned lds_addr) { asm volatile("s_mov_b32 m0, %0\n\ts_nop 0" ::"s"(lds_addr) : "memory", "m0"); }

// One 1 KiB global -> LDS copy: lane i's 16 bytes at buffer offset voff + IMM
// land at LDS byte m0 + IMM + 16 i (inline assembly for the same reason as in
// the large-tile kernel; m0 is set by set_m0 and used by nothing else).
template <int IMM>
__device__ inline void copy_1k_at(const i32x4 &rsrc, unsigned voff)
{
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen offset:%2 lds" ::"v"(voff), "s"(rsrc), "n"(IMM) : "memory");
}

__device__ inline void wait_all_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int N>
__device__ inline void wait_copies_le() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
__device__ inline void wait_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// EPI: EPI_PLAIN, or the activation of the fused epilogue (bias, then the
// activation, before rounding).
template <int EPI>
__global__ __attribute__((amdgpu_flat_work_group_size(THREADS, THREADS), amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_nt_small_kernel(Problem p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
    constexpr bool FUSED = EPI != EPI_PLAIN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1;   // 32-row half of the tile (A rows)
    const int wn = wave >> 1;  // 32-column half (B rows)
    const int l16 = lane & 15;
    const int grp = lane >> 4;
    const int K = p.K;

    // fragment of a 16-row block: row l16, logical chunk grp (first half of
    // the step) or 4 + grp (second half)
    const int kofs[2] = {swizzle(l16, grp) << 4, swizzle(l16, 4 + grp) << 4};
    // Stage layout: wave region w (4 KiB) = A rows 16 w .. 16 w + 15 (two
    // 1 KiB blocks of 8 rows), then B rows 16 w .. 16 w + 15. Row r of A sits
    // at (r / 16) * 4096 + ((r / 8) & 1) * 1024 + (r & 7) * 128, row r of B
    // 2048 bytes further.
    const int a_frag = (2 * wm) * 4096 + (l16 >> 3) * 1024 + (l16 & 7) * ROW_BYTES;
    const int b_frag = 2048 + (2 * wn) * 4096 + (l16 >> 3) * 1024 + (l16 & 7) * ROW_BYTES;
    const int copy_row = lane >> 3;

    const unsigned lds_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)lds;
    const i32x4 ra = rsrc_words(static_cast<const uint8_t *>(p.a) - SHIFT, (unsigned)p.M * (unsigned)K * 2u + SHIFT);
    const i32x4 rb = rsrc_words(static_cast<const uint8_t *>(p.b) - SHIFT, (unsigned)p.N * (unsigned)K * 2u + SHIFT);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.c, (unsigned)p.M * (unsigned)p.N * 2u);
    // fused epilogue: bias[n] (zeros past N and without a bias: an empty range)
    const __amdgpu_buffer_rsrc_t rbias = make_rsrc(p.bias, FUSED && p.bias ? (unsigned)p.N * 2u : 0u);
    const int nk = (K + BK - 1) / BK;

    for (int round = 0;; ++round) {
        const int pos = schedule_position(blockIdx.x, round, p.grid);
        if (pos >= p.tiles)
            break;
        int tm, tn;
        supergroup_tile(pos, p.tiles_m, p.tiles_n, p.supergroup, tm, tn);

        // Copy t (0..3) of a step: rows 16 wave + 8 (t & 1) .. + 7 of the A
        // tile (t < 2) or of the B tile, into LDS bytes 1024 t of the wave's
        // region; lane i fills position i & 7 of row i / 8 of the block.
        int off[COPIES], chunk_k[COPIES];
#pragma unroll
        for (int t = 0; t < COPIES; ++t) {
            const int row = 16 * wave + 8 * (t & 1) + copy_row;
            const int c = swizzle(row, lane & 7);
            chunk_k[t] = 8 * c;
            off[t] = (((t < 2 ? tm * TM : tn * TN) + row) * K + 8 * c) * 2 + SHIFT - 1024 * t;
        }
        // Steps at or past the end of K, and the K tail, read as zeros; rows
        // past M or N fall outside the buffer and do too.
        auto copy = [&](int s, auto t_c) {
            constexpr int t = decltype(t_c)::value;
            const int k0 = s * BK;
            const bool valid = s < nk && k0 + chunk_k[t] < K;
            copy_1k_at<1024 * t>(t < 2 ? ra : rb, valid ? (unsigned)(off[t] + k0 * 2) : OOB_SHIFTED);
        };
        auto copy_base = [&](int s) {
            return lds_base + (unsigned)((s % STAGES) * STAGE_BYTES + wave * 4096);
        };

        f32x4 acc[2][2];
        bf16x8 fa[2][2][2], fb[2][2][2];   // [buffer][half][block]
        // read q (0..7) of a step: half q / 4, A block (q / 2) & 1 for even q,
        // B block for odd q (block b of the wave's operand rows is 4096 bytes
        // after block 0)
        auto read = [&](int s, int buf, int q) {
            const uint8_t *stage = lds + (s % STAGES) * STAGE_BYTES;
            const int h = q >> 2, i = (q >> 1) & 1;
            if (q & 1)
                fb[buf][h][i] = *reinterpret_cast<const bf16x8 *>(stage + b_frag + i * 4096 + kofs[h]);
            else
                fa[buf][h][i] = *reinterpret_cast<const bf16x8 *>(stage + a_frag + i * 4096 + kofs[h]);
        };
        auto read_step = [&](int s, int buf) {
#pragma unroll
            for (int q = 0; q < 8; ++q)
                read(s, buf, q);
        };
        // matrix instruction t (0..7): half t / 4, block ((t / 2) & 1, t & 1)
        auto mma = [&](int buf, int t, bool first) {
            const int h = t >> 2, i = (t >> 1) & 1, j = t & 1;
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[buf][h][j], fa[buf][h][i],
                                                               (first && h == 0) ? f32x4{} : acc[i][j], 0, 0, 0);
        };

        // The previous tile's copies, reads and stores are done before the
        // ring is refilled; then steps 0 .. STAGES - 1 fill it.
        wait_reads();
        wait_all_copies();
        lds_barrier();
        // fused epilogue: bias[n .. n + 3] of this lane's columns in blocks
        // 0 and 1 (older than every copy of the tile, so landed by the first
        // step's wait)
        u32x2 bias_w[2];
        if constexpr (FUSED) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int n = tn * TN + wn * 32 + 16 * j + 4 * grp;
                bias_w[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rbias, n < p.N ? n * 2 : OOB, 0, 0));
            }
        }
        for (int s = 0; s < STAGES - 1; ++s) {
            set_m0(copy_base(s));
            copy(s, Int<0>{});
            copy(s, Int<1>{});
            copy(s, Int<2>{});
            copy(s, Int<3>{});
        }
        wait_copies_le<COPIES * (STAGES - 2)>();
        lds_barrier();
        read_step(0, 0);

        auto step = [&](int s, int buf, bool first) {
            // fragments of step s have arrived and this wave's copies of step
            // s + 1 have landed; after the barrier the stage of step s is free
            // step s + STAGES - 1 goes into the stage of step s - 1, which every
            // wave finished reading before the previous barrier
            set_m0(copy_base(s + STAGES - 1));
            copy(s + STAGES - 1, Int<0>{});
            copy(s + STAGES - 1, Int<1>{});
            copy(s + STAGES - 1, Int<2>{});
            copy(s + STAGES - 1, Int<3>{});
            wait_reads();
            wait_copies_le<COPIES * (STAGES - 2)>();
            lds_barrier();
            SCHED_FENCE();
            // matrix instruction t, then reads 2 t, 2 t + 1
            static_for<8>([&](auto tc) {
                constexpr int t = decltype(tc)::value;
                mma(buf, t, first);
                if constexpr (t < 4) {
                    read(s + 1, buf ^ 1, 2 * t);
                    read(s + 1, buf ^ 1, 2 * t + 1);
                }
                SCHED_VALU_ONLY();
            });
        };

        if (nk == 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = f32x4{};
        } else {
            step(0, 0, true);
            int s = 1;
            for (; s + 1 < nk; s += 2) {
                step(s, 1, false);
                step(s + 1, 0, false);
            }
            if (s < nk)
                step(s, 1, false);
        }

        // Epilogue as in the large-tile kernel: lane (l16, grp) of block (i, j)
        // holds C[m][n .. n + 3], m = m0 + 16 i + l16, n = n0 + 16 j + 4 grp;
        // v_permlane16_swap turns the block pair (0, 1) into one 16-byte row
        // segment per lane.
        const int m = tm * TM + wm * 32 + l16;
        const int n = tn * TN + wn * 32 + 16 * (grp & 1) + 8 * (grp >> 1);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            f32x4 x = acc[i][0];
            f32x4 y = acc[i][1];
            if constexpr (FUSED) {
                x = epilogue4<EPI>(x, bias_w[0]);
                y = epilogue4<EPI>(y, bias_w[1]);
            }
            const unsigned x0 = pack_bf16(x[0], x[1]), x1 = pack_bf16(x[2], x[3]);
            const unsigned y0 = pack_bf16(y[0], y[1]), y1 = pack_bf16(y[2], y[3]);
            const auto s0 = __builtin_amdgcn_permlane16_swap(x0, y0, false, false);
            const auto s1 = __builtin_amdgcn_permlane16_swap(x1, y1, false, false);
            const u32x4 out = {s0[0], s1[0], s0[1], s1[1]};
            const int mm = m + 16 * i;
            const int o = (mm < p.M && n < p.N) ? (mm * p.N + n) * 2 : OOB;
            __builtin_amdgcn_raw_buffer_store_b128(out, rc, o, 0, 0);
        }
    }
    wait_reads();
    wait_all_copies(); // no copy may still be writing LDS when the workgroup ends
}

} // namespace bf16_small
} // namespace gemm355
