// gemm_bf16_small_long.hpp -- the 64 x 64-tile BF16 NT GEMM of
// gemm_bf16_small.hpp, restaged for long K with enough tiles to keep HBM busy
// (the skinny workload: M = 128 against N = K = 8192, 256 tiles).
//
// There the kernel streams B from HBM, and what the memory delivers depends on
// how much of a row one request covers: B is row-major with K-long rows, and
// a K step of 64 touches only 128 bytes of each of its 64 rows. This variant
// fetches B in 512-byte row segments (four steps at a time) and keeps A, which
// stays in L2, in per-step units. The results are bitwise those of the other
// 64 x 64 kernel (same blocks, same per-element summation order).
//
//   * 4 waves in 2 x 2, each wave 32 x 32 = 2 x 2 blocks of
//     v_mfma_f32_16x16x32_bf16 (16 accumulation registers per lane).
//   * K advances 64 per step. The A tile of a step (64 rows of 128 bytes,
//     8 KiB) has a ring of 8 units. B, which streams from HBM, comes in
//     super-steps of 4 steps: 64 rows of 512 bytes (32 KiB), a ring of 3.
//     Measured with a streaming probe on MI355X (LDS-DMA of a 128 MiB
//     row-major matrix, one workgroup per unit): 128-byte row segments per
//     request stream at 4.0 TB/s, 512-byte ones at 4.6 and 1 KiB at 4.9; with
//     the A copies beside them, 44.7 against 38.3 us for the whole transfer.
//   * Copies are LDS-DMA (buffer_load_dwordx4 ... lds). Wave w copies A rows
//     16 w .. 16 w + 15 of each step (two 1 KiB copies of 8 rows x 128 bytes,
//     chunk c of row r at position c ^ ((r >> 1) & 7)) and B rows 16 w .. 16 w
//     + 15 of each super-step (eight 1 KiB copies of 2 rows x 512 bytes, two
//     per step; chunk c of row r at position c ^ (r & 15), which keeps the
//     fragment reads -- 16 rows at one chunk -- on 16 distinct bank groups).
//   * Step s: copy part s % 4 of super-step s / 4 + 2 into the unit of
//     super-step s / 4 - 1 and the A tile of step s + 7 into the unit of step
//     s - 1 (every wave finished reading both before the previous barrier),
//     wait until this wave's copies of step s + 1 have landed, one barrier,
//     then read the fragments of step s + 1 interleaved with the eight matrix
//     instructions of step s on fragments read during step s - 1.
#pragma once

#include "common.hpp"

#include <utility>

namespace gemm355 {
namespace bf16_small_long {

constexpr int TM = 64;                       // output tile rows
constexpr int TN = 64;                       // output tile columns
constexpr int BK = 64;                       // K elements per step
constexpr int ROW_BYTES = BK * 2;            // 128-byte A rows
constexpr int A_UNIT = TM * ROW_BYTES;       // A tile of one step: 8 KiB
constexpr int A_SLOTS = 8;
constexpr int B_BASE = A_SLOTS * A_UNIT;
constexpr int A_COPIES = 2;                  // 1 KiB copies per wave per step
constexpr int B_COPIES = 2;                  // 1 KiB copies per wave per step

// B staging: SUPER steps per B unit (512-byte rows), B_SLOTS units beside
// the A ring. (A template over SUPER; only SUPER = 4 is instantiated: with
// one step per B unit the kernel in gemm_bf16_small.hpp is faster.)
template <int SUPER>
struct BStage {
    static constexpr int ROW = SUPER * ROW_BYTES;        // bytes per B row in a unit
    static constexpr int UNIT = TN * ROW;                // 32 KiB
    static constexpr int SLOTS = 3;
    static constexpr int ROWS_PER_COPY = 1024 / ROW;     // rows one 1 KiB copy covers
    static constexpr int COPIES = SUPER * B_COPIES;      // this wave's copies of one unit
    static constexpr int LDS = B_BASE + SLOTS * UNIT;
    // At the wait of step s: this wave's copies issued after its last copy
    // of step s + 1 (B parts first, then A, in every step), by the phase s %
    // SUPER -- the vmcnt the wait may leave in flight.
    static constexpr int wait_left(int phase) { return phase == 0 ? 22 : phase == 3 ? 18 : 24; }
    static_assert(SUPER == 4, "the waits above are derived for four steps per B unit");
    static_assert(LDS <= 163840, "LDS rings exceed the 160 KiB of a gfx950 workgroup");
    static_assert((A_SLOTS - 1) * A_COPIES + (SLOTS - 1) * COPIES + 4 <= 63,
                  "vmcnt counts at most 63 outstanding operations");
};

static_assert(TM == 64 && TN == 64 && THREADS == 256, "the copy map assumes 64 x 64 tiles and 4 waves");

__device__ inline int swizzle(int r, int c) { return c ^ ((r >> 1) & 7); }      // A rows (8 chunks)
// B rows: 32 chunks of 512-byte rows
template <int SUPER>
__device__ inline int swizzle_b(int r, int c) { return c ^ (r & 15); }

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

__device__ inline void wait_all_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ inline void wait_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Two 1 KiB copies under one m0: lane i's 16 bytes at buffer offsets v0 and
// v1 + 1024 land at LDS bytes lds_addr + 16 i and lds_addr + 1024 + 16 i
// (inline assembly so that the compiler does not order every later LDS read
// after the in-flight LDS writes; the kernel orders them with vmcnt waits and
// barriers). On gfx9 an LDS-DMA instruction must not directly follow a scalar
// write of m0 (one wait state), hence the s_nop; nothing else uses m0.
__device__ inline void copy_pair(const i32x4 &rsrc, unsigned lds_addr, unsigned v0, unsigned v1)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %1, %3, 0 offen offset:0 lds\n\t"
                 "buffer_load_dwordx4 %2, %3, 0 offen offset:1024 lds"
                 :
                 : "s"(lds_addr), "v"(v0), "v"(v1), "s"(rsrc)
                 : "memory", "m0");
}

template <int N>
__device__ inline void wait_copies_left() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// EPI: EPI_PLAIN, or the activation of the fused epilogue (bias, then the
// activation, before rounding). SUPER: steps per B unit (4).
template <int EPI, int SUPER>
__global__ __attribute__((amdgpu_flat_work_group_size(THREADS, THREADS), amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_nt_small_long_kernel(Problem p)
{
    using BS = BStage<SUPER>;
    constexpr int B_ROW = BS::ROW, B_UNIT = BS::UNIT, B_SLOTS = BS::SLOTS;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[BS::LDS];
    constexpr bool FUSED = EPI != EPI_PLAIN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1;   // 32-row half of the tile (A rows)
    const int wn = wave >> 1;  // 32-column half (B rows)
    const int l16 = lane & 15;
    const int grp = lane >> 4;
    const int K = p.K;

    // Fragments of a 16-row block: row l16, logical chunk grp (first half of
    // the step) or 4 + grp (second half). A rows are 128 bytes in their
    // step's unit; B rows 512 bytes in their super-step's unit, where step
    // s % 4 holds logical chunks 8 (s % 4) .. 8 (s % 4) + 7.
    const int a_kofs[2] = {swizzle(l16, grp) << 4, swizzle(l16, 4 + grp) << 4};
    const int a_frag = (32 * wm + l16) * ROW_BYTES;
    const int b_frag = B_BASE + (32 * wn + l16) * B_ROW;
    auto b_kofs = [&](int phase, int h) { return swizzle_b<SUPER>(l16, 8 * phase + 4 * h + grp) << 4; };

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

        // A copy t (0, 1) of a step: rows 16 wave + 8 t .. + 7 of the A tile,
        // lane i at position i & 7 of row i / 8 (LDS byte 1024 t + 16 i of the
        // wave's 2 KiB). B copy u of a unit: rows 16 wave + R u .. + R - 1 (R =
        // 2 rows of 512 bytes, or 8 of 128), lane i at position i % (64 / R)
        // of row i / (64 / R) (LDS byte 1024 u + 16 i of the wave's 16 rows).
        // Offsets are per tile, less the instruction offset 1024 (t or u odd);
        // a step's K offset is added per copy.
        constexpr int R = BS::ROWS_PER_COPY, PER_ROW = 64 / R;
        unsigned a_off[A_COPIES], b_off[BS::COPIES];
        int a_k[A_COPIES], b_k[BS::COPIES];   // the lane's chunk, in K elements from the step / unit
#pragma unroll
        for (int t = 0; t < A_COPIES; ++t) {
            const int row = 16 * wave + 8 * t + (lane >> 3);
            a_k[t] = 8 * swizzle(row, lane & 7);
            a_off[t] = (unsigned)(((tm * TM + row) * K + a_k[t]) * 2 + SHIFT - 1024 * t);
        }
#pragma unroll
        for (int u = 0; u < BS::COPIES; ++u) {
            const int row = 16 * wave + R * u + lane / PER_ROW;
            b_k[u] = 8 * swizzle_b<SUPER>(row, lane % PER_ROW);
            b_off[u] = (unsigned)(((tn * TN + row) * K + b_k[u]) * 2 + SHIFT - 1024 * (u & 1));
        }
        // Steps and super-steps at or past the end of K, and the K tail, read
        // as zeros; rows past M or N fall outside the buffer and do too.
        auto copy_a = [&](int s) {
            const int k0 = s * BK;
            const unsigned dst = lds_base + (unsigned)((s % A_SLOTS) * A_UNIT + wave * 2048);
            unsigned v[A_COPIES];
#pragma unroll
            for (int t = 0; t < A_COPIES; ++t)
                v[t] = k0 + a_k[t] < K ? a_off[t] + (unsigned)(k0 * 2) : OOB_SHIFTED;
            copy_pair(ra, __builtin_amdgcn_readfirstlane(dst), v[0], v[1]);
        };
        // part `part` (0..3: copies 2 part, 2 part + 1) of super-step j
        auto copy_b = [&](int j, auto part_c) {
            constexpr int part = decltype(part_c)::value;
            const int k0 = j * SUPER * BK;
            const unsigned dst = lds_base + (unsigned)(B_BASE + (j % B_SLOTS) * B_UNIT + wave * 16 * B_ROW + part * 2048);
            unsigned v[2];
#pragma unroll
            for (int x = 0; x < 2; ++x)
                v[x] = k0 + b_k[2 * part + x] < K ? b_off[2 * part + x] + (unsigned)(k0 * 2) : OOB_SHIFTED;
            copy_pair(rb, __builtin_amdgcn_readfirstlane(dst), v[0], v[1]);
        };

        f32x4 acc[2][2];
        bf16x8 fa[2][2][2], fb[2][2][2];   // [buffer][half][block]
        // read q (0..7) of step s (phase s % 4): half q / 4, A block (q / 2) & 1
        // for even q, B block for odd q
        auto read = [&](int s, auto phase_c, int buf, int q) {
            constexpr int phase = decltype(phase_c)::value;
            const int h = q >> 2, i = (q >> 1) & 1;
            if (q & 1)
                fb[buf][h][i] = *reinterpret_cast<const bf16x8 *>(lds + ((s / SUPER) % B_SLOTS) * B_UNIT + b_frag +
                                                                  i * 16 * B_ROW + b_kofs(phase, h));
            else
                fa[buf][h][i] = *reinterpret_cast<const bf16x8 *>(lds + (s % A_SLOTS) * A_UNIT + a_frag +
                                                                  i * 16 * ROW_BYTES + a_kofs[h]);
        };
        // matrix instruction t (0..7): half t / 4, block ((t / 2) & 1, t & 1)
        auto mma = [&](int buf, int t, bool first) {
            const int h = t >> 2, i = (t >> 1) & 1, j = t & 1;
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[buf][h][j], fa[buf][h][i],
                                                               (first && h == 0) ? f32x4{} : acc[i][j], 0, 0, 0);
        };

        // The previous tile's copies, reads and stores are done before the
        // rings are refilled.
        wait_reads();
        wait_all_copies();
        lds_barrier();
        // fused epilogue: bias[n .. n + 3] of this lane's columns in blocks
        // 0 and 1 (older than every copy of the tile, so landed by the first
        // wait)
        u32x2 bias_w[2];
        if constexpr (FUSED) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int n = tn * TN + wn * 32 + 16 * j + 4 * grp;
                bias_w[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rbias, n < p.N ? n * 2 : OOB, 0, 0));
            }
        }
        // Prologue: the copies the steps before step 0 would have issued, in
        // the same order (B parts first, then A), so that the waits below count
        // alike: step t < 0 issues part t % SUPER of unit t / SUPER + B_SLOTS - 1
        // and the A tile of step t + A_SLOTS - 1, where those are >= 0.
        static_for<SUPER * (B_SLOTS - 1)>([&](auto ic) {
            constexpr int t = decltype(ic)::value - SUPER * (B_SLOTS - 1);   // virtual step, < 0
            constexpr int part = (t % SUPER + SUPER) % SUPER;
            constexpr int unit = (t - part) / SUPER + B_SLOTS - 1;
            if constexpr (unit >= 0)
                copy_b(unit, Int<part>{});
            if constexpr (t + A_SLOTS - 1 >= 0)
                copy_a(t + A_SLOTS - 1);
        });
        wait_copies_left<BS::wait_left(SUPER - 1)>();   // as at the wait of step -1: step 0 has landed
        lds_barrier();
#pragma unroll
        for (int q = 0; q < 8; ++q)
            read(0, Int<0>{}, 0, q);

        // Step s, phase s % 4 (fragment buffer s % 2): the copies of super-step
        // s / 4 + 2 (one part) and of A step s + 7; this wave's reads of step s
        // and its copies of step s + 1 are done after the wait; the barrier
        // makes everybody's copies of step s + 1 visible and frees the units
        // of step s - 1 (read during step s - 2).
        // idx: the step's place in its group of four (s % 4): phase idx % SUPER,
        // fragment buffer idx % 2
        auto step = [&](int s, auto idx_c, bool first) {
            constexpr int idx = decltype(idx_c)::value;
            constexpr int phase = idx % SUPER;
            constexpr int buf = idx & 1;
            copy_b(s / SUPER + B_SLOTS - 1, Int<phase>{});
            copy_a(s + A_SLOTS - 1);
            wait_reads();
            wait_copies_left<BS::wait_left(phase)>();
            lds_barrier();
            SCHED_FENCE();
            // matrix instruction t, then reads 2 t, 2 t + 1 of step s + 1
            static_for<8>([&](auto tc) {
                constexpr int t = decltype(tc)::value;
                mma(buf, t, first);
                if constexpr (t < 4) {
                    read(s + 1, Int<(idx + 1) % SUPER>{}, buf ^ 1, 2 * t);
                    read(s + 1, Int<(idx + 1) % SUPER>{}, buf ^ 1, 2 * t + 1);
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
            // steps in groups of four; the last group may be short
            for (int s = 0; s < nk; s += 4) {
                step(s, Int<0>{}, s == 0);
                if (s + 1 < nk)
                    step(s + 1, Int<1>{}, false);
                if (s + 2 < nk)
                    step(s + 2, Int<2>{}, false);
                if (s + 3 < nk)
                    step(s + 3, Int<3>{}, false);
            }
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

} // namespace bf16_small_long
} // namespace gemm355
