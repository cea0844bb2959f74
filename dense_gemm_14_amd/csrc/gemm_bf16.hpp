// gemm_bf16.hpp -- persistent BF16 NT GEMM for gfx950 with operands copied
// straight from global memory into LDS (buffer_load_dwordx4 ... lds).
//
// Work decomposition
//   * Output tile 256 x 256 per workgroup, 4 waves in a 2 x 2 layout; each
//     wave owns a 128 x 128 block = 4 x 4 blocks of v_mfma_f32_32x32x16_bf16
//     whose FP32 accumulators (256 per lane) stay in the accumulation registers
//     for the whole K loop.
//   * K advances 64 at a time through two LDS stages of 64 KiB (A tile
//     256 x 64, then B tile 256 x 64, BF16). Each 1 KiB block of a stage is
//     written by one copy instruction of the memory pipeline (lane i fills
//     bytes 16 i .. 16 i + 15 of the block: 8 rows x 128 bytes), so operands
//     pass through no registers and no LDS-write instructions, and every
//     request is one whole 128-byte row segment of A or B.
//   * LDS tile rows are 128 bytes (64 elements, eight 16-byte chunks); logical
//     chunk c of row r sits at chunk position c ^ ((r >> 1) & 7). gfx950 serves
//     a ds_read_b128 16 lanes (256 bytes over 64 four-byte banks) per cycle;
//     the 16 lanes read 16 consecutive rows at one logical chunk, row parity
//     picks the 128-byte half of the bank space and (r >> 1) & 7 the chunk
//     within it, so the 16 lanes hit 16 distinct bank groups (measured: 4
//     cycles per read, no conflicts). The swizzle is applied on the global
//     side: the lane that fills position p of row r fetches logical chunk
//     p ^ ((r >> 1) & 7).
//   * Step kt (one barrier): sub-steps 0..2 run 16 matrix instructions each
//     on stage kt & 1 while the next sub-step's fragments are read; each wave
//     then waits for its own copies of slice kt + 1 (vmcnt), the barrier makes
//     all of them visible and releases stage kt & 1, and sub-step 3 runs while
//     the first fragments of slice kt + 1 are read and slice kt + 2 is
//     requested into the stage just released.
#pragma once

#include "common.hpp"

namespace gemm355 {
namespace bf16 {

constexpr int BK = 64;                       // K elements per pipeline step
constexpr int ROW_BYTES = BK * 2;            // 128-byte LDS rows
constexpr int TILE_BYTES = BM * ROW_BYTES;   // 32 KiB per operand per stage
constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // A tile then B tile
constexpr int STAGES = 2;
constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
constexpr int COPIES = 16;                   // 1 KiB copies per wave per step (8 A + 8 B)

static_assert(LDS_BYTES <= 163840, "LDS ring exceeds the 160 KiB of a gfx950 workgroup");
static_assert(BM == 256 && BN == 256 && THREADS == 256, "the copy map assumes 256 x 256 tiles and 4 waves");

// Physical 16-byte chunk position of logical chunk c in LDS tile row r (an
// involution: it also gives the logical chunk stored at position c).
__device__ inline int swizzle(int r, int c) { return c ^ ((r >> 1) & 7); }

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource as four scalar words, for the inline-assembly copies.
__device__ inline i32x4 rsrc_words(const void *p, unsigned bytes)
{
    const unsigned long long a = reinterpret_cast<unsigned long long>(p);
    return i32x4{(int)(unsigned)a, (int)(unsigned)(a >> 32), (int)bytes, (int)RSRC_WORD3};
}

// One 1 KiB global -> LDS copy: lane i's 16 bytes at byte offset `voff` of the
// buffer land at LDS byte lds_addr + 16 i. Written as inline assembly so the
// compiler does not treat the in-flight LDS write as aliasing every later LDS
// read (it would wait for all copies before each read); the kernel orders the
// copies itself with explicit vmcnt waits and barriers. m0 holds the LDS base;
// nothing else in this kernel uses m0.
__device__ inline void copy_1k(const i32x4 &rsrc, unsigned lds_addr, int voff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

// Every copy this wave issued has landed in LDS (stores too).
__device__ inline void wait_all_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__global__ __attribute__((amdgpu_flat_work_group_size(THREADS, THREADS), amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_nt_kernel(Problem p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1;   // wave's 128-row half of the tile (A rows)
    const int wn = wave >> 1;  // wave's 128-column half (B rows)
    const int l32 = lane & 31;
    const int half = lane >> 5;
    const int K = p.K;

    // Fragment reads: row l32 + 32 i of the wave's block, logical chunk
    // 2 kk + half for sub-step kk (rows differ from l32 by multiples of 32,
    // which leaves the swizzle unchanged).
    const int a_frag = (wm * 128 + l32) * ROW_BYTES;
    const int b_frag = TILE_BYTES + (wn * 128 + l32) * ROW_BYTES;
    int kofs[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        kofs[kk] = swizzle(l32, 2 * kk + half) << 4;

    // Copies: wave w fills blocks 8 w .. 8 w + 7 (rows 64 w .. 64 w + 63) of the
    // A tile and of the B tile; lane i fills position i & 7 of row 8 b + i / 8.
    const int copy_row = lane >> 3;
    const unsigned lds_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)lds;

    const i32x4 ra = rsrc_words(p.a, (unsigned)p.M * (unsigned)K * 2u);
    const i32x4 rb = rsrc_words(p.b, (unsigned)p.N * (unsigned)K * 2u);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.c, (unsigned)p.M * (unsigned)p.N * 2u);
    const int nk = (K + BK - 1) / BK;

    for (int round = 0;; ++round) {
        const int pos = schedule_position(blockIdx.x, round, p.grid);
        if (pos >= p.tiles)
            break;
        int tm, tn;
        supergroup_tile(pos, p.tiles_m, p.tiles_n, p.supergroup, tm, tn);

        // per block: byte offset of this lane's chunk in its A row and B row,
        // and the chunk's first K index (the K tail switches whole chunks off)
        int a_off[8], b_off[8], chunk_k[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int row = 8 * (8 * wave + j) + copy_row;
            const int c = swizzle(row, lane & 7);   // logical chunk stored at position lane & 7
            chunk_k[j] = 8 * c;
            a_off[j] = ((tm * BM + row) * K + 8 * c) * 2;
            b_off[j] = ((tn * BN + row) * K + 8 * c) * 2;
        }

        // Copy t (0..15) of K slice `slice` into its stage: block 8 w + t / 2
        // of A for even t, of B for odd t. Slices at or past K, and the K tail,
        // read as zeros; rows past M or N fall outside the buffer and do too.
        auto copy = [&](int slice, int t) {
            const int k0 = slice * BK;
            const int j = t >> 1;
            const bool valid = k0 + chunk_k[j] < K;
            const unsigned dst = lds_base + (unsigned)((slice % STAGES) * STAGE_BYTES +
                                                       ((t & 1) ? TILE_BYTES : 0) + (8 * wave + j) * 1024);
            const int off = (t & 1) ? b_off[j] : a_off[j];
            copy_1k((t & 1) ? rb : ra, dst, valid ? off + k0 * 2 : OOB);
        };

        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = f32x16{};

        bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
        // fragment read r (0..7): A block r for r < 4, B block r - 4 otherwise
        auto read_frag = [&](const uint8_t *stage, int kofs, bf16x8 *fa, bf16x8 *fb, int r) {
            if (r < 4)
                fa[r] = *reinterpret_cast<const bf16x8 *>(stage + a_frag + r * 32 * ROW_BYTES + kofs);
            else
                fb[r - 4] = *reinterpret_cast<const bf16x8 *>(stage + b_frag + (r - 4) * 32 * ROW_BYTES + kofs);
        };
        // matrix instruction t (0..15) of a sub-step: block (t / 4, t % 4)
        auto mma = [&](const bf16x8 *fa, const bf16x8 *fb, int t) {
            const int i = t >> 2, j = t & 3;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
        };

        // Copies of the previous tile (including its zero slices past K) and its
        // stores have landed before the stages are refilled.
        wait_all_copies();
        lds_barrier();
#pragma unroll
        for (int t = 0; t < COPIES; ++t)
            copy(0, t);
        wait_all_copies();
        lds_barrier();
#pragma unroll
        for (int r = 0; r < 8; ++r)
            read_frag(lds, kofs[0], fa0, fb0, r);
#pragma unroll
        for (int t = 0; t < COPIES; ++t)
            copy(1, t);
        SCHED_FENCE();

        // The instruction order inside a step is fixed by hand (SCHED_FENCE
        // after every group): each matrix instruction is followed by at most
        // one fragment read and one copy.
        for (int kt = 0; kt < nk; ++kt) {
            const uint8_t *cur = lds + (kt % STAGES) * STAGE_BYTES;
            const uint8_t *nxt = lds + ((kt + 1) % STAGES) * STAGE_BYTES;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                mma(fa0, fb0, t);
                if (t < 8)
                    read_frag(cur, kofs[1], fa1, fb1, t);
                SCHED_FENCE();
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                mma(fa1, fb1, t);
                if (t < 8)
                    read_frag(cur, kofs[2], fa0, fb0, t);
                SCHED_FENCE();
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                mma(fa0, fb0, t);
                if (t < 8)
                    read_frag(cur, kofs[3], fa1, fb1, t);
                SCHED_FENCE();
            }
            wait_all_copies();     // this wave's copies of slice kt + 1 have landed
            lds_barrier();         // ... and everybody's; stage `cur` is released
            SCHED_FENCE();
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                mma(fa1, fb1, t);
                if (t < 8)
                    read_frag(nxt, kofs[0], fa0, fb0, t);
                copy(kt + 2, t);   // slice kt + 2 into the released stage
                SCHED_FENCE();
            }
        }

        store_tile(acc, rc, p.M, p.N, tm * BM + wm * 128, tn * BN + wn * 128, l32, half);
    }
    wait_all_copies(); // no copy may still be writing LDS when the workgroup ends
}

} // namespace bf16
} // namespace gemm355
