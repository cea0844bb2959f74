// gemm_mxfp4.hpp -- microscaled FP4 NT GEMM for gfx950 on the matrix cores'
// own block scaling: E2M1 codes (two per byte, even k in the low nibble) with
// one E8M0 (power-of-two) scale per 32 consecutive K elements of a row, fed
// undecoded to v_mfma_scale_f32_16x16x128_f8f6f4, which multiplies 128 K of
// a 16 x 16 block at four times the BF16 rate and applies each lane's scale
// to the 32 elements it holds.
//
// The format is not the pages' (their FP4 variant scales every 16 elements by
// an E4M3 value, "NVFP4 GEMM on Blackwell", section "NVFP4 Datatype", which
// has mantissa bits the hardware scaling cannot apply); it is the one whose
// scales the matrix cores take as operands, the MI355X counterpart of the
// page's block-scaled MMA with scales applied inside the instruction.
//
// Work decomposition
//   * Output tile 256 x 256 per workgroup, 8 waves in 2 x 4, each wave 128 x
//     64 = 8 x 4 blocks of 16 x 16 (128 accumulators per lane), two waves per
//     SIMD, so that one wave's matrix instructions run while the other is
//     held issuing copies or waiting on fragment reads. 16 x 16 blocks rather
//     than 32 x 32: half the accumulator traffic per product.
//   * K advances 128 per step: 64 bytes of codes per row (the LDS row) and 4
//     scale bytes. A stage holds the A and B code tiles (16 KiB each); four
//     stages (128 KiB) form a ring that runs on across the workgroup's tiles:
//     a tile's last three steps copy the next tile's first three, so neither
//     its epilogue stores nor a refill of the ring stall the next tile. Scales
//     come in blocks of four steps (16
//     bytes per row, 8 KiB per block for A and B) in a ring of two blocks
//     beside it (144 KiB in all). Code rows are 64 bytes:
//     logical 16-byte chunk c of row r sits at position c ^ ((r >> 2) & 3), so
//     the 16 rows a fragment read serves per cycle at one chunk cover the 16
//     bank groups of 256 bytes.
//   * Copies are LDS-DMA only (no registers carry operands): per step and
//     wave, two 1 KiB code copies of A (rows 32 w .. 32 w + 31, 16 rows
//     each) and two of B; per block of four steps one 1 KiB scale copy (64
//     rows of A for waves 0..3, of B for waves 4..7, 16 bytes each). Step k + 3 is
//     requested during step k, after the barrier that frees step k - 1's
//     stage, one copy every four matrix instructions over the first half of
//     the step (issued together they stall the wave).
//   * Per step each wave issues 32 matrix instructions, in groups of four
//     sharing an A block. Fragment reads (16 bytes per lane: row l % 16 of a
//     block, the 32 K of group l / 16) and the lane's scale byte of each
//     block are read three groups ahead for A, a step ahead for B.
#pragma once

#include "common.hpp"

#include <utility>

namespace gemm355 {
namespace mx {

constexpr int TM = 256;                          // output tile rows
constexpr int TN = 256;                          // output tile columns
constexpr int BK = 128;                          // K elements per step
constexpr int ROW_BYTES = BK / 2;                // 64 bytes of codes per row and step
constexpr int CODE_UNIT = TM * ROW_BYTES;        // 16 KiB
constexpr int SCALE_ROW = BK / 32;               // 4 scale bytes per row and step
constexpr int A_CODES = 0, B_CODES = CODE_UNIT;
constexpr int STAGE_BYTES = 2 * CODE_UNIT;       // A then B codes of one step
constexpr int STAGES = 4;
// Scales travel in blocks of four steps: 16 bytes per row (one 16-byte lane
// of a copy; a copy per step of 4 bytes per row touches a cache line per row
// and costs as much as all the code copies). Two blocks form their own ring.
constexpr int SCALE_STEPS = 4;
constexpr int SCALE_BLOCK_ROW = SCALE_STEPS * SCALE_ROW;   // 16 bytes
constexpr int SCALE_BLOCK = 2 * TM * SCALE_BLOCK_ROW;     // A then B: 8 KiB
constexpr int SCALES_BASE = STAGES * STAGE_BYTES;
constexpr int LDS_BYTES = SCALES_BASE + 2 * SCALE_BLOCK;
constexpr int THREADS_MX = 512;                  // 8 waves, two per SIMD
constexpr int COPIES = 4;                        // code copies per wave and step (2 + 2)
constexpr int SCALE_COPIES = 1;                  // per wave and scale block (A or B)
constexpr int EPILOGUE_STORES = 16;              // 16-byte stores per wave per tile (128 x 64 BF16)
constexpr int EPILOGUE_LOADS = 4;                // fused epilogue: bias loads per wave (one per 16-column block)

static_assert(LDS_BYTES <= 163840, "LDS ring exceeds the 160 KiB of a gfx950 workgroup");
static_assert(TM == 256 && TN == 256 && THREADS_MX == 512, "the copy map assumes 256 x 256 tiles and 8 waves");
// in flight at most: the copies of three steps ahead, a scale block and one
// epilogue's loads and stores (at a tile boundary fewer: the next tile's
// steps 1 and 2 and the epilogue)
static_assert((STAGES - 1) * COPIES + SCALE_COPIES + EPILOGUE_LOADS + EPILOGUE_STORES <= 63,
              "vmcnt counts at most 63 outstanding operations");

// Physical 16-byte chunk position of logical chunk c (0..3) in tile row r.
__device__ inline int swizzle(int r, int c) { return c ^ ((r >> 2) & 3); }

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ inline i32x4 rsrc_words(const void *p, unsigned bytes)
{
    const unsigned long long a = reinterpret_cast<unsigned long long>(p);
    return i32x4{(int)(unsigned)a, (int)(unsigned)(a >> 32), (int)bytes, (int)RSRC_WORD3};
}

// Resources start SHIFT bytes before their operand (and span SHIFT bytes
// more) so that per-lane offsets less an instruction offset stay non-negative;
// OOB_SHIFTED lies past every range and stays below 2^32 after any
// instruction and scalar offset is added (operand extents, and so scalar K
// offsets, are below 2^31).
constexpr int SHIFT = 3072;
constexpr unsigned OOB_SHIFTED = 0x80000000u;

// m0 = LDS base of the following copies; one wait state before LDS-DMA.
__device__ inline void set_m0(unsigned lds_addr) { asm volatile("s_mov_b32 m0, %0\n\ts_nop 0" ::"s"(lds_addr) : "memory", "m0"); }

// 1 KiB copy: lane i's 16 bytes at buffer offset voff + soff + IMM land at
// LDS byte m0 + IMM + 16 i. Rows past the operand have voff past its range;
// the scalar K offset soff (at most the row length) keeps them there.
template <int IMM>
__device__ inline void copy_1k(const i32x4 &rsrc, unsigned voff, int soff)
{
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:%3 lds" ::"v"(voff), "s"(rsrc), "s"(soff), "n"(IMM) : "memory");
}

__device__ inline void wait_all_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
template <int N>
__device__ inline void wait_copies_le() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
__device__ inline void wait_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Kernel arguments: Problem with a, b the codes and sfa, sfb the E8M0 scales.
// EPI: EPI_PLAIN, or the activation of the fused epilogue.
template <int EPI>
__global__ __attribute__((amdgpu_flat_work_group_size(THREADS_MX, THREADS_MX), amdgpu_waves_per_eu(2, 2)))
void gemm_mxfp4_nt_kernel(Problem p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // 0 .. 7; waves w and w + 4 share a SIMD
    const int wm = wave & 1;   // 128-row half of the tile (A rows)
    const int wn = wave >> 1;  // 64-column quarter (B rows)
    const int l16 = lane & 15;
    const int grp = lane >> 4;
    const int K = p.K;
    const unsigned kb = (unsigned)K / 2;       // code bytes per row
    const unsigned sb = (unsigned)K / 32;      // scale bytes per row
    const int nk = (K + BK - 1) / BK;

    const unsigned lds_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)lds;
    const i32x4 ra = rsrc_words(static_cast<const uint8_t *>(p.a) - SHIFT, (unsigned)p.M * kb + SHIFT);
    const i32x4 rb = rsrc_words(static_cast<const uint8_t *>(p.b) - SHIFT, (unsigned)p.N * kb + SHIFT);
    const i32x4 rsa = rsrc_words(static_cast<const uint8_t *>(p.sfa) - SHIFT, (unsigned)p.M * sb + SHIFT);
    const i32x4 rsb = rsrc_words(static_cast<const uint8_t *>(p.sfb) - SHIFT, (unsigned)p.N * sb + SHIFT);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.c, (unsigned)p.M * (unsigned)p.N * 2u);
    const __amdgpu_buffer_rsrc_t rbias = make_rsrc(p.bias, EPI != EPI_PLAIN && p.bias ? (unsigned)p.N * 2u : 0u);

    // Copy map. Code copy t (0, 1) of an operand: tile rows 32 wave + 16 t +
    // lane / 4, lane position lane % 4 of the row, which fetches logical chunk
    // (lane % 4) ^ swizzle; scale copy: waves 0..3 copy A rows, 4..7 B rows,
    // tile row 64 (wave % 4) + lane, its 16 bytes of a block of four steps.
    // Per-lane offsets are set per tile (rows past M or N lie past the buffer
    // and read zeros; a round without a tile reads zeros throughout); the
    // step's K offset is the scalar offset.
    const int copy_row = lane >> 2;
    const int swave = wave & 3;
    const bool scales_of_b = wave >= 4;
    const int srow = 64 * swave + lane;
    const i32x4 rs = scales_of_b ? rsb : rsa;
    int chunk_b[2];   // byte offset (within the step's 64) of each code copy's chunk
#pragma unroll
    for (int t = 0; t < 2; ++t)
        chunk_b[t] = 16 * swizzle(32 * wave + 16 * t + copy_row, lane & 3);

    // Per-lane copy offsets of the current tile (rows past M or N lie past
    // the buffer and read zeros); the step's K offset is the scalar offset,
    // and steps past K (requested ahead of the tile's end) read zeros.
    // Offsets of the current tile and of the workgroup's next one: the last
    // three steps of a tile copy the next tile's first three (K % 512 == 0
    // makes every tile's step count a multiple of the four stages, so they
    // land in the stages the next tile reads them from), and its first scale
    // block. Without a next tile they read zeros.
    unsigned a_off[2], b_off[2], s_off, na_off[2], nb_off[2], ns_off;
    bool has_next = false;
    auto offsets = [&](int tm, int tn, unsigned (&ao)[2], unsigned (&bo)[2], unsigned &so) {
        const int am = tm * TM, bn = tn * TN;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int row = 32 * wave + 16 * t + copy_row;
            ao[t] = (unsigned)(am + row) * kb + (unsigned)chunk_b[t] + SHIFT - 1024u * t;
            bo[t] = (unsigned)(bn + row) * kb + (unsigned)chunk_b[t] + SHIFT - 1024u * t;
        }
        so = (unsigned)((scales_of_b ? bn : am) + srow) * sb + SHIFT;
    };
    // Copy q (0..3) of K step k into stage `stage`: step k of the current
    // tile, or for k >= nk step k - nk of the next; q 0, 1 A codes, 2, 3 B
    // codes, each pair after one m0 write.
    auto copy_one = [&](int k, int stage, int q) {
        const unsigned base = lds_base + (unsigned)(stage * STAGE_BYTES);
        const bool nxt = k >= nk;
        const bool in = !nxt || has_next;
        const int ko = in ? (nxt ? k - nk : k) * ROW_BYTES : 0;
        switch (q) {
        case 0: set_m0(__builtin_amdgcn_readfirstlane(base + A_CODES + 2048 * wave));
                copy_1k<0>(ra, in ? (nxt ? na_off[0] : a_off[0]) : OOB_SHIFTED, ko); break;
        case 1: copy_1k<1024>(ra, in ? (nxt ? na_off[1] : a_off[1]) : OOB_SHIFTED, ko); break;
        case 2: set_m0(__builtin_amdgcn_readfirstlane(base + B_CODES + 2048 * wave));
                copy_1k<0>(rb, in ? (nxt ? nb_off[0] : b_off[0]) : OOB_SHIFTED, ko); break;
        default: copy_1k<1024>(rb, in ? (nxt ? nb_off[1] : b_off[1]) : OOB_SHIFTED, ko); break;
        }
    };
    // Scale block b (steps 4 b .. 4 b + 3; b = nk / 4 is the next tile's
    // block 0) into slot (gb0 + b) % 2, gb0 = blocks of the workgroup's
    // earlier tiles: A rows, then B rows 4 KiB on (K % 512 == 0: every block
    // is whole). One copy per wave.
    int gb0 = 0;
    auto copy_scales = [&](int b) {
        const unsigned base = lds_base + (unsigned)(SCALES_BASE + ((gb0 + b) & 1) * SCALE_BLOCK) +
                              (scales_of_b ? TM * SCALE_BLOCK_ROW : 0) + 1024u * swave;
        const bool nxt = b * SCALE_STEPS >= nk;
        const bool in = !nxt || has_next;
        const int so = in ? (nxt ? b - nk / SCALE_STEPS : b) * SCALE_BLOCK_ROW : 0;
        set_m0(__builtin_amdgcn_readfirstlane(base));
        copy_1k<0>(rs, in ? (nxt ? ns_off : s_off) : OOB_SHIFTED, so);
    };
    auto copy_step = [&](int k, int stage) {
#pragma unroll
        for (int q = 0; q < COPIES; ++q)
            copy_one(k, stage, q);
    };

    // Fragments: 16 bytes per lane (the instruction reads the low four dwords
    // of an eight-dword FP4 operand): row l16 of a 16-row block, the 32 K
    // elements of group grp, i.e. logical chunk grp of the row's 64 bytes.
    // A blocks in a ring of four (block i in fa[i % 4], read three groups of
    // matrix instructions ahead of its use), B blocks in one set per step
    // parity. Scales: byte grp of the row's four for the step, read alone,
    // so the instruction's byte select is 0 and no shift is needed (the
    // counters show about six bank-conflict cycles per scale read, as for a
    // dword read of the row's four; the fragment reads have none). Rows of a
    // lane's blocks differ by multiples of 16, so one chunk offset serves all.
    i32x4 fa[4], fb[2][4];
    unsigned sa[4], sbv[2][4];
    const int a_row0 = 128 * wm + l16, b_row0 = 64 * wn + l16;   // block 0 rows; block i is 16 i rows on
    int kofs = swizzle(l16, grp) << 4;
    int a_frag = A_CODES + a_row0 * ROW_BYTES, b_frag = B_CODES + b_row0 * ROW_BYTES;
    int a_sc = SCALES_BASE + a_row0 * SCALE_BLOCK_ROW + grp, b_sc = SCALES_BASE + TM * SCALE_BLOCK_ROW + b_row0 * SCALE_BLOCK_ROW + grp;
    // scales of K step k: dword k % 4 of the rows' 16 bytes in slot (gb0 + k / 4) % 2
    auto scale_at = [&](int k) { return lds + ((gb0 + (k >> 2)) & 1) * SCALE_BLOCK + (k & 3) * SCALE_ROW; };
    // A block i of K step k (stage `stage`) and its scales
    auto read_a = [&](int stage, int k, int i) {
        fa[i & 3] = *reinterpret_cast<const i32x4 *>(lds + stage * STAGE_BYTES + a_frag + i * 16 * ROW_BYTES + kofs);
        sa[i & 3] = *reinterpret_cast<const uint8_t *>(scale_at(k) + a_sc + 16 * i * SCALE_BLOCK_ROW);
    };
    // B block j of K step k into set `buf`, and its scales
    auto read_b = [&](int stage, int k, int buf, int j) {
        fb[buf][j] = *reinterpret_cast<const i32x4 *>(lds + stage * STAGE_BYTES + b_frag + j * 16 * ROW_BYTES + kofs);
        sbv[buf][j] = *reinterpret_cast<const uint8_t *>(scale_at(k) + b_sc + 16 * j * SCALE_BLOCK_ROW);
    };

    f32x4 acc[8][4];
    // Matrix instruction t (0..31) of a step on B set `buf`: block (t / 4,
    // t % 4), format 4 (E2M1) for both operands. B rows are the first
    // operand, so lane (l16, grp) of block (i, j) holds C[m][n .. n + 3] with
    // m = row l16 of A block i, n = 4 grp + column 16 j (checked on the
    // device: D = first . second^T, lane l holding row l % 16 and K group
    // l / 16, its scale applied to those 32 elements).
    auto mma1 = [&](int buf, int t) {
        const int i = t >> 2, j = t & 3;
        const i32x8 x = __builtin_shufflevector(fb[buf][j], fb[buf][j], 0, 1, 2, 3, -1, -1, -1, -1);
        const i32x8 y = __builtin_shufflevector(fa[i & 3], fa[i & 3], 0, 1, 2, 3, -1, -1, -1, -1);
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, acc[i][j], 4, 4, 0, (int)sbv[buf][j], 0,
                                                                 (int)sa[i & 3]);
    };
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = f32x4{};
    };

    int tm = 0, tn = 0;
    if (schedule_position(blockIdx.x, 0, p.grid) < p.tiles)
        supergroup_tile(schedule_position(blockIdx.x, 0, p.grid), p.tiles_m, p.tiles_n, p.supergroup, tm, tn);
    bool first = true;
    for (int round = 0; schedule_position(blockIdx.x, round, p.grid) < p.tiles; ++round) {
        const int npos = schedule_position(blockIdx.x, round + 1, p.grid);
        has_next = npos < p.tiles;
        int ntm = 0, ntn = 0;
        if (has_next)
            supergroup_tile(npos, p.tiles_m, p.tiles_n, p.supergroup, ntm, ntn);
        offsets(tm, tn, a_off, b_off, s_off);
        offsets(ntm, ntn, na_off, nb_off, ns_off);
        zero_acc();

        if (nk > 0) {
            if (first) {
                // fill the ring with steps 0 .. STAGES - 2 and scale block 0,
                // and wait for all but step 2's copies, so that step 0's
                // wait (written for a tile after another) holds here too
                copy_scales(0);
#pragma unroll
                for (int s = 0; s < STAGES - 1; ++s)
                    copy_step(s, s);
                wait_copies_le<COPIES * (STAGES - 3)>();
                lds_barrier();
#pragma unroll
                for (int i = 0; i < 3; ++i)
                    read_a(0, 0, i);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    read_b(0, 0, 0, j);
            }
            // (otherwise the previous tile's last steps copied steps 0 .. 2
            // and read step 0's first A blocks, its B blocks and their scales)

            // K step k on stage k % STAGES, B set k % 2. The step's shape is
            // fixed at compile time (the first step of a scale block): a
            // branch inside the loop body would let the compiler sink a
            // step's matrix instructions past it, away from the reads and
            // copies they are interleaved with.
            auto step = [&](int k, auto buf_c, auto block_start_c) {
                constexpr int buf = decltype(buf_c)::value;
                constexpr bool block_start = decltype(block_start_c)::value;   // k % 4 == 0
                const int stage = k & (STAGES - 1);
                const int next_stage = (k + 1) & (STAGES - 1);
                const int copy_stage = (k + STAGES - 1) & (STAGES - 1);
                // LDS address bases, hidden from the optimiser at every step so
                // that each stage's addresses are formed where they are used
                asm volatile("" : "+v"(kofs), "+v"(a_frag), "+v"(b_frag), "+v"(a_sc), "+v"(b_sc));
                // this wave's reads of step k - 1 and k and its copies of step
                // k + 1 (and every older scale block) are done. Copies complete
                // in issue order among themselves, so while one of step k + 1's
                // is pending all COPIES of step k + 2 are too: at most COPIES
                // outstanding operations means step k + 1 has landed, whatever
                // else is counted (a scale block copied after step k + 2's
                // codes; at step 0 after a previous tile, that tile's epilogue
                // loads and stores, whose completion order against the copies
                // is not relied on)
                wait_reads();
                wait_copies_le<COPIES * (STAGES - 3)>();
                // after the barrier every wave is done with step k - 1's stage
                // and step k + 1's stage is complete
                lds_barrier();
                // 32 matrix instructions in groups of four sharing an A block,
                // order fixed: group g reads A block g + 3 (blocks 0..2 of step
                // k + 1 in groups 5..7), groups 0..3 step k + 1's B block g;
                // the copies of step k + STAGES - 1 into step k - 1's stage
                // one every four matrix instructions over the first half
                SCHED_FENCE();
                static_for<32>([&](auto tc) {
                    constexpr int t = decltype(tc)::value;
                    constexpr int g = t >> 2;
                    mma1(buf, t);
                    if constexpr (t % 4 == 0) {
                        if constexpr (g < 5)
                            read_a(stage, k, g + 3);
                        else
                            read_a(next_stage, k + 1, g - 5);
                    }
                    if constexpr (t % 4 == 2 && g < 4)
                        read_b(next_stage, k + 1, buf ^ 1, g);
                    if constexpr (t % 4 == 1 && t < 4 * COPIES)
                        copy_one(k + STAGES - 1, copy_stage, t / 4);
                    SCHED_VALU_ONLY();
                });
                // the next scale block during the first step of a block: its
                // slot held block k / 4 - 1, whose steps every wave finished
                // before this step's barrier
                if constexpr (block_start)
                    copy_scales((k >> 2) + 1);
            };
            // nk is a multiple of 4 (K % 512 == 0): steps go in fours
            for (int k = 0; k < nk; k += 4) {
                step(k, Int<0>{}, Int<1>{});
                step(k + 1, Int<1>{}, Int<0>{});
                step(k + 2, Int<0>{}, Int<0>{});
                step(k + 3, Int<1>{}, Int<0>{});
            }
        }
        store_tile16<EPI>(acc, rc, rbias, p.M, p.N, tm * TM + 128 * wm, tn * TN + 64 * wn, lane);
        gb0 += nk / SCALE_STEPS;
        tm = ntm;
        tn = ntn;
        first = false;
    }
    wait_reads();
    wait_all_copies(); // no copy may still be writing LDS when the workgroup ends
}

} // namespace mx
} // namespace gemm355
