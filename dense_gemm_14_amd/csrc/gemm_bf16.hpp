// gemm_bf16.hpp -- persistent BF16 NT GEMM for gfx950: v_mfma_f32_16x16x32_bf16
// on operands copied straight from global memory into a ring of LDS slots.
//
// Work decomposition
//   * Output tile 256 x 256 per workgroup, 4 waves in a 2 x 2 layout; each
//     wave owns a 128 x 128 block = 8 x 8 blocks of 16 x 16 whose FP32
//     accumulators (256 per lane) stay in the accumulation registers for the
//     whole K loop. The 16 x 16 x 32 instruction moves half the accumulator
//     data per multiply-add of the 32 x 32 x 16 one, which lowers the energy
//     per product and so the clock throttling under the board power limit.
//   * K advances 64 per step. A step is 64 block pairs (the first 32 walk
//     rows 0..3 column by column, the last 32 rows 4..7): each pair is the
//     block's two matrix instructions, K 0..31 and then K 32..63 of the step,
//     back to back on the same accumulators. An instruction whose accumulator input is the
//     result of the one just before it takes that result from the matrix
//     core instead of the register file: on MI355X a loop of such pairs held
//     a 5 % higher clock under the board power limit than the same
//     instructions with every accumulator touched once per K = 32 (2.14
//     against 2.04 GHz with random BF16 data; 696 against 776 W with zeros
//     at full clock), and power is what bounds this kernel. The summation
//     order per element is the same either way.
//   * Fragments (8 A blocks and 8 B blocks of 16 rows, both K halves: 16
//     bytes per lane and half each) live in one register set; a block's
//     fragment of the next step is read into its registers once the block's
//     last pair of this step has issued, at least eight pairs before its
//     first use there. B block j (0..6) of step s + 1 is read after pair
//     36 + 4 j of step s (its last use in step s is pair 35 + 4 j), A blocks
//     0..3 after pairs 34..46; A blocks 4..7 and B block 7 of a step are read
//     in the step itself, before its barrier. The 32 reads spread evenly over
//     the step.
//   * LDS is a ring of five 32 KiB slots; a slot holds one unit, the A tile
//     (256 rows x 64 K) or the B tile of one step, as 256 rows of 128 bytes.
//     Unit 2 s + op (op 0 = A, 1 = B) lives in slot (2 s + op) mod 5. Each 1
//     KiB block of a unit is written by one copy instruction of the memory
//     pipeline (lane i fills bytes 16 i .. 16 i + 15 of the block: 8 rows x
//     128 bytes), so operands pass through no registers and no LDS-write
//     instructions, and every request is one whole 128-byte row segment.
//   * One barrier per step, after pair 31. Before it each wave has finished
//     reading step s (its last reads, A block 7, follow pair 26), so both of
//     its slots are free, and its copies of step s + 1 have landed; step
//     s + 1 is read from pair 34 on. The barrier opens a copy window that
//     runs until the next barrier: the B tile of step s + 2 (into the slot of
//     A_s, needed one step later) and the A tile of step s + 3 (into the slot
//     of B_s, needed two steps later). Five slots give every copy at least a
//     whole step, and half of them two steps, between issue and first use.
//   * LDS rows are 128 bytes (eight 16-byte chunks); logical chunk c of row r
//     sits at chunk position c ^ ((r >> 1) & 7). A fragment read serves 16
//     lanes (256 bytes over the 64 four-byte banks) per cycle; those lanes
//     read 16 consecutive rows at one logical chunk, row parity picks the
//     128-byte half of the bank space and (r >> 1) & 7 the chunk within it,
//     so the 16 lanes hit 16 distinct bank groups. The swizzle is applied on
//     the global side: the lane that fills position p of row r fetches
//     logical chunk p ^ ((r >> 1) & 7).
#pragma once

#include "common.hpp"

#include <utility>

namespace gemm355 {
namespace bf16 {

constexpr int BK = 64;                       // K elements per step
constexpr int ROW_BYTES = BK * 2;            // 128-byte LDS rows
constexpr int UNIT_BYTES = BM * ROW_BYTES;   // one operand tile of one step: 32 KiB
constexpr int SLOTS = 5;
constexpr int LDS_BYTES = SLOTS * UNIT_BYTES;
constexpr int UNIT_COPIES = 8;               // 1 KiB copies per wave per unit (64 rows)
constexpr int EPILOGUE_STORES = 32;          // 16-byte stores per wave per tile

static_assert(LDS_BYTES <= 163840, "LDS ring exceeds the 160 KiB of a gfx950 workgroup");
static_assert(BM == 256 && BN == 256 && THREADS == 256, "the copy map assumes 256 x 256 tiles and 4 waves");
// Most vector memory operations a wave has in flight: after a tile change
// the 32 epilogue stores and the copies of A2, B2 and A3 of the new tile.
static_assert(3 * UNIT_COPIES + EPILOGUE_STORES <= 63, "vmcnt counts at most 63 outstanding operations");

// Block pairs of a step (0..63; the barrier follows pair 31): the first
// half walks rows 0..3 column by column, the second rows 4..7, so B block j
// is used at pairs 4 j .. 4 j + 3 and 32 + 4 j .. 32 + 4 j + 3, A blocks 0..3
// only before the barrier and A blocks 4..7 only after it.
constexpr int pair_row(int p) { return (p < 32 ? 0 : 4) + (p & 3); }
constexpr int pair_col(int p) { return (p & 31) >> 2; }
// Fragment reads, each into registers whose last use is behind it and at
// least eight pairs before its first use: A block i (4..7) and B block 7 of
// the step itself after pairs a_read_at(i) and B7_READ (before the barrier);
// A block i (0..3) and B block j (0..6) of the next step after pairs
// a_read_at(i) and b_read_at(j) (after the barrier, once their copies are
// visible to every wave).
constexpr int a_read_at(int i) { return i < 4 ? 34 + 4 * i : 8 + 6 * (i - 4); }
constexpr int b_read_at(int j) { return 36 + 4 * j; }
constexpr int B7_READ = 2;
// The copies of a unit go out in four pairs (blocks 2 q and 2 q + 1 of the
// wave's eight), one copy pair every eight block pairs, A before the barrier
// and B after it, each inside a block pair: one copy after each of its two
// matrix instructions, so that the first issues in the shadow of the first
// instruction, whose result the second waits for anyway (1.2 % faster at
// 8192^3 and 1.5 % at 8000^3 than both copies after the pair, same box,
// alternating; one copy per block pair, every two, three or four pairs,
// measured in between).
// In a tile's last two steps, which copy the next tile's first two, the B
// copies come every two pairs, so that they have landed when the epilogue
// waits for every copy.
constexpr int a_copy_at(int q) { return 8 * q + 2; }
constexpr int b_copy_at(int q, bool last = false) { return 32 + (last ? 2 : 8) * q; }

// Buffer resources for the copies start SHIFT bytes before their operand (and
// span SHIFT bytes more): block j of a pair is addressed with instruction
// offset 1024 (j % 4), which moves the LDS destination and the global address
// alike, and the per-lane offset (global offset + SHIFT - 1024 (j % 4)) stays
// non-negative. OOB_OFF is beyond every range even after the scalar step
// offset and the instruction offset are added (operand extents are < 2^31).
constexpr int SHIFT = 3072;
constexpr int OOB_OFF = (int)0x80000000;

__device__ inline int swizzle(int r, int c) { return c ^ ((r >> 1) & 7); }

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource as four scalar words, for the inline-assembly copies.
__device__ inline i32x4 rsrc_words(const void *p, unsigned bytes)
{
    const unsigned long long a = reinterpret_cast<unsigned long long>(p);
    return i32x4{(int)(unsigned)a, (int)(unsigned)(a >> 32), (int)bytes, (int)RSRC_WORD3};
}

// Two 1 KiB global -> LDS copies: lane i's 16 bytes at byte base + v + O
// land at LDS byte lds_addr + O + 16 i (v = v0, O = O0 and v = v1, O = O1),
// base being the operand's address less SHIFT plus the step's K offset (the
// global form of the LDS-DMA load, 1.4 % faster at 8192^3 than the buffer
// form, same box, alternating runs; it has no range check, so every address
// it gets lies inside the operand). Written as inline assembly so the compiler does not treat the
// in-flight LDS writes as aliasing every later LDS read (it would wait for all
// copies before each read); the kernel orders the copies itself with explicit
// vmcnt waits and barriers. m0 holds the LDS base; nothing else in this kernel
// uses m0. On gfx9 an LDS-DMA instruction must not directly follow a scalar
// write of m0 (one wait state), hence the s_nop.
template <int O0, int O1>
__device__ inline void copy_pair(unsigned long long base, unsigned lds_addr, int v0, int v1)
{
    static_assert(O0 >= 0 && O1 >= 0 && O0 <= SHIFT && O1 <= SHIFT, "instruction offsets must stay within SHIFT");
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, %3 offset:%4\n\t"
                 "global_load_lds_dwordx4 %2, %3 offset:%5"
                 :
                 : "s"(lds_addr), "v"(v0), "v"(v1), "s"(base), "n"(O0), "n"(O1)
                 : "memory", "m0");
}

// The same two copies in the buffer form, for the step that copies the K
// tail: lane offsets v0, v1 plus the scalar offset soff within the buffer
// resource; an offset of OOB_OFF lies past the range and reads zeros.
template <int O0, int O1>
__device__ inline void copy_pair_buffer(const i32x4 &rsrc, unsigned lds_addr, int v0, int v1, int soff)
{
    static_assert(O0 >= 0 && O1 >= 0 && O0 <= SHIFT && O1 <= SHIFT, "instruction offsets must stay within SHIFT");
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %1, %3, %4 offen offset:%5 lds\n\t"
                 "buffer_load_dwordx4 %2, %3, %4 offen offset:%6 lds"
                 :
                 : "s"(lds_addr), "v"(v0), "v"(v1), "s"(rsrc), "s"(soff), "n"(O0), "n"(O1)
                 : "memory", "m0");
}

// Single copies for the main loop, which issues each copy inside a block
// pair: m0 is set before the pair's first matrix instruction (which supplies
// the wait state), one copy follows each of its two instructions.
__device__ inline void set_m0(unsigned lds_addr) { asm volatile("s_mov_b32 m0, %0" ::"s"(lds_addr) : "m0"); }
template <int O>
__device__ inline void copy_one(unsigned long long base, int v)
{
    static_assert(O >= 0 && O <= SHIFT, "instruction offsets must stay within SHIFT");
    asm volatile("global_load_lds_dwordx4 %0, %1 offset:%2" ::"v"(v), "s"(base), "n"(O) : "memory");
}
template <int O>
__device__ inline void copy_one_buffer(const i32x4 &rsrc, int v, int soff)
{
    static_assert(O >= 0 && O <= SHIFT, "instruction offsets must stay within SHIFT");
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:%3 lds" ::"v"(v), "s"(rsrc), "s"(soff), "n"(O) : "memory");
}

// Every copy this wave issued has landed in LDS (stores too).
__device__ inline void wait_all_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// At most N copies of this wave are still in flight (they complete in order).
template <int N>
__device__ inline void wait_copies_le() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
// Every LDS read this wave issued has returned.
__device__ inline void wait_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }


// Lane index recomputed where it is used (volatile, so it is not hoisted
// into a register that would have to live through the whole tile loop).
__device__ inline int fresh_lane_id()
{
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// EPI: EPI_PLAIN, or the activation of the fused epilogue (bias, then the
// activation, before rounding). KTAIL: K is not a multiple of 64; every copy
// then goes through the buffer form, whose range check zero-fills the chunks
// of the last K step that lie at or past K.
template <int EPI, bool KTAIL>
__global__ __attribute__((amdgpu_flat_work_group_size(THREADS, THREADS), amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_nt_kernel(Problem p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
    constexpr bool FUSED = EPI != EPI_PLAIN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1;   // wave's 128-row half of the tile (A rows)
    const int wn = wave >> 1;  // wave's 128-column half (B rows)
    const int l16 = lane & 15;
    const int grp = lane >> 4;
    const int K = p.K;

    // Fragment of a 16-row block: lane (l16, grp) reads row l16 of the block,
    // logical chunk grp (K 0..31 of the step) or 4 + grp (K 32..63).
    // Blocks start at multiples of 16 rows, which leaves the swizzle unchanged.
    const int kofs0 = swizzle(l16, grp) << 4;
    const int kofs1 = swizzle(l16, 4 + grp) << 4;
    const int a_frag = (wm * 128 + l16) * ROW_BYTES;
    const int b_frag = (wn * 128 + l16) * ROW_BYTES;
    const int copy_row = lane >> 3;

    const unsigned lds_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)lds;
    const i32x4 ra = rsrc_words(static_cast<const uint8_t *>(p.a) - SHIFT, (unsigned)p.M * (unsigned)K * 2u + SHIFT);
    const i32x4 rb = rsrc_words(static_cast<const uint8_t *>(p.b) - SHIFT, (unsigned)p.N * (unsigned)K * 2u + SHIFT);
    const unsigned long long ga = reinterpret_cast<unsigned long long>(p.a) - SHIFT;
    const unsigned long long gb = reinterpret_cast<unsigned long long>(p.b) - SHIFT;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.c, (unsigned)p.M * (unsigned)p.N * 2u);
    const int nk = (K + BK - 1) / BK;   // >= 4: smaller K goes to the 64 x 64 instance

    int round = 0;
    int tm, tn;
    {
        const int pos = schedule_position(blockIdx.x, 0, p.grid);
        if (pos >= p.tiles)
            return;
        supergroup_tile(pos, p.tiles_m, p.tiles_n, p.supergroup, tm, tn);
    }

    f32x4 acc[8][8];
    // Fused epilogue: bias[n .. n + 3] (two BF16 pairs) for this lane's
    // columns n of block column 2 jp + h of tile column ctn; zeros past N and
    // without a bias (an empty range).
    const __amdgpu_buffer_rsrc_t rbias = make_rsrc(p.bias, FUSED && p.bias ? (unsigned)p.N * 2u : 0u);
    auto load_bias = [&](int ctn, int jp, int h, int ln) {
        const int n = ctn * BN + wn * 128 + 16 * (2 * jp + h) + 4 * (ln >> 4);
        return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rbias, n < p.N ? n * 2 : OOB, 0, 0));
    };
    // Epilogue of one pair of blocks. Lane (l16, grp) of block (i, j) holds
    // C[m][n .. n + 3] with m = m0 + 16 i + l16 and n = n0 + 16 j + 4 grp. For
    // x = block (i, 2 jp) and y = block (i, 2 jp + 1), v_permlane16_swap
    // exchanges lane groups so that group 0 holds columns 0..7 of x, group 1
    // columns 0..7 of y, group 2 columns 8..15 of x and group 3 columns 8..15
    // of y: one 16-byte store per lane, 64 contiguous bytes per C row.
    auto store_pair = [&](int ctm, int ctn, int i, int jp, int ln, u32x2 bx, u32x2 by) {
        const int l16 = ln & 15, grp = ln >> 4;
        f32x4 x = acc[i][2 * jp];
        f32x4 y = acc[i][2 * jp + 1];
        if constexpr (FUSED) {
            x = epilogue4<EPI>(x, bx);
            y = epilogue4<EPI>(y, by);
        }
        const unsigned x0 = pack_bf16(x[0], x[1]), x1 = pack_bf16(x[2], x[3]);
        const unsigned y0 = pack_bf16(y[0], y[1]), y1 = pack_bf16(y[2], y[3]);
        const auto s0 = __builtin_amdgcn_permlane16_swap(x0, y0, false, false);
        const auto s1 = __builtin_amdgcn_permlane16_swap(x1, y1, false, false);
        const u32x4 out = {s0[0], s1[0], s0[1], s1[1]};
        const int mm = ctm * BM + wm * 128 + l16 + 16 * i;
        const int n = ctn * BN + wn * 128 + 16 * (grp & 1) + 8 * (grp >> 1) + 32 * jp;
        const int off = (mm < p.M && n < p.N) ? (mm * p.N + n) * 2 : OOB;
        __builtin_amdgcn_raw_buffer_store_b128(out, rc, off, 0, 0);
    };

    // The workgroup's tiles run as one continuous sequence of steps: the ring,
    // the copy windows and the fragment reads carry on across tile
    // boundaries, so the copies of a tile's first units and the fragments of
    // its first row are fetched during the previous tile's last steps. Every
    // step runs the same code: what differs (the K step the copies fetch,
    // the tile whose rows they read, the wait of a tile's first step) is
    // uniform arithmetic or a uniform branch around it, so the accumulators
    // are carried by one loop and every step uses the same registers.

    // Copies: wave w fills blocks 8 w .. 8 w + 7 (rows 64 w .. 64 w + 63) of
    // every unit; copy j of the wave fills block 8 w + j, lane i position
    // i & 7 of its row i / 8. voff[op][j]: this lane's offset for copy j of
    // operand op (0 = A, 1 = B) at K step 0 of the tile the copies read, in
    // the shifted buffer and less the instruction offset 1024 (j % 4); a step
    // adds 128 bytes per K step through the step's base. Two steps before a
    // tile ends they are recomputed for the next tile, whose first two steps
    // the tile's last two steps copy (for the same tile after the last one,
    // so the copies a last tile issues for its successor read valid rows and
    // are never used). Rows past M or N are clamped to the last row: the
    // copies read valid memory, and those rows only feed outputs the epilogue
    // does not store.
    int voff[2][UNIT_COPIES];
    bool tail_ok[2];   // per block parity: this lane's chunk of step nk - 1 lies below K
    auto offsets = [&](int t_m, int t_n, int (&o)[2][UNIT_COPIES]) {
        const int ln = fresh_lane_id();
#pragma unroll
        for (int j = 0; j < UNIT_COPIES; ++j) {
            const int row = 8 * (UNIT_COPIES * wave + j) + (ln >> 3);
            const int c = swizzle(row, ln & 7);   // logical chunk stored at position ln & 7
            const int am = min(t_m * BM + row, p.M - 1), bn = min(t_n * BN + row, p.N - 1);
            o[0][j] = (am * K + 8 * c) * 2 + SHIFT - 1024 * (j & 3);
            o[1][j] = (bn * K + 8 * c) * 2 + SHIFT - 1024 * (j & 3);
        }
    };
    offsets(tm, tn, voff);
#pragma unroll
    for (int j = 0; j < 2; ++j)
        tail_ok[j] = (nk - 1) * BK + 8 * swizzle(8 * (UNIT_COPIES * wave + j) + copy_row, lane & 7) < K;
    bool has_next = false;
    int ntm = 0, ntn = 0;
    auto find_next = [&]() {
        const int pos = schedule_position(blockIdx.x, round + 1, p.grid);
        has_next = pos < p.tiles;
        if (has_next)
            supergroup_tile(pos, p.tiles_m, p.tiles_n, p.supergroup, ntm, ntn);
    };
    find_next();

    // Per-step bases, hidden from the optimiser again at every step so that
    // addresses are formed where they are used instead of being hoisted out
    // of the loop into registers (which would spill).
    unsigned copy_base[2] = {lds_base + (unsigned)(UNIT_COPIES * wave * 1024),
                             lds_base + (unsigned)(UNIT_COPIES * wave * 1024 + 4096)};
    int a_ofs[2] = {a_frag + kofs0, a_frag + kofs1};
    int b_ofs[2] = {b_frag + kofs0, b_frag + kofs1};

    // ring[x]: LDS offset of the slot of unit 2 s + x during step s (x =
    // 0..4). The next step sees the same slots rotated by two units, so the
    // offsets are carried in scalar registers and renamed, never computed.
    int ring[SLOTS];
#pragma unroll
    for (int x = 0; x < SLOTS; ++x)
        ring[x] = x * UNIT_BYTES;
    auto rotate = [&]() {
        const int r0 = ring[0], r1 = ring[1];
        ring[0] = ring[2];
        ring[1] = ring[3];
        ring[2] = ring[4];
        ring[3] = r0;
        ring[4] = r1;
    };
    // Pair q of operand op's unit at K step ks_off / 128 into slot `slot`.
    // With a K tail (KTAIL), every copy goes through the buffer form, and in
    // the step that copies K step nk - 1 (tail) the chunks at or past K read
    // as zeros (the buffer's range check turns OOB_OFF into zeros).
    auto copies = [&](int op, auto q_c, int slot, int ks_off, bool tail) {
        constexpr int q = decltype(q_c)::value;
        constexpr int j0 = 2 * q, j1 = 2 * q + 1;
        int v0 = voff[op][j0];
        int v1 = voff[op][j1];
        if constexpr (KTAIL) {
            v0 = tail && !tail_ok[0] ? OOB_OFF : v0;
            v1 = tail && !tail_ok[1] ? OOB_OFF : v1;
            copy_pair_buffer<1024 * (j0 & 3), 1024 * (j1 & 3)>(op ? rb : ra, copy_base[q >> 1] + (unsigned)slot, v0,
                                                                v1, ks_off);
        } else {
            copy_pair<1024 * (j0 & 3), 1024 * (j1 & 3)>((op ? gb : ga) + (unsigned)ks_off,
                                                         copy_base[q >> 1] + (unsigned)slot, v0, v1);
        }
    };

    bf16x8 fa[2][8], fb[2][8];
    // Both K halves of A block i / B block j of the step whose unit sits in
    // slot `slot`.
    auto read_a = [&](int slot, int i) {
        fa[0][i] = *reinterpret_cast<const bf16x8 *>(lds + (a_ofs[0] + slot) + i * 16 * ROW_BYTES);
        SCHED_FENCE();
        fa[1][i] = *reinterpret_cast<const bf16x8 *>(lds + (a_ofs[1] + slot) + i * 16 * ROW_BYTES);
    };
    auto read_b = [&](int slot, int j) {
        fb[0][j] = *reinterpret_cast<const bf16x8 *>(lds + (b_ofs[0] + slot) + j * 16 * ROW_BYTES);
        SCHED_FENCE();
        fb[1][j] = *reinterpret_cast<const bf16x8 *>(lds + (b_ofs[1] + slot) + j * 16 * ROW_BYTES);
    };
    // Block pair p: block (pair_row(p), pair_col(p)), K 0..31 then K 32..63 of the step,
    // nothing scheduled between the two. B rows are the first operand and A
    // rows the second, so each 16 x 16 result arrives transposed (one C row
    // per lane, four adjacent columns). The empty statement takes the second
    // half's fragments as inputs, so the compiler's wait for them (the later
    // of each pair of reads) comes before the pair and none between its two
    // instructions.
    auto mma2 = [&](int p) {
        const int i = pair_row(p), j = pair_col(p);
        asm volatile("" ::"v"(fb[1][j]), "v"(fa[1][i]));
        SCHED_FENCE();
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[0][j], fa[0][i], acc[i][j], 0, 0, 0);
        SCHED_FENCE();
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[1][j], fa[1][i], acc[i][j], 0, 0, 0);
        SCHED_FENCE();
    };

    // Block pair p with copy pair q of operand op's unit at K step ks_off /
    // 128 into slot `slot` issued inside it (copies() is the same pair on its
    // own).
    auto mma2_copies = [&](int p, int op, auto q_c, int slot, int ks_off, bool tail) {
        constexpr int q = decltype(q_c)::value;
        constexpr int j0 = 2 * q, j1 = 2 * q + 1;
        constexpr int O0 = 1024 * (j0 & 3), O1 = 1024 * (j1 & 3);
        int v0 = voff[op][j0];
        int v1 = voff[op][j1];
        if constexpr (KTAIL) {
            v0 = tail && !tail_ok[0] ? OOB_OFF : v0;
            v1 = tail && !tail_ok[1] ? OOB_OFF : v1;
        }
        const unsigned long long base = (op ? gb : ga) + (unsigned)ks_off;
        const int i = pair_row(p), j = pair_col(p);
        asm volatile("" ::"v"(fb[1][j]), "v"(fa[1][i]));
        set_m0(copy_base[q >> 1] + (unsigned)slot);
        SCHED_FENCE();
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[0][j], fa[0][i], acc[i][j], 0, 0, 0);
        SCHED_FENCE();
        if constexpr (KTAIL)
            copy_one_buffer<O0>(op ? rb : ra, v0, ks_off);
        else
            copy_one<O0>(base, v0);
        SCHED_FENCE();
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[1][j], fa[1][i], acc[i][j], 0, 0, 0);
        SCHED_FENCE();
        if constexpr (KTAIL)
            copy_one_buffer<O1>(op ? rb : ra, v1, ks_off);
        else
            copy_one<O1>(base, v1);
        SCHED_FENCE();
    };

    // Prologue of the workgroup's first tile: units A0, B0, A1, B1 (A2 comes
    // with the first step's copies, as for every later tile), all landed
    // before the first barrier, then the fragments of step 0 that the
    // previous tile's last step reads for every later tile: A blocks 0..3 and
    // B blocks 0..6.
#pragma unroll
    for (int u = 0; u < SLOTS - 1; ++u)
        static_for<UNIT_COPIES / 2>([&](auto q) { copies(u & 1, q, u * UNIT_BYTES, (u >> 1) * ROW_BYTES, false); });
    wait_all_copies();
    lds_barrier();
    // (in the order a step issues them, which the compiler's waits for them
    // at the top of the loop assume)
#pragma unroll
    for (int j = 0; j < 7; ++j) {
        if (j < 4) {
            read_a(ring[0], j);
            SCHED_FENCE();
        }
        read_b(ring[1], j);
        SCHED_FENCE();
    }

    // Step s of the current tile. Its copies fetch K step s + 2 (steps 0 and
    // 1 of the next tile in the last two steps): the A tile before the
    // barrier into the slot of B_{s-1} (freed by the previous barrier), the B
    // tile after it into the slot of A_s. The barrier follows this wave's
    // last read of step s and the landing of its copies of step s + 1 (a
    // tile's first step waits for none: the epilogue before it waited for
    // all). Only the copies' order among themselves is relied on, never their
    // order relative to stores. The
    // order of matrix instructions, LDS reads, copies and scalar
    // instructions inside a step is fixed by hand (a scheduling barrier after
    // every block pair and what follows it); only plain vector ALU work may
    // move across those barriers, so its dependency chains spread over
    // several matrix instructions instead of stalling the issue of the next
    // one. Fragment reads are waited for by the compiler's own counter waits,
    // just before the pair that uses them, so the B reads issued at the end
    // of a step overlap the next step's first row.
    auto step = [&](int s, auto first_c, auto last_c) {
        constexpr bool first = decltype(first_c)::value;
        constexpr bool last = decltype(last_c)::value;
        asm volatile("" : "+v"(a_ofs[0]), "+v"(a_ofs[1]), "+v"(b_ofs[0]), "+v"(b_ofs[1]), "+s"(copy_base[0]), "+s"(copy_base[1]));
        const int ks = s + 2 < nk ? s + 2 : s + 2 - nk;   // K step the copies fetch
        const int ks_off = ks * ROW_BYTES;
        const bool tail = KTAIL && ks == nk - 1;
        // pairs 0..31: step s's A blocks 4..7 and B block 7; the A copies
        static_for<32>([&](auto pc) {
            constexpr int p = decltype(pc)::value;
            constexpr int a_step = a_copy_at(1) - a_copy_at(0);
            if constexpr (p >= a_copy_at(0) && (p - a_copy_at(0)) % a_step == 0 && p <= a_copy_at(UNIT_COPIES / 2 - 1))
                mma2_copies(p, 0, Int<(p - a_copy_at(0)) / a_step>{}, ring[4], ks_off, tail);
            else
                mma2(p);
            if constexpr (p == B7_READ)
                read_b(ring[1], 7);
#pragma unroll
            for (int i = 4; i < 8; ++i)
                if (p == a_read_at(i))
                    read_a(ring[0], i);
            SCHED_VALU_ONLY();
        });
        wait_reads();
        if constexpr (!first)
            wait_copies_le<UNIT_COPIES>();
        lds_barrier();
        SCHED_FENCE();
        // pairs 32..63: step s + 1's A blocks 0..3 and B blocks 0..6 (the
        // next tile's first step after a tile's last); the B copies
        static_for<32>([&](auto pc) {
            constexpr int p = 32 + decltype(pc)::value;
            constexpr int b0 = b_copy_at(0, last), b_step = b_copy_at(1, last) - b0;
            if constexpr (p >= b0 && (p - b0) % b_step == 0 && p <= b_copy_at(UNIT_COPIES / 2 - 1, last))
                mma2_copies(p, 1, Int<(p - b0) / b_step>{}, ring[0], ks_off, tail);
            else
                mma2(p);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (p == a_read_at(i))
                    read_a(ring[2], i);
#pragma unroll
            for (int j = 0; j < 7; ++j)
                if (p == b_read_at(j))
                    read_b(ring[3], j);
            SCHED_VALU_ONLY();
        });
        SCHED_FENCE();
        rotate();
    };

    for (;;) {
        // Accumulators start from zero, written into them (one zero per
        // block that the compiler cannot see through, so that no instruction
        // of the first step takes an immediate or shared zero instead): every
        // pair runs in place on its block's registers.
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float zero;
                asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
                acc[i][j] = f32x4{zero, zero, zero, zero};
            }
        // the first step (it waits for no copies), then two loops over the
        // same step (in the second the B copies come early): between them the
        // copy offsets
        // move to the next tile's rows (a branch for it inside the loop makes
        // the compiler treat the slot offsets as divergent)
        step(0, Int<1>{}, Int<0>{});
        for (int s = 1; s < nk - 2; ++s)
            step(s, Int<0>{}, Int<0>{});
        offsets(has_next ? ntm : tm, has_next ? ntn : tn, voff);
#pragma clang loop unroll(disable)
        for (int s = nk - 2; s < nk; ++s)
            step(s, Int<0>{}, Int<1>{});
        // epilogue: the next tile's first two steps have landed (waited for
        // here, before the first store, so that the next tile's first step
        // needs no wait: the counter may see copies and stores complete out of
        // order, and later waits rely only on copies completing in order among
        // themselves), its first fragments are read
        wait_all_copies();
        const int ln = fresh_lane_id();
        if constexpr (FUSED) {
            // by block-column pairs, the bias of the next pair requested
            // while the current one is stored
            u32x2 bx = load_bias(tn, 0, 0, ln), by = load_bias(tn, 0, 1, ln);
#pragma unroll
            for (int jp = 0; jp < 4; ++jp) {
                u32x2 nbx = {}, nby = {};
                if (jp < 3) {
                    nbx = load_bias(tn, jp + 1, 0, ln);
                    nby = load_bias(tn, jp + 1, 1, ln);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    store_pair(tm, tn, i, jp, ln, bx, by);
                bx = nbx;
                by = nby;
            }
        } else {
#pragma unroll
            for (int jp = 0; jp < 4; ++jp)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    store_pair(tm, tn, i, jp, ln, u32x2{}, u32x2{});
        }
        if (!has_next)
            break;
        // switch to the next tile
        tm = ntm;
        tn = ntn;
        ++round;
        find_next();
    }

    wait_reads();
    wait_all_copies(); // no copy may still be writing LDS when the workgroup ends
}

} // namespace bf16
} // namespace gemm355
