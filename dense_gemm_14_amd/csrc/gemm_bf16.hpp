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
//   * K advances 64 per step. A step is split into two half-steps of K = 32;
//     a half-step is 64 matrix instructions on one set of fragments (8 A
//     blocks, 8 B blocks, 16 bytes per lane each) while the other set is
//     read from LDS.
//   * LDS is a ring of five 32 KiB slots; a slot holds one unit, the A tile
//     (256 rows x 64 K) or the B tile of one step, as 256 rows of 128 bytes.
//     Unit 2 s + op (op 0 = A, 1 = B) lives in slot (2 s + op) mod 5. Each 1
//     KiB block of a unit is written by one copy instruction of the memory
//     pipeline (lane i fills bytes 16 i .. 16 i + 15 of the block: 8 rows x
//     128 bytes), so operands pass through no registers and no LDS-write
//     instructions, and every request is one whole 128-byte row segment.
//   * One barrier per step, between its two half-steps. Before it each wave
//     has finished reading step s (so both of its slots are free) and its
//     copies of step s + 1 have landed. The barrier opens a copy window that
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

// Instruction positions inside a half-step of 64 matrix instructions.
// Fragment read r (0..15) follows matrix instruction read_at(r): all reads are
// issued in the first three quarters so they have landed by the half-step's end.
constexpr int read_at(int r) { return 3 * r + 1; }
// The copies of a unit go out in four pairs (blocks 2 p and 2 p + 1 of the
// wave's eight), one pair every sixteen matrix instructions: A pairs in the
// first half-step, B pairs in the second. In the last step of a tile the B
// pairs (the next tile's B1) come one every four matrix instructions, so that
// they have landed by the epilogue, which waits for every copy.
constexpr int a_pair_at(int p) { return 16 * p + 4; }
constexpr int b_pair_at(int p, bool last) { return last ? 4 * p + 1 : 16 * p + 1; }
// Fragment read order: A0, B0..B7, A1..A7, so the first matrix instructions of
// a half-step (A block 0 against every B block) wait for two reads only.
constexpr int read_block(int r) { return r == 0 ? 0 : r <= 8 ? 8 + (r - 1) : r - 8; }

// Buffer resources for the copies start SHIFT bytes before their operand (and
// span SHIFT bytes more): block j of a pair is addressed with instruction
// offset 1024 (j % 4), which moves the LDS destination and the global address
// alike, and the per-lane offset (global offset + SHIFT - 1024 (j % 4)) stays
// non-negative. OOB_OFF is beyond every range even after the scalar step
// offset and the instruction offset are added (operand extents are < 2^31).
constexpr int SHIFT = 3072;
constexpr int OOB_OFF = (int)0x80000000;

// Step kinds of a tile (at least four steps; smaller K goes to the 64 x 64
// instance): FIRST (step 0, matrix instructions start from zero), MID (1 ..
// nk - 4), TAIL (nk - 3: copies step nk - 1, the only one with a K tail),
// NEXT0 and NEXT1 (nk - 2, nk - 1: copy the next tile's steps 0 and 1).
enum StepKind : int { FIRST, MID, TAIL, NEXT0, NEXT1 };

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

// Every copy this wave issued has landed in LDS (stores too).
__device__ inline void wait_all_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// At most N copies of this wave are still in flight (they complete in order).
template <int N>
__device__ inline void wait_copies_le() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
// Every LDS read this wave issued has returned.
__device__ inline void wait_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// The same as an instruction the compiler knows about, so that it drops its
// own waits for the fragments read before it.
__device__ inline void wait_reads_known() { __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4)); }


// Lane index recomputed where it is used (volatile, so it is not hoisted
// into a register that would have to live through the whole tile loop).
__device__ inline int fresh_lane_id()
{
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// EPI: EPI_PLAIN, or the activation of the fused epilogue (bias, then the
// activation, before rounding).
template <int EPI>
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
    // logical chunk grp (first half-step) or 4 + grp (second half-step).
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
    // boundaries, so the copies of a tile's first units are issued during the
    // previous tile's last steps, and the previous tile's accumulators are
    // converted and stored while the first half-step of the next tile
    // overwrites them block by block (its matrix instructions start from 0).

    // Copies: wave w fills blocks 8 w .. 8 w + 7 (rows 64 w .. 64 w + 63) of
    // every unit; copy j of the wave fills block 8 w + j, lane i position
    // i & 7 of its row i / 8. voff[op][j]: this lane's offset for copy j of
    // operand op (0 = A, 1 = B) at step 0 of the current tile, in the shifted
    // buffer and less the instruction offset 1024 (j % 4); a step adds 128
    // bytes per K step through the step's base. nvoff: the same for the
    // next tile (equal to voff after the last tile, so the copies a last tile
    // issues for its successor read valid rows and are never used). Rows past
    // M or N are clamped to the last row: the copies read valid memory, and
    // those rows only feed outputs the epilogue does not store.
    int voff[2][UNIT_COPIES], nvoff[2][UNIT_COPIES];
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
        offsets(has_next ? ntm : tm, has_next ? ntn : tn, nvoff);
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
    // Pair p of operand op's unit at K step ks_off / 128 into slot `slot`;
    // NEXT: the next tile's rows; TAIL: chunks at or past K read as zeros
    // (through the buffer form, whose range check turns OOB_OFF into zeros).
    auto copies = [&](int op, auto p_c, int slot, int ks_off, bool next, bool tail) {
        constexpr int p = decltype(p_c)::value;
        constexpr int j0 = 2 * p, j1 = 2 * p + 1;
        int v0 = next ? nvoff[op][j0] : voff[op][j0];
        int v1 = next ? nvoff[op][j1] : voff[op][j1];
        if (tail) {
            v0 = tail_ok[0] ? v0 : OOB_OFF;
            v1 = tail_ok[1] ? v1 : OOB_OFF;
            copy_pair_buffer<1024 * (j0 & 3), 1024 * (j1 & 3)>(op ? rb : ra, copy_base[p >> 1] + (unsigned)slot, v0,
                                                                v1, ks_off);
        } else {
            copy_pair<1024 * (j0 & 3), 1024 * (j1 & 3)>((op ? gb : ga) + (unsigned)ks_off,
                                                         copy_base[p >> 1] + (unsigned)slot, v0, v1);
        }
    };

    bf16x8 fa[2][8], fb[2][8];
    // Read r of half-step h of the step whose units sit in slots sa, sb.
    auto read = [&](int sa, int sb, int h, int r) {
        const int q = read_block(r);
        if (q < 8)
            fa[h][q] = *reinterpret_cast<const bf16x8 *>(lds + (a_ofs[h] + sa) + q * 16 * ROW_BYTES);
        else
            fb[h][q - 8] = *reinterpret_cast<const bf16x8 *>(lds + (b_ofs[h] + sb) + (q - 8) * 16 * ROW_BYTES);
    };
    // Matrix instruction t of a half-step: block (t / 8, t % 8). B rows are
    // the first operand and A rows the second, so each 16 x 16 result arrives
    // transposed (one C row per lane, four adjacent columns).
    auto mma = [&](int h, int t, bool first) {
        const int i = t >> 3, j = t & 7;
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[h][j], fa[h][i], first ? f32x4{} : acc[i][j], 0, 0, 0);
    };

    // Prologue of the workgroup's first tile: units A0, B0, A1, B1 (A2 comes
    // with the first step's copies, as for every later tile). All four have
    // landed before the first barrier, as the epilogue of every later tile
    // waits for the next tile's first two steps.
#pragma unroll
    for (int u = 0; u < SLOTS - 1; ++u)
        static_for<UNIT_COPIES / 2>([&](auto pr) { copies(u & 1, pr, u * UNIT_BYTES, (u >> 1) * ROW_BYTES, false, false); });
    wait_all_copies();
    lds_barrier();
#pragma unroll
    for (int r = 0; r < 16; ++r)
        read(ring[0], ring[1], 0, r);
    SCHED_FENCE();

    // Step s of the current tile. Its copies fetch step s + 2: the A tile
    // during the first half-step into the slot of B_{s-1} (freed by the
    // previous barrier), the B tile during the second into the slot of A_s.
    // The barrier between the half-steps follows this wave's last read of
    // step s and the landing of its copies of step s + 1; FIRST needs no
    // wait there, since the copies of steps 0 and 1 had all landed before the
    // previous tile's epilogue stores (or before the prologue's barrier).
    // Only the copies' order among themselves is relied on, never their order
    // relative to stores. The order of matrix instructions, LDS reads, copies
    // and scalar instructions inside each half-step is fixed by hand (a
    // scheduling barrier after every matrix instruction and what follows
    // it); only plain vector ALU work may move across those barriers, so its
    // dependency chains spread over several matrix instructions instead of
    // stalling the issue of the next one.
    auto step = [&](int s, auto kind_c) {
        constexpr int kind = decltype(kind_c)::value;
        constexpr bool first = kind == FIRST, next = kind == NEXT0 || kind == NEXT1, tail = kind == TAIL;
        asm volatile("" : "+v"(a_ofs[0]), "+v"(a_ofs[1]), "+v"(b_ofs[0]), "+v"(b_ofs[1]), "+s"(copy_base[0]), "+s"(copy_base[1]));
        // byte offset of the K step the copies fetch (step 0 or 1 of the next tile for NEXT0 / NEXT1)
        const int ks_off = kind == NEXT0 ? 0 : kind == NEXT1 ? ROW_BYTES : (kind == TAIL ? nk - 1 : s + 2) * ROW_BYTES;
        // first half-step: fragments 0; read the second half of step s
        static_for<64>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            mma(0, t, first);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (t == read_at(r))
                    read(ring[0], ring[1], 1, r);
            if constexpr (t >= a_pair_at(0) && (t - a_pair_at(0)) % 16 == 0 && t <= a_pair_at(UNIT_COPIES / 2 - 1))
                copies(0, Int<(t - a_pair_at(0)) / 16>{}, ring[4], ks_off, next, tail);
            SCHED_VALU_ONLY();
        });
        wait_reads();
        if constexpr (!first)
            wait_copies_le<UNIT_COPIES>();
        lds_barrier();
        SCHED_FENCE();
        // second half-step: fragments 1; read the first half of step s + 1
        // (the next tile's first step after a tile's last)
        static_for<64>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            mma(1, t, false);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (t == read_at(r))
                    read(ring[2], ring[3], 0, r);
            constexpr int b_step = b_pair_at(1, kind == NEXT1) - b_pair_at(0, kind == NEXT1);
            constexpr int b0 = b_pair_at(0, kind == NEXT1);
            if constexpr (t >= b0 && (t - b0) % b_step == 0 && (t - b0) / b_step < UNIT_COPIES / 2)
                copies(1, Int<(t - b0) / b_step>{}, ring[0], ks_off, next, tail);
            SCHED_VALU_ONLY();
        });
        wait_reads_known();
        SCHED_FENCE();
        rotate();
    };

    for (;;) {
        step(0, Int<FIRST>{});
        for (int s = 1; s < nk - 3; ++s)
            step(s, Int<MID>{});
        step(nk - 3, Int<TAIL>{});
        step(nk - 2, Int<NEXT0>{});
        step(nk - 1, Int<NEXT1>{});
        // epilogue; the next tile's first two steps are in LDS or landing
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
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int jp = 0; jp < 4; ++jp)
                    store_pair(tm, tn, i, jp, ln, u32x2{}, u32x2{});
        }
        if (!has_next)
            break;
        // switch to the next tile
#pragma unroll
        for (int j = 0; j < UNIT_COPIES; ++j) {
            voff[0][j] = nvoff[0][j];
            voff[1][j] = nvoff[1][j];
        }
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
