// gemm_fp4.hpp -- persistent block-scaled FP4 NT GEMM for gfx950.
//
// The operands are E2M1 codes (two per byte, even k in the low nibble) with
// one E4M3 scale per 16 consecutive K elements of a row ("NVFP4 GEMM on
// Blackwell", section "NVFP4 Datatype"). They are decoded exactly to FP16
// while being staged into LDS, so the matrix-core loop is the ordinary FP16
// one (v_mfma_f32_16x16x32_f16, same rate as BF16).
//
// Work decomposition
//   * Output tile 256 x 256 per workgroup, 8 waves in a 2 x 4 layout, two per
//     SIMD, each wave owning a 128 x 64 block = 8 x 4 MFMA blocks of 16 x 16
//     (128 FP32 accumulators per lane). 16 x 16 x 32 rather than 32 x 32 x 16
//     instructions: the same cycles per product, but half the accumulator
//     reads and writes per product, and the chip runs at a power limit, so
//     the clock it holds under this loop is higher (measured 5-7 % faster at
//     4096^3 to 8192^3, bitwise the same C).
//   * Two waves per SIMD because the decode is vector ALU work beside the
//     matrix instructions: measured on gfx950 with a probe (one
//     32 x 32 x 16 FP16 matrix instruction and n conversions or packed
//     multiplies issued after it, in a loop), one wave per SIMD loses 12, 18
//     and 25 % of the matrix rate at n = 2, 3 and 4, while two waves per SIMD
//     lose 1, 3 and 4 %: the other wave's matrix instructions fill the issue
//     cycles the vector instructions take.
//   * K advances 64 at a time through a 2-stage LDS ring (2 x 64 KiB): while
//     the matrix cores work on stage s, the next K slice sitting in registers
//     (codes and scales, 10 registers per lane) is decoded and written into
//     stage s^1, and the slice three steps ahead is requested from memory into
//     one of three register sets. One workgroup barrier per K step separates
//     reuse of a stage. LDS holds the A tiles of both stages, then the B
//     tiles, so a stage's 32 KiB offset fits the immediate offset of the LDS
//     instructions and no address arithmetic is repeated per step.
//   * LDS rows are 128 bytes (64 FP16 values); the 16-byte chunk c of row r is
//     stored at chunk position c ^ s(r), s(r) = ((r >> 1) & 7) ^ ((r & 1) << 1).
//     Measured on gfx950 (a probe timing each access pattern): ds_read_b128
//     serves 16 lanes (256 bytes over 64 four-byte banks) per cycle, and the
//     fragment reads -- 16 rows at one logical chunk -- hit 16 distinct bank
//     groups for any s whose (row parity, s) pairs are distinct; ds_write_b128
//     serves 8 lanes per cycle within a 128-byte bank window, and a staging
//     write -- four consecutive rows, two chunks 4 apart each -- needs s & 3
//     distinct over every aligned group of four rows. The plain (r >> 1) & 7
//     fails the second (16 against 13 cycles per write); folding row bit 0
//     into bit 1 satisfies both.
#pragma once

#include "common.hpp"

#include <utility>

namespace gemm355 {
namespace fp4 {

constexpr int BK = 64;                       // K elements per pipeline step
constexpr int ROW_BYTES = BK * 2;            // one LDS tile row: 64 x FP16
constexpr int TILE_BYTES = BM * ROW_BYTES;   // 32 KiB per operand per stage
constexpr int STAGES = 2;
constexpr int A_TILES = 0;                        // A tile of stage s at A_TILES + s * TILE_BYTES
constexpr int B_TILES = STAGES * TILE_BYTES;      // B tile of stage s at B_TILES + s * TILE_BYTES
constexpr int LDS_BYTES = 2 * STAGES * TILE_BYTES;
constexpr int THREADS_FP4 = 512;             // 8 waves, two per SIMD
static_assert(BM == 256 && BN == 256, "the staging map assumes 256 x 256 tiles");

// Physical 16-byte chunk position of logical chunk `chunk` in LDS tile row `row`.
__device__ inline int swizzle(int row, int chunk)
{
    return chunk ^ (((row >> 1) & 7) ^ ((row & 1) << 1));
}

// ---- block-scaled FP4 operands ---------------------------------------------
//
// Thread t stages row t / 2 of the A tile and of the B tile, K half t % 2 of
// each step: 16 bytes of packed codes (32 elements) and the two scale bytes
// of that half per operand, held in one of three register sets (the step
// being written to LDS and the two after it, already requested from
// memory). The two threads of a pair read the two halves of the same 32-byte
// row segment, so each load instruction touches 32 rows instead of 64: the
// memory pipeline's cost follows the number of distinct lines a load
// touches, and each instruction has a cost of its own (timing-only variants
// at 8192^3: without the code loads 9 % faster, without the scale loads 7 %,
// though those move an eighth of the bytes). So the scales of a pair of
// steps come with one instruction: for an even step s the thread with K half
// h loads the four scale bytes of step s + h (a dword), and each thread takes
// the two it needs from its own dword or its partner's (adjacent lanes, one
// lane swap): half the scale instructions, 2 % faster at 8192^3. (With K %
// 64 == 32 a row's scales are not dword aligned; that instance keeps one
// 16-bit load per thread and step.)
// Decoding ("NVFP4 GEMM on Blackwell", section "NVFP4 Datatype"): each code
// pair converts to two FP16 E2M1 values (v_cvt_scalef32_pk_f16_fp4 with a unit
// scale), then one packed FP16 multiply applies the E4M3 scale of its 16-element
// block. Both steps are exact: an E4M3 value and every product e2m1 * e4m3
// lie in FP16's normal range with at most 6 significant bits. (gfx950's scaled
// FP4 conversion applies only the exponent of its scale operand, which is why
// the E4M3 mantissa goes through the multiply, and FP16 rather than BF16 is
// used because gfx950 has a packed FP16 multiply but no packed BF16 one; the
// FP16 and BF16 matrix instructions have the same rate.)
struct StageRegs {
    u32x4 a_code, b_code;   // this thread's 32 codes of its A row and of its B row
    unsigned a_sf, b_sf;    // their two scale bytes (16-element blocks 2 kh, 2 kh + 1 of the step) in bytes 0, 1
};

// 8 codes (one dword) scaled by `s` -> 8 FP16 values.
__device__ inline f16x8 decode8(unsigned codes, f16x2 s)
{
    f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s;
    f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s;
    f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s;
    f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s;
    f16x8 r = {v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
    return r;
}

// E4M3 scale bytes 0 and 1 of `sf` as FP16 (exact: FP16 holds every E4M3
// value), one conversion for the two 16-element blocks of a half step.
__device__ inline f16x2 scales2(unsigned sf) { return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sf, 1.0f, false); }

// Scale BLK (0 or 1) of such a pair in both halves.
template <int BLK>
__device__ inline f16x2 scale2(f16x2 s)
{
    return f16x2{s[BLK], s[BLK]};
}

// ---- dynamic tile order (a measurement option) -------------------------------
//
// "NVFP4 GEMM on Blackwell", "Production Kernel", "Static vs Dynamic Tile
// Scheduling": instead of the fixed round-robin order, a workgroup asks for
// its next tile when it starts the current one. Here a ticket counter per XCD
// keeps each XCD's tiles the ones the static order gives it (so their A and B
// strips still share that XCD's L2); a workgroup whose XCD has no tiles left
// takes them from the other XCDs' counters in turn, which is where the order
// can rebalance work. Ticket i of XCD x (g = grid / 8 workgroups per XCD) is
// position (i / g) grid + x g + i % g of the visiting order; tickets 0 .. g - 1
// are the first round, which each workgroup takes without asking. Each
// counter has its own 256-byte line. The counters start at zero, and the last
// workgroup to finish sets them back to zero, so every launch finds them
// cleared; launches that overlap on one GPU share them and must not use this
// option.
struct DynamicOrder {
    unsigned next[8][64];   // next[x][0]: tickets handed out on XCD x beyond the first round
    unsigned done[64];      // done[0]: workgroups that found no tile left
};
__device__ DynamicOrder g_dynamic_order;

constexpr int CHUNK_EVERY = 6;   // matrix instructions per written chunk
constexpr int LOADS = 4;         // staging loads per thread and step
constexpr int LOAD_AT = 2;       // first of them (then one every LOAD_EVERY instructions)
constexpr int LOAD_EVERY = 12;
constexpr int SETS = 3;          // register sets: a step's loads are issued three steps before it is computed

// EPI: EPI_PLAIN, or the activation of the fused epilogue (bias, then the
// activation, before rounding). DYN: the dynamic tile order above instead of
// the static one. KTAIL: K % 64 == 32 (else K % 64 == 0), so the upper
// 32-element half of the last step lies past K: its code and scale loads are
// pointed out of range and read zeros (rows are contiguous, so reading on
// would fetch the next row's codes).
template <int EPI, bool KTAIL, bool DYN = false>
__global__ __attribute__((amdgpu_flat_work_group_size(THREADS_FP4, THREADS_FP4), amdgpu_waves_per_eu(2, 2)))
void gemm_nvfp4_nt_kernel(Problem p)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
    __shared__ int next_pos;   // DYN: the workgroup's next tile, written by thread 0
    typedef f16x8 frag;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;   // wave's 128-row half of the tile (A rows)
    const int wn = wave >> 1;  // wave's 64-column quarter (B rows)
    const int l16 = lane & 15;
    const int grp = lane >> 4;
    const int K = p.K;

    // Per-lane LDS fragment addresses in stage 0: row l16 of the wave's first
    // block, logical chunk (4 h + grp) for K sub-step h of 32 elements; block
    // i and stage s add 16 i rows and s * TILE_BYTES (immediate offsets)
    int fa_at[2], fb_at[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int ko = swizzle(l16, 4 * h + grp) << 4;   // rows differ from l16 by multiples of 16
        fa_at[h] = A_TILES + (wm * 128 + l16) * ROW_BYTES + ko;
        fb_at[h] = B_TILES + (wn * 64 + l16) * ROW_BYTES + ko;
    }
    // Staged row r0 = tid / 2 of each operand, K half kh = tid % 2 of each
    // step, i.e. logical chunks 4 kh .. 4 kh + 3 of the row; wa[d] / wb[d]:
    // LDS position of chunk 4 kh + d in stage 0's A / B tile
    const int r0 = tid >> 1, kh = tid & 1;
    int wa[4], wb[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        wa[d] = A_TILES + r0 * ROW_BYTES + (swizzle(r0, 4 * kh + d) << 4);
        wb[d] = wa[d] - A_TILES + B_TILES;
    }

    const unsigned kc = (unsigned)K / 2, ks = (unsigned)K / 16;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, (unsigned)p.M * kc);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.b, (unsigned)p.N * kc);
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(p.sfa, (unsigned)p.M * ks);
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(p.sfb, (unsigned)p.N * ks);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.c, (unsigned)p.M * (unsigned)p.N * 2u);
    const __amdgpu_buffer_rsrc_t rbias = make_rsrc(p.bias, EPI != EPI_PLAIN && p.bias ? (unsigned)p.N * 2u : 0u);
    const int nk = (K + BK - 1) / BK;

    // dynamic order: XCDs (counters) and workgroups per XCD, and this one's XCD
    const int nx = p.grid % 8 == 0 ? 8 : 1, per_xcd = p.grid / nx, xcd = blockIdx.x % nx;
    auto ticket_position = [&](int x, unsigned i) {
        return (int)(i / (unsigned)per_xcd) * p.grid + x * per_xcd + (int)(i % (unsigned)per_xcd);
    };
    int pos = schedule_position(blockIdx.x, 0, p.grid);
    for (int round = 0;; ++round) {
        if (!DYN)
            pos = schedule_position(blockIdx.x, round, p.grid);
        if (pos >= p.tiles)
            break;
        // DYN: the ticket for the next tile, requested now (one lane, a
        // vector-memory atomic), turned into a position after the prologue
        unsigned ticket = 0;
        if (DYN && tid == 0)
            ticket = atomicAdd(&g_dynamic_order.next[xcd][0], 1u);
        int tm, tn;
        supergroup_tile(pos, p.tiles_m, p.tiles_n, p.supergroup, tm, tn);

        const int a_code_off = (tm * BM + r0) * (int)kc + 16 * kh, b_code_off = (tn * BN + r0) * (int)kc + 16 * kh;
        // scale offsets: KTAIL, the thread's two bytes of each step; else the
        // dword of step 2 b + kh for a pair of steps 2 b, 2 b + 1 (see load)
        const int sf_lane = KTAIL ? 2 * kh : 4 * kh;
        const int a_sf_off = (tm * BM + r0) * (int)ks + sf_lane, b_sf_off = (tn * BN + r0) * (int)ks + sf_lane;
        StageRegs regs[SETS];
        // load q (0..3) of step kt into register set `set`: A codes, A scales,
        // B codes, B scales. The per-lane part of the offset is fixed for the
        // tile (rows past M or N lie beyond the buffer and read zeros); the
        // step's K offset is uniform and goes in the scalar offset. A step is
        // whole or past K, except with KTAIL the upper half of the last step,
        // whose loads go out of range and read zeros (zero codes: the half adds
        // nothing). Steps past K are requests made ahead for a step the tile
        // never computes, and read step 0 again instead.
        auto load = [&](int kt, int set, int q) {
            const int k0 = kt * BK < K ? kt * BK : 0;
            auto at = [&](int off) {
                if constexpr (KTAIL)
                    return (kh && kt == nk - 1) ? OOB : off;
                return off;
            };
            StageRegs &r = regs[set];
            switch (q) {
            case 0: r.a_code = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, at(a_code_off), k0 / 2, 0)); break;
            case 1:
                if constexpr (KTAIL)
                    r.a_sf = __builtin_amdgcn_raw_buffer_load_b16(rsa, at(a_sf_off), k0 / 16, 0);
                else
                    r.a_sf = __builtin_amdgcn_raw_buffer_load_b32(rsa, a_sf_off, k0 / 16, 0);
                break;
            case 2: r.b_code = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, at(b_code_off), k0 / 2, 0)); break;
            default:
                if constexpr (KTAIL)
                    r.b_sf = __builtin_amdgcn_raw_buffer_load_b16(rsb, at(b_sf_off), k0 / 16, 0);
                else
                    r.b_sf = __builtin_amdgcn_raw_buffer_load_b32(rsb, b_sf_off, k0 / 16, 0);
                break;
            }
        };
        // chunk c (0..7) of register set `set` (step s) into stage `st`: A for
        // c < 4, else B; chunk 4 kh + c % 4 of the thread's row. Its two scale
        // bytes: KTAIL, in set `set`; else in set `sf_set` (s's own set for an
        // even s, step s - 1's for an odd one), in the dword lane 2 (r0 % 32)
        // + (s % 2) loaded, bytes 2 kh and 2 kh + 1.
        auto write_chunk = [&](int st, int set, auto c_c, int sf_set, auto odd_c) {
            constexpr int c = decltype(c_c)::value;
            constexpr int d = c & 3;
            const StageRegs &r = regs[set];
            const unsigned codes = (c < 4 ? r.a_code : r.b_code)[d];
            const int src = KTAIL ? set : sf_set;
            unsigned sf = c < 4 ? regs[src].a_sf : regs[src].b_sf;
            if constexpr (!KTAIL) {
                constexpr int odd = decltype(odd_c)::value;
                // the pair's lanes are adjacent: swap within each pair
                const unsigned other = (unsigned)__builtin_amdgcn_mov_dpp((int)sf, 0xB1, 0xF, 0xF, false);
                sf = (kh == odd ? sf : other) >> (16 * kh);
            }
            const f16x2 s = scale2<d / 2>(scales2(sf));
            *reinterpret_cast<f16x8 *>(lds + (c < 4 ? wa[d] : wb[d]) + st * TILE_BYTES) = decode8(codes, s);
        };

        f32x4 acc[8][4];
        // A fragments in a ring of four (block i in fa[i % 4], read three
        // blocks ahead of its use), B fragments in one set per sub-step
        frag fa[4], fb[2][4];
        auto read_a = [&](int st, int h, int i) {
            fa[i & 3] = *reinterpret_cast<const frag *>(lds + fa_at[h] + st * TILE_BYTES + i * 16 * ROW_BYTES);
        };
        auto read_b = [&](int st, int h, int j) {
            fb[h][j] = *reinterpret_cast<const frag *>(lds + fb_at[h] + st * TILE_BYTES + j * 16 * ROW_BYTES);
        };
        // matrix instruction u (0..31) of sub-step h: block (u / 4, u % 4)
        auto mma = [&](int h, int u, bool first) {
            const int i = u >> 2, j = u & 3;
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fb[h][j], fa[i & 3], first ? f32x4{} : acc[i][j], 0, 0, 0);
        };

        // Prologue: step 0 into stage 0, steps 1 and 2 requested into sets 1, 2.
        lds_barrier();            // every wave is done with the previous tile's stages
#pragma unroll
        for (int kt = 0; kt < SETS; ++kt)
#pragma unroll
            for (int q = 0; q < LOADS; ++q)
                if (KTAIL || (kt % 2 == 0) || q % 2 == 0)   // an odd step's scales come with the even one's
                    load(kt, kt, q);
        static_for<8>([&](auto c) { write_chunk(0, 0, c, 0, Int<0>{}); });
        // DYN: the ticket has returned by now (it was requested before the
        // loads just written out); thread 0 turns it into the next tile
        if (DYN && tid == 0) {
            int np = ticket_position(xcd, (unsigned)per_xcd + ticket);
            // this XCD has no tile left: take one from the other XCDs in turn
            for (int d = 1; d < nx && np >= p.tiles; ++d) {
                const int y = (xcd + d) % nx;
                np = ticket_position(y, (unsigned)per_xcd + atomicAdd(&g_dynamic_order.next[y][0], 1u));
            }
            next_pos = np;
        }
        lds_barrier();
#pragma unroll
        for (int i = 0; i < 3; ++i)
            read_a(0, 0, i);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            read_b(0, 0, j);
        SCHED_FENCE();

        // Step kt computes on LDS stage kt % 2 (par) in two sub-steps h of 32
        // matrix instructions (K = 32 each), in groups of four that share an
        // A block. Group g of a sub-step reads the A block three groups ahead
        // (into the ring slot group g - 1 has just finished with); during
        // sub-step 0 the B blocks of sub-step 1 are read into the other B set.
        // Meanwhile the register set holding step kt + 1 is decoded and
        // written into the other stage, one chunk every six matrix
        // instructions, and step kt + 3 is requested into the set step kt
        // occupied (kt % 3, already written). The step's single barrier, after
        // group 4 of sub-step 1 (the last read of stage par), makes the new
        // stage visible and releases the current one; group 5 then reads the
        // next step's four B blocks, and groups 5..7 its first three A blocks.
        // Matrix instructions, LDS accesses and loads keep their hand-fixed
        // order; the decode arithmetic may move across the scheduling
        // barriers, so the dependent conversions and multiplies of a chunk
        // spread over several matrix instructions. Set and stage indices are
        // compile-time values so that the register sets are named statically
        // (a runtime index would put them in scratch memory).
        auto step = [&](int kt, auto par_c, auto set_c, auto first_c) {
            constexpr int par = decltype(par_c)::value;
            constexpr bool first = decltype(first_c)::value;
            constexpr int set_free = decltype(set_c)::value;   // held step kt, already written
            constexpr int set_next = (set_free + 1) % SETS;    // holds step kt + 1
            static_for<64>([&](auto tc) {
                constexpr int t = decltype(tc)::value;
                constexpr int h = t >> 5, u = t & 31, g = u >> 2;
                if constexpr (h == 1 && u == 20) {
                    // the next stage is written by every wave, the current one fully read
                    lds_barrier();
                    SCHED_FENCE();
                }
                mma(h, u, first && h == 0);
                if constexpr (u % 4 == 0) {
                    if constexpr (g < 5)
                        read_a(par, h, g + 3);
                    else if constexpr (h == 0)
                        read_a(par, 1, g - 5);
                    else
                        read_a(par ^ 1, 0, g - 5);
                }
                if constexpr (h == 0 && u % 4 == 2 && g < 4)
                    read_b(par, 1, g);
                if constexpr (h == 1 && u >= 20 && u < 24)
                    read_b(par ^ 1, 0, u - 20);
                // step kt + 1 has parity par ^ 1; an odd one's scales sit in
                // step kt's set
                if constexpr (t % CHUNK_EVERY == 1 && t / CHUNK_EVERY < 8)
                    write_chunk(par ^ 1, set_next, Int<t / CHUNK_EVERY>{}, par == 0 ? set_free : set_next, Int<par ^ 1>{});
                // step kt + 3 has parity par ^ 1: without KTAIL an odd step
                // loads no scales, which keeps set_free's scale registers (step
                // kt's dword pair, whose odd half step kt + 1 uses) intact
                if constexpr (t >= LOAD_AT && (t - LOAD_AT) % LOAD_EVERY == 0 && (t - LOAD_AT) / LOAD_EVERY < LOADS) {
                    constexpr int q = (t - LOAD_AT) / LOAD_EVERY;
                    if constexpr (KTAIL || par == 1 || q % 2 == 0)
                        load(kt + SETS, set_free, q);
                }
                SCHED_VALU_ONLY();
            });
        };

        if (nk == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = f32x4{};
        } else {
            // step kt uses LDS stage kt % 2 and register set kt % 3: six step
            // bodies cover both cycles
            step(0, Int<0>{}, Int<0>{}, Int<1>{});
            int kt = 1;
            for (; kt + 5 < nk; kt += 6) {
                step(kt, Int<1>{}, Int<1>{}, Int<0>{});
                step(kt + 1, Int<0>{}, Int<2>{}, Int<0>{});
                step(kt + 2, Int<1>{}, Int<0>{}, Int<0>{});
                step(kt + 3, Int<0>{}, Int<1>{}, Int<0>{});
                step(kt + 4, Int<1>{}, Int<2>{}, Int<0>{});
                step(kt + 5, Int<0>{}, Int<0>{}, Int<0>{});
            }
            if (kt < nk)
                step(kt, Int<1>{}, Int<1>{}, Int<0>{});
            if (kt + 1 < nk)
                step(kt + 1, Int<0>{}, Int<2>{}, Int<0>{});
            if (kt + 2 < nk)
                step(kt + 2, Int<1>{}, Int<0>{}, Int<0>{});
            if (kt + 3 < nk)
                step(kt + 3, Int<0>{}, Int<1>{}, Int<0>{});
            if (kt + 4 < nk)
                step(kt + 4, Int<1>{}, Int<2>{}, Int<0>{});
        }

        store_tile16<EPI>(acc, rc, rbias, p.M, p.N, tm * BM + wm * 128, tn * BN + wn * 64, lane);
        if (DYN)
            pos = next_pos;   // written before the prologue's barrier, rewritten only after the next one
    }
    if (DYN && tid == 0) {
        // every workgroup that finished has stopped asking for tickets: the
        // last one clears the counters for the next launch
        if (atomicAdd(&g_dynamic_order.done[0], 1u) == (unsigned)p.grid - 1) {
            for (int x = 0; x < 8; ++x)
                atomicExch(&g_dynamic_order.next[x][0], 0u);
            atomicExch(&g_dynamic_order.done[0], 0u);
        }
    }
}

} // namespace fp4
} // namespace gemm355
