// gemm_fp4.hpp -- persistent block-scaled FP4 NT GEMM for gfx950.
//
// The operands are E2M1 codes (two per byte, even k in the low nibble) with
// one E4M3 scale per 16 consecutive K elements of a row ("NVFP4 GEMM on
// Blackwell", section "NVFP4 Datatype"). They are decoded exactly to FP16
// while being staged into LDS, so the matrix-core loop is the ordinary FP16
// one (v_mfma_f32_32x32x16_f16, same rate as BF16).
//
// Work decomposition
//   * Output tile 256 x 256 per workgroup, 4 waves in a 2 x 2 layout, each
//     wave owning a 128 x 128 block = 4 x 4 MFMA blocks of 32 x 32 whose FP32
//     accumulators (256 per lane) live in the accumulation registers.
//   * K advances 64 at a time through a 2-stage LDS ring (2 x 64 KiB): while
//     the matrix cores work on stage s, the next K slice sitting in registers
//     (codes and scales, 18 registers per lane) is decoded and written into
//     stage s^1, and the slice after it is requested from memory. One
//     workgroup barrier per K step separates reuse of a stage.
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
constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // A tile then B tile
constexpr int STAGES = 2;
constexpr int LDS_BYTES = STAGES * STAGE_BYTES;

// Physical 16-byte chunk position of logical chunk `chunk` in LDS tile row `row`.
__device__ inline int swizzle(int row, int chunk)
{
    return chunk ^ (((row >> 1) & 7) ^ ((row & 1) << 1));
}

// ---- block-scaled FP4 operands ---------------------------------------------
//
// Thread t stages rows t / 2 and t / 2 + 128 of the A tile and of the B
// tile, K half t % 2 of each step: 16 bytes of packed codes (32 elements) and
// the row's 4 scale bytes (of which it uses the two of its half) per row and
// operand, held in one of two register sets (the step being written to LDS
// and the step after it, already requested from memory). The two threads of a
// pair read the two halves of the same 32-byte row segment, so each load
// instruction touches 32 rows instead of 64: the memory pipeline's cost
// follows the number of distinct lines a load touches.
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
    u32x4 a_code[2], b_code[2];   // [row r0, r0 + 128]: this thread's 32 codes of each row
    unsigned a_sf[2], b_sf[2];    // the rows' scale dwords (4 blocks of 16)
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

// ---- the persistent kernel --------------------------------------------------
//
// Step kt computes on LDS stage kt & 1 in four sub-steps of 16 matrix
// instructions (K = 16 each); each sub-step's fragments are read during the
// previous one. During sub-steps 0..2 the register set holding step kt + 1 is
// decoded and written into the other stage, 16-byte chunk by chunk (one chunk
// every three matrix instructions, so the decode arithmetic fits in the issue
// gaps of the matrix pipe), and step kt + 2 is requested into the register set
// step kt occupied. The step's single barrier, before sub-step 3, makes the
// new stage visible and releases the current one. Fragment reads are spread
// one per two matrix instructions. Matrix instructions, LDS accesses and loads
// keep their hand-fixed order; the decode arithmetic may move across the
// scheduling barriers, so the dependent conversions and multiplies of a chunk
// spread over several matrix instructions (on gfx950 a wave fits about four
// vector instructions under one 32 x 32 x 16 matrix instruction before the
// matrix rate drops; measured).
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

constexpr int CHUNK_EVERY = 3;   // matrix instructions per written chunk
constexpr int LOADS = 8;         // staging loads per thread and step
constexpr int LOAD_AT = 2;       // first of them (then one every 4 instructions)

// EPI: EPI_PLAIN, or the activation of the fused epilogue (bias, then the
// activation, before rounding). DYN: the dynamic tile order above instead of
// the static one. KTAIL: K % 64 == 32 (else K % 64 == 0), so
// the upper 32-element half of the last step lies past K: its code and scale
// loads are pointed out of range and read zeros (rows are contiguous, so
// reading on would fetch the next row's codes), and a half's two scale bytes
// are loaded with a 16-bit load, since rows of K / 16 scale bytes are then
// only 2-byte aligned.
template <int EPI, bool KTAIL, bool DYN = false>
__global__ __attribute__((amdgpu_flat_work_group_size(THREADS, THREADS), amdgpu_waves_per_eu(1, 1)))
void gemm_nvfp4_nt_kernel(Problem p)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
    __shared__ int next_pos;   // DYN: the workgroup's next tile, written by thread 0
    typedef f16x8 frag;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;   // wave's 128-row half of the tile (A rows)
    const int wn = wave >> 1;  // wave's 128-column half (B rows)
    const int l32 = lane & 31;
    const int half = lane >> 5;
    const int K = p.K;

    // Per-lane LDS fragment addresses: row (l32 + 32 i) of the wave's block,
    // logical chunk (2 kk + half) for K sub-step kk of 16 elements.
    int a_row = (wm * 128 + l32) * ROW_BYTES;
    int b_row = TILE_BYTES + (wn * 128 + l32) * ROW_BYTES;
    int kofs[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        kofs[kk] = swizzle(l32, 2 * kk + half) << 4;   // rows differ from l32 by multiples of 32
    // Staged rows r0 = tid / 2 and r0 + 128 (same swizzle: they differ by a
    // multiple of 16 rows), K half kh = tid % 2 of each step, i.e. logical
    // chunks 4 kh .. 4 kh + 3 of each row. wpos[d]: LDS position of chunk
    // 4 kh + d of row r0; row r0 + 128 is 128 rows further.
    const int r0 = tid >> 1, kh = tid & 1;
    // this half's two scale bytes, moved to bytes 0 and 1 (a 16-bit load puts them there already)
    const int sf_shift = KTAIL ? 0 : 16 * kh;
    int wpos[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
        wpos[d] = r0 * ROW_BYTES + (swizzle(r0, 4 * kh + d) << 4);

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
        const int a_sf_off = (tm * BM + r0) * (int)ks + (KTAIL ? 2 * kh : 0);
        const int b_sf_off = (tn * BN + r0) * (int)ks + (KTAIL ? 2 * kh : 0);
        const int row2_codes = 128 * (int)kc, row2_sf = 128 * (int)ks;   // row r0 + 128
        StageRegs regs[2];
        // load q (0..7) of step kt into register set `set`: codes of row r0,
        // codes of row r0 + 128, scales of r0, scales of r0 + 128, for A (q < 4)
        // then B. The per-lane part of the offset is fixed for the tile (rows
        // past M or N lie beyond the buffer and read zeros); the step's K
        // offset is uniform and goes in the scalar offset. A step is whole or
        // past K, except with KTAIL the upper half of the last step, whose
        // loads go out of range and read zeros (zero codes: the half adds
        // nothing). Steps past K are requests made ahead for a step the tile
        // never computes, and read step 0 again instead.
        auto load = [&](int kt, int set, int q) {
            const int k0 = kt * BK < K ? kt * BK : 0;
            // per-lane offset of this half (row r0 or r0 + 128 of either operand)
            auto at = [&](int off) {
                if constexpr (KTAIL)
                    return (kh && kt == nk - 1) ? OOB : off;
                return off;
            };
            auto sf = [&](__amdgpu_buffer_rsrc_t rs, int off) -> unsigned {
                if constexpr (KTAIL)
                    return __builtin_amdgcn_raw_buffer_load_b16(rs, at(off), k0 / 16, 0);
                return __builtin_amdgcn_raw_buffer_load_b32(rs, off, k0 / 16, 0);
            };
            StageRegs &r = regs[set];
            switch (q) {
            case 0: r.a_code[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, at(a_code_off), k0 / 2, 0)); break;
            case 1: r.a_code[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, at(a_code_off + row2_codes), k0 / 2, 0)); break;
            case 2: r.a_sf[0] = sf(rsa, a_sf_off); break;
            case 3: r.a_sf[1] = sf(rsa, a_sf_off + row2_sf); break;
            case 4: r.b_code[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, at(b_code_off), k0 / 2, 0)); break;
            case 5: r.b_code[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, at(b_code_off + row2_codes), k0 / 2, 0)); break;
            case 6: r.b_sf[0] = sf(rsb, b_sf_off); break;
            default: r.b_sf[1] = sf(rsb, b_sf_off + row2_sf); break;
            }
        };
        // chunk c (0..15) of register set `set` into `stage`: A for c < 8,
        // else B; row r0 + 128 * ((c / 4) & 1); chunk 4 kh + c % 4 of the row
        auto write_chunk = [&](uint8_t *stage, int set, auto c_c) {
            constexpr int c = decltype(c_c)::value;
            constexpr int rr = (c >> 2) & 1, d = c & 3;
            const StageRegs &r = regs[set];
            const unsigned codes = (c < 8 ? r.a_code : r.b_code)[rr][d];
            const f16x2 s = scale2<d / 2>(scales2((c < 8 ? r.a_sf : r.b_sf)[rr] >> sf_shift));
            *reinterpret_cast<f16x8 *>(stage + (c < 8 ? 0 : TILE_BYTES) + rr * 128 * ROW_BYTES + wpos[d]) = decode8(codes, s);
        };

        f32x16 acc[4][4];
        frag fa[2][4], fb[2][4];
        auto read_frags = [&](const uint8_t *stage, int kk, int set) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                fa[set][i] = *reinterpret_cast<const frag *>(stage + a_row + i * 32 * ROW_BYTES + kofs[kk]);
                fb[set][i] = *reinterpret_cast<const frag *>(stage + b_row + i * 32 * ROW_BYTES + kofs[kk]);
            }
        };
        // fragment read r (0..7): A block r for r < 4, else B block r - 4
        auto read_frag = [&](const uint8_t *stage, int kk, int set, int r) {
            if (r < 4)
                fa[set][r] = *reinterpret_cast<const frag *>(stage + a_row + r * 32 * ROW_BYTES + kofs[kk]);
            else
                fb[set][r - 4] = *reinterpret_cast<const frag *>(stage + b_row + (r - 4) * 32 * ROW_BYTES + kofs[kk]);
        };
        auto mma = [&](int set, int t, bool first) {
            const int i = (t >> 2) & 3, j = t & 3;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[set][j], fa[set][i], first ? f32x16{} : acc[i][j], 0, 0, 0);
        };

        // Prologue: step 0 into stage 0, step 1 requested into set 1.
        lds_barrier();            // every wave is done with the previous tile's stages
#pragma unroll
        for (int q = 0; q < LOADS; ++q)
            load(0, 0, q);
#pragma unroll
        for (int q = 0; q < LOADS; ++q)
            load(1, 1, q);
        static_for<16>([&](auto c) { write_chunk(lds, 0, c); });
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
        read_frags(lds, 0, 0);
        SCHED_FENCE();

        // par = kt & 1, a compile-time value so that the register sets are
        // named statically (a runtime index would put them in scratch memory)
        auto step = [&](int kt, auto par_c, auto first_c) {
            constexpr int par = decltype(par_c)::value;
            constexpr bool first = decltype(first_c)::value;
            uint8_t *cur = lds + par * STAGE_BYTES;
            uint8_t *nxt = lds + (par ^ 1) * STAGE_BYTES;
            constexpr int set_next = par ^ 1;   // holds step kt + 1
            constexpr int set_free = par;       // held step kt, already written
            // LDS address bases, hidden from the optimiser again at every step so
            // that the addresses of both stages are formed where they are used
            // instead of all being hoisted out of the loop (which spills)
            asm volatile("" : "+v"(wpos[0]), "+v"(wpos[1]), "+v"(wpos[2]), "+v"(wpos[3]), "+v"(kofs[0]),
                         "+v"(kofs[1]), "+v"(kofs[2]), "+v"(kofs[3]), "+v"(a_row), "+v"(b_row));
            // sub-steps 0..2: fragments of sub-step kk + 1 read during sub-step kk
            static_for<48>([&](auto tc) {
                constexpr int t = decltype(tc)::value;
                constexpr int kk = t >> 4;
                mma(kk & 1, t & 15, first && kk == 0);
                if constexpr ((t & 15) % 2 == 0)
                    read_frag(cur, kk + 1, (kk + 1) & 1, (t & 15) / 2);
                if constexpr (t % CHUNK_EVERY == 1 && t / CHUNK_EVERY < 16)
                    write_chunk(nxt, set_next, Int<t / CHUNK_EVERY>{});
                if constexpr (t >= LOAD_AT && (t - LOAD_AT) % 4 == 0 && (t - LOAD_AT) / 4 < LOADS)
                    load(kt + 2, set_free, (t - LOAD_AT) / 4);
                SCHED_VALU_ONLY();
            });
            // the next stage is written by every wave, the current one fully read
            lds_barrier();
            SCHED_FENCE();
            // sub-step 3 on fragments set 1, first fragments of the next stage
            static_for<16>([&](auto tc) {
                constexpr int t = decltype(tc)::value;
                mma(1, t, false);
                if constexpr (t % 2 == 0)
                    read_frag(nxt, 0, 0, t / 2);
                SCHED_VALU_ONLY();
            });
        };

        if (nk == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = f32x16{};
        } else {
            step(0, Int<0>{}, Int<1>{});
            int kt = 1;
            for (; kt + 1 < nk; kt += 2) {
                step(kt, Int<1>{}, Int<0>{});
                step(kt + 1, Int<0>{}, Int<0>{});
            }
            if (kt < nk)
                step(kt, Int<1>{}, Int<0>{});
        }

        store_tile<EPI>(acc, rc, rbias, p.M, p.N, tm * BM + wm * 128, tn * BN + wn * 128, l32, half);
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
