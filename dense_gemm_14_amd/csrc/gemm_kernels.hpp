// gemm_kernels.hpp -- gfx950 device code of libgemm355.
//
// One persistent kernel template computes C = A * B^T for row-major A (M x K)
// and B (N x K); two staging policies feed it:
//   * Bf16Staging: BF16 operands copied global -> registers -> LDS;
//   * Fp4Staging:  E2M1 codes + E4M3 scales decoded exactly to FP16 while
//     they are staged, so the same LDS layout and matrix-core loop follow.
//
// Work decomposition
//   * Output tile 256 x 256 per workgroup, 4 waves in a 2 x 2 layout, each
//     wave owning a 128 x 128 block = 4 x 4 MFMA blocks of 32 x 32 whose FP32
//     accumulators (256 per lane) live in the accumulation registers.
//   * K advances 64 at a time through a 2-stage LDS ring (2 x 64 KiB): while
//     the matrix cores work on stage s, the next K slice already sitting in
//     registers is written into stage s^1 and the slice after it is requested
//     from memory, so each global load has a whole K step to arrive. One
//     workgroup barrier per K step separates reuse of a stage.
//   * LDS rows are 128 bytes (64 elements); the 16-byte chunk c of row r is
//     stored at chunk position c ^ ((r >> 1) & 7). gfx950's LDS serves a
//     ds_read_b128 16 lanes (256 bytes, 64 banks of 4 bytes) per cycle; the 16
//     consecutive rows one such group reads at the same logical chunk then
//     cover all 16 bank groups (row parity picks the 128-byte half of the bank
//     space, (r >> 1) & 7 the chunk within it). Measured on the device: 4 LDS
//     cycles per ds_read_b128 and no bank conflicts, against 8 cycles with the
//     c ^ (r & 7) swizzle that suits a 32-bank LDS.
//   * The matrix instruction is v_mfma_f32_32x32x16_{bf16,f16}. It is fed
//     B rows as its first operand and A rows as its second, so the 32 x 32
//     result block arrives transposed: each lane holds one row m of C and
//     runs of 4 consecutive columns, which the epilogue pairs across the two
//     half-waves (v_permlane32_swap) into 16-byte row segments.
//   * Operands are read through buffer resources whose range ends at the
//     operand's last byte: rows past M or N read as zero, and a K tail or
//     masked store uses an offset beyond every range (loads return 0, stores
//     are dropped), so no tile needs a bounds branch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "schedule.hpp"

namespace gemm355 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256;                      // output tile rows (M)
constexpr int BN = 256;                      // output tile columns (N)
constexpr int BK = 64;                       // K elements per pipeline step
constexpr int THREADS = 256;                 // 4 waves of 64 lanes
constexpr int ROW_BYTES = BK * 2;            // one LDS tile row: 64 x 16-bit
constexpr int TILE_BYTES = BM * ROW_BYTES;   // 32 KiB per operand per stage
constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // A tile then B tile
constexpr int STAGES = 2;
constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
constexpr int OOB = (int)0x80000000;         // beyond every buffer range
constexpr unsigned RSRC_WORD3 = 0x00020000u; // raw buffer, 32-bit data format

static_assert(BM == BN, "the staging maps assume square tiles");

struct Problem {
    const void *a;    // BF16 A, or E2M1 codes of A
    const void *b;    // BF16 B, or E2M1 codes of B
    const void *sfa;  // E4M3 scales of A (FP4 only)
    const void *sfb;  // E4M3 scales of B (FP4 only)
    void *c;
    int M, N, K;
    int tiles_m, tiles_n, tiles;
    int supergroup;
    int grid;
};

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *p, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, RSRC_WORD3);
}

// Physical 16-byte chunk position of logical chunk `chunk` in LDS tile row `row`.
__device__ inline int swizzle(int row, int chunk)
{
    return chunk ^ ((row >> 1) & 7);
}

// Byte offset of 16-byte chunk `chunk` of LDS tile row `row`.
__device__ inline int lds_offset(int row, int chunk)
{
    return row * ROW_BYTES + (swizzle(row, chunk) << 4);
}

__device__ inline unsigned pack_bf16(float lo, float hi)
{
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2)); // RNE
}

// ---- instruction interleaving hints ---------------------------------------
//
// Each hint asks the scheduler for `n` instructions of one class at this point
// of the region's order (classes: matrix, LDS read, LDS write, global read,
// vector ALU). A K step issues 64 matrix instructions of 32 cycles each per
// wave; everything else is threaded between them so that the matrix pipe never
// waits for an issue slot.
enum : int { SG_VALU = 0x002, SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100, SG_DS_WRITE = 0x200 };
#define SCHED(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// Nothing is moved across this point by the scheduler.
#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// One sub-step: 16 matrix instructions with the 8 fragment reads of the next
// sub-step threaded in, one read after each of the first 8.
__device__ inline void schedule_reads_with_mma()
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        SCHED(SG_MFMA, 1);
        SCHED(SG_DS_READ, 1);
    }
    SCHED(SG_MFMA, 8);
}

// ---- BF16 operands --------------------------------------------------------
//
// Each thread copies, per operand and K step, 8 chunks of 16 bytes: rows
// (tid / 8) + 32 i, chunk tid % 8 -- eight consecutive lanes cover one
// 128-byte row segment, so every load instruction reads whole cache lines.
struct Bf16Staging {
    typedef bf16x8 frag;
    __amdgpu_buffer_rsrc_t ra, rb;
    int a_row_off, b_row_off; // byte offset of this thread's first row + its chunk
    int chunk_k;              // K index of this thread's chunk within a step
    int lds_off;              // LDS byte offset of this thread's first chunk
    int K;
    u32x4 a_reg[8], b_reg[8];

    __device__ void init(const Problem &p, int tm, int tn, int tid)
    {
        ra = make_rsrc(p.a, (unsigned)p.M * (unsigned)p.K * 2u);
        rb = make_rsrc(p.b, (unsigned)p.N * (unsigned)p.K * 2u);
        const int row = tid >> 3, chunk = tid & 7;
        K = p.K;
        chunk_k = chunk * 8;
        a_row_off = ((tm * BM + row) * p.K + chunk_k) * 2;
        b_row_off = ((tn * BN + row) * p.K + chunk_k) * 2;
        lds_off = lds_offset(row, chunk);
    }

    __device__ void load(int k0)
    {
        const bool valid = k0 + chunk_k < K;   // K % 8 == 0: a chunk is all in or all out
        const int step = 32 * K * 2;           // 32 rows further down
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int oa = valid ? a_row_off + i * step + k0 * 2 : OOB;
            const int ob = valid ? b_row_off + i * step + k0 * 2 : OOB;
            a_reg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, oa, 0, 0));
            b_reg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, ob, 0, 0));
        }
    }

    __device__ void commit(uint8_t *stage)
    {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            *reinterpret_cast<u32x4 *>(stage + lds_off + i * 32 * ROW_BYTES) = a_reg[i];
            *reinterpret_cast<u32x4 *>(stage + TILE_BYTES + lds_off + i * 32 * ROW_BYTES) = b_reg[i];
        }
    }

    static __device__ f32x16 mma(frag s0, frag s1, f32x16 acc)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(s0, s1, acc, 0, 0, 0);
    }

    // Sub-step 1: 16 matrix instructions, 8 fragment reads, the 16 LDS
    // writes of the next slice.
    static __device__ void schedule_commit()
    {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            SCHED(SG_MFMA, 1);
            SCHED(SG_DS_READ, 1);
            SCHED(SG_DS_WRITE, 1);
            SCHED(SG_MFMA, 1);
            SCHED(SG_DS_WRITE, 1);
        }
    }

    // Sub-step 2: 16 matrix instructions, 8 fragment reads, the 16 global
    // reads of the slice after next.
    static __device__ void schedule_load()
    {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            SCHED(SG_MFMA, 1);
            SCHED(SG_DS_READ, 1);
            SCHED(SG_VMEM_READ, 2);
            SCHED(SG_MFMA, 1);
        }
    }
};

// ---- block-scaled FP4 operands ---------------------------------------------
//
// Thread t stages row t of the A tile and row t of the B tile: per K step of
// 64 elements that is 32 bytes of packed codes and 4 scale bytes per row.
// Decoding ("NVFP4 GEMM on Blackwell", section "NVFP4 Datatype"): each code
// pair converts to two FP16 E2M1 values (v_cvt_scalef32_pk_f16_fp4 with a unit
// scale), then one packed FP16 multiply applies the E4M3 scale of its 16-element
// block. Both steps are exact: an E4M3 value and every product e2m1 * e4m3
// lie in FP16's normal range with at most 6 significant bits. (gfx950's scaled
// FP4 conversion applies only the exponent of its scale operand, which is why
// the E4M3 mantissa goes through the multiply, and FP16 rather than BF16 is
// used because gfx950 has a packed FP16 multiply but no packed BF16 one; the
// FP16 and BF16 matrix instructions have the same rate.)
struct Fp4Staging {
    typedef f16x8 frag;
    __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
    int a_code_off, b_code_off, a_sf_off, b_sf_off;
    int lds_off;
    int K;
    u32x4 a_code[2], b_code[2];
    unsigned a_sf, b_sf;

    __device__ void init(const Problem &p, int tm, int tn, int tid)
    {
        const unsigned kc = (unsigned)p.K / 2, ks = (unsigned)p.K / 16;
        K = p.K;
        ra = make_rsrc(p.a, (unsigned)p.M * kc);
        rb = make_rsrc(p.b, (unsigned)p.N * kc);
        rsa = make_rsrc(p.sfa, (unsigned)p.M * ks);
        rsb = make_rsrc(p.sfb, (unsigned)p.N * ks);
        a_code_off = (tm * BM + tid) * (int)kc;
        b_code_off = (tn * BN + tid) * (int)kc;
        a_sf_off = (tm * BM + tid) * (int)ks;
        b_sf_off = (tn * BN + tid) * (int)ks;
        lds_off = tid * ROW_BYTES;
    }

    __device__ void load(int k0)
    {
        // K % 64 == 0: every step is whole; a step at or past K reads zeros
        const bool valid = k0 < K;
        const int oc = k0 / 2, os = k0 / 16;
        const int ac = valid ? a_code_off + oc : OOB, bc = valid ? b_code_off + oc : OOB;
        a_code[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, ac, 0, 0));
        a_code[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, ac + 16, 0, 0));
        b_code[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, bc, 0, 0));
        b_code[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, bc + 16, 0, 0));
        a_sf = __builtin_amdgcn_raw_buffer_load_b32(rsa, valid ? a_sf_off + os : OOB, 0, 0);
        b_sf = __builtin_amdgcn_raw_buffer_load_b32(rsb, valid ? b_sf_off + os : OOB, 0, 0);
    }

    // 8 codes (one dword) scaled by `s` -> 8 FP16 values.
    static __device__ f16x8 decode8(unsigned codes, f16x2 s)
    {
        f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s;
        f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s;
        f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s;
        f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s;
        f16x8 r = {v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
        return r;
    }

    // Scale block BLK (elements 16 BLK .. 16 BLK + 15 of the step) of one row.
    template <int BLK>
    static __device__ void decode_block(uint8_t *row_base, int row, const u32x4 *code, unsigned sf)
    {
        const _Float16 s = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)sf, BLK); // exact
        const f16x2 s2 = {s, s};
#pragma unroll
        for (int h = 0; h < 2; ++h) {                    // two dwords = 16 elements
            const int d = BLK * 2 + h;                   // 16-byte chunk d of the row
            const unsigned codes = code[d >> 2][d & 3];
            *reinterpret_cast<f16x8 *>(row_base + (swizzle(row, d) << 4)) = decode8(codes, s2);
        }
    }

    static __device__ void decode_row(uint8_t *row_base, int row, const u32x4 *code, unsigned sf)
    {
        decode_block<0>(row_base, row, code, sf);
        decode_block<1>(row_base, row, code, sf);
        decode_block<2>(row_base, row, code, sf);
        decode_block<3>(row_base, row, code, sf);
    }

    __device__ void commit(uint8_t *stage)
    {
        const int row = lds_off / ROW_BYTES;
        decode_row(stage + lds_off, row, a_code, a_sf);
        decode_row(stage + TILE_BYTES + lds_off, row, b_code, b_sf);
    }

    static __device__ f32x16 mma(frag s0, frag s1, f32x16 acc)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(s0, s1, acc, 0, 0, 0);
    }

    // Sub-step 1: 16 matrix instructions, 8 fragment reads, the decode
    // (vector ALU) and 16 LDS writes of the next slice.
    static __device__ void schedule_commit()
    {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            SCHED(SG_MFMA, 1);
            SCHED(SG_DS_READ, 1);
            SCHED(SG_VALU, 9);
            SCHED(SG_DS_WRITE, 1);
            SCHED(SG_MFMA, 1);
            SCHED(SG_VALU, 9);
            SCHED(SG_DS_WRITE, 1);
        }
    }

    // Sub-step 2: 16 matrix instructions, 8 fragment reads, the 6 global
    // reads of the slice after next.
    static __device__ void schedule_load()
    {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            SCHED(SG_MFMA, 1);
            SCHED(SG_DS_READ, 1);
            SCHED(SG_VMEM_READ, 1);
            SCHED(SG_MFMA, 1);
        }
    }
};

// ---- the persistent kernel --------------------------------------------------

// Make this wave's LDS writes visible to the workgroup and wait for all waves.
// Only LDS is fenced: global loads still in flight stay in flight.
__device__ inline void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <class Staging>
__global__ __attribute__((amdgpu_flat_work_group_size(THREADS, THREADS), amdgpu_waves_per_eu(1, 1)))
void gemm_nt_kernel(Problem p)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
    typedef typename Staging::frag frag;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;   // wave's 128-row half of the tile (A rows)
    const int wn = wave >> 1;  // wave's 128-column half (B rows)
    const int l32 = lane & 31;
    const int half = lane >> 5;

    // Per-lane LDS fragment addresses: row (l32 + 32 i) of the wave's block,
    // logical chunk (2 kk + half) for K sub-step kk of 16 elements.
    const int a_row = (wm * 128 + l32) * ROW_BYTES;
    const int b_row = TILE_BYTES + (wn * 128 + l32) * ROW_BYTES;
    int kofs[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        kofs[kk] = swizzle(l32, 2 * kk + half) << 4;   // rows differ from l32 by multiples of 32

    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.c, (unsigned)p.M * (unsigned)p.N * 2u);
    const int nk = (p.K + BK - 1) / BK;

    auto read_frags = [&](const uint8_t *stage, int kk, frag *fa, frag *fb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            fa[i] = *reinterpret_cast<const frag *>(stage + a_row + i * 32 * ROW_BYTES + kofs[kk]);
            fb[i] = *reinterpret_cast<const frag *>(stage + b_row + i * 32 * ROW_BYTES + kofs[kk]);
        }
    };

    for (int round = 0;; ++round) {
        const int pos = schedule_position(blockIdx.x, round, p.grid);
        if (pos >= p.tiles)
            break;
        int tm, tn;
        supergroup_tile(pos, p.tiles_m, p.tiles_n, p.supergroup, tm, tn);

        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = f32x16{};

        auto mma_all = [&](const frag *fa, const frag *fb) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = Staging::mma(fb[j], fa[i], acc[i][j]);
        };

        Staging st;
        st.init(p, tm, tn, tid);
        frag fa0[4], fb0[4], fa1[4], fb1[4];
        st.load(0);
        lds_barrier();            // every wave is done with the previous tile's stages
        st.commit(lds);
        st.load(BK);
        lds_barrier();
        read_frags(lds, 0, fa0, fb0);

        // Software pipeline over K steps. Step kt computes on LDS stage kt & 1
        // in four sub-steps of 16; each sub-step's fragments were read from LDS
        // during the previous sub-step's matrix instructions. Along the way the
        // step writes the registers holding slice kt + 1 into the other stage,
        // requests slice kt + 2 from memory, and -- after the step's single
        // barrier -- reads the first fragments of the other stage. The body has
        // no branches, so the compiler can interleave all of it with the matrix
        // instructions; slices at or past K load as zeros and are never used.
        for (int kt = 0; kt < nk; ++kt) {
            const uint8_t *cur = lds + (kt & 1) * STAGE_BYTES;
            uint8_t *nxt = lds + ((kt + 1) & 1) * STAGE_BYTES;

            read_frags(cur, 1, fa1, fb1);
            mma_all(fa0, fb0);
            schedule_reads_with_mma();
            SCHED_FENCE();

            read_frags(cur, 2, fa0, fb0);
            st.commit(nxt);
            mma_all(fa1, fb1);
            Staging::schedule_commit();
            SCHED_FENCE();

            read_frags(cur, 3, fa1, fb1);
            st.load((kt + 2) * BK);
            mma_all(fa0, fb0);
            Staging::schedule_load();
            SCHED_FENCE();

            // every wave is done reading stage `nxt` (last step) and writing it (this step)
            lds_barrier();
            SCHED_FENCE();
            read_frags(nxt, 0, fa0, fb0);
            mma_all(fa1, fb1);
            schedule_reads_with_mma();
            SCHED_FENCE();
        }

        // Epilogue: lane holds C[m][nb + 8 g + 4 half + e] in acc[i][j][4 g + e].
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = tm * BM + wm * 128 + i * 32 + l32;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int nb = tn * BN + wn * 128 + j * 32;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int g0 = 2 * q;
                    unsigned x0 = pack_bf16(acc[i][j][4 * g0 + 0], acc[i][j][4 * g0 + 1]);
                    unsigned x1 = pack_bf16(acc[i][j][4 * g0 + 2], acc[i][j][4 * g0 + 3]);
                    unsigned y0 = pack_bf16(acc[i][j][4 * g0 + 4], acc[i][j][4 * g0 + 5]);
                    unsigned y1 = pack_bf16(acc[i][j][4 * g0 + 6], acc[i][j][4 * g0 + 7]);
                    // lower half-wave keeps group g0 and receives the upper half's
                    // part of it; the upper half-wave ends up with group g0 + 1.
                    auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
                    auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
                    const u32x4 out = {s0[0], s1[0], s0[1], s1[1]};
                    const int n = nb + (g0 + half) * 8;
                    const int off = (m < p.M && n < p.N) ? (m * p.N + n) * 2 : OOB;
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, out), rc, off, 0, 0);
                }
            }
        }
    }
}

} // namespace gemm355
